"""Pins of the oracle against facts fixed by the pages and by mathematics (CPU only).

Each test checks a property that a plausible mistake in the oracle would break:
a dropped term, a wrong sign, index or axis, a transposed operand, a wrong
pairing of RoPE dimensions, a wrong GQA mapping, a wrong tie-break.  None of them
re-types the oracle's own formula.
"""
import math
import os

import numpy as np
import pytest

from oracle import backbone as O

RNG = np.random.default_rng(1234)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_dims(**kw):
    d = dict(hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, ffn=96, eps=1e-6, theta=1e6)
    d.update(kw)
    return O.Dims(**d)


def rand_layer(dims, rng, std=0.2, zero=()):
    hd, H, Hk = dims.head_dim, dims.n_heads, dims.n_kv_heads
    shapes = dict(attn_norm=(dims.hidden,), wq=(H * hd, dims.hidden), wk=(Hk * hd, dims.hidden),
                  wv=(Hk * hd, dims.hidden), q_norm=(hd,), k_norm=(hd,), wo=(dims.hidden, H * hd),
                  ffn_norm=(dims.hidden,), w_gate=(dims.ffn, dims.hidden),
                  w_up=(dims.ffn, dims.hidden), w_down=(dims.hidden, dims.ffn))
    a = {}
    for k, s in shapes.items():
        if len(s) == 1:
            a[k] = 1.0 + 0.1 * rng.standard_normal(s)
        else:
            a[k] = std * rng.standard_normal(s)
        if k in zero:
            a[k] = np.zeros(s)
    return O.Layer.from_arrays(a)


# ---------------------------------------------------------------------------
# Hyper-parameters: the pages' printed values
# ---------------------------------------------------------------------------

def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    return vals


def test_hparams_match_pages():
    from workload import configs as C
    g = read_golden("backbone_hparams.txt")
    s = C.Shape()
    assert s.n_layers == int(g["block_count"])
    assert s.hidden == int(g["embedding_length"])
    assert s.ffn == int(g["feed_forward_length"])
    assert s.n_heads == int(g["head_count"])
    assert s.n_kv_heads == int(g["head_count_kv"])
    assert s.head_dim == int(g["key_length"])
    assert s.eps == float(g["layer_norm_rms_eps"])
    assert s.theta == float(g["rope_freq_base"])
    w = C.c4().extra
    assert w["n_cb"] == int(g["num_audio_codebook"])
    assert w["cb_vocab"] == int(g["audio_vocab_size"])
    assert w["mask_id"] == int(g["audio_mask_id"])
    assert w["text_vocab"] == int(g["vocab_size"])
    assert w["layer_penalty"] == float(g["layer_penalty_factor"])
    assert w["n_steps"] == int(g["num_step"])
    assert C.c3().shape.n_layers == int(g["code_predictor_layers"])
    assert C.c3().extra["steps"] == int(g["code_predictor_steps"])
    assert C.c2().extra["n_cb"] == int(g["talker_codebooks"])
    assert C.c2().extra["head_vocab"] == int(g["talker_head_vocab"])


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------

def test_rmsnorm_unit_rms_before_gain():
    x = RNG.standard_normal((5, 1024)) * 3.0
    y = O.rms_norm(x, np.ones(1024), 1e-6)
    ms = np.mean(x * x, axis=-1)
    # exact: rms(y) = sqrt(ms / (ms + eps)); for ms ~ 9 this is 1 - 5.6e-8
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), np.sqrt(ms / (ms + 1e-6)),
                               rtol=1e-13)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=1e-7)


def test_rmsnorm_constant_vector_eps_inside_root():
    # c * 1 maps to c / sqrt(c^2 + eps); at c = 1e-3 and eps = 1e-6 that is 1/sqrt(2)
    for c in (1e-3, 0.5, -2.0):
        y = O.rms_norm(np.full(16, c), np.ones(16), 1e-6)
        np.testing.assert_allclose(y, c / math.sqrt(c * c + 1e-6), rtol=1e-14)
    y = O.rms_norm(np.full(16, 1e-3), np.ones(16), 1e-6)
    np.testing.assert_allclose(y, 1.0 / math.sqrt(2.0), rtol=1e-14)


def test_rmsnorm_scale_invariance_and_gain():
    x = RNG.standard_normal(128)
    g = 1.0 + 0.3 * RNG.standard_normal(128)
    y1 = O.rms_norm(x, g, 1e-6)
    y2 = O.rms_norm(37.0 * x, g, 1e-6)
    np.testing.assert_allclose(y1, y2, rtol=1e-6)
    np.testing.assert_allclose(O.rms_norm(x, g, 1e-6), O.rms_norm(x, np.ones(128), 1e-6) * g,
                               rtol=1e-15)
    # normalisation is per row (last axis), not over the whole array
    X = np.stack([x, 10 * x])
    Y = O.rms_norm(X, np.ones(128), 0.0)
    np.testing.assert_allclose(Y[0], Y[1], rtol=1e-13)


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def test_rope_position_zero_is_identity():
    u = RNG.standard_normal((3, 128))
    np.testing.assert_array_equal(O.rope(u, 0, 1e6), u)


def test_rope_preserves_pair_norms():
    u = RNG.standard_normal(128)
    r = O.rope(u, 4321, 1e6)
    np.testing.assert_allclose(u[:64] ** 2 + u[64:] ** 2, r[:64] ** 2 + r[64:] ** 2, rtol=1e-12)


def test_rope_pairs_dim_j_with_j_plus_half():
    # a unit vector on dimension 0 rotates into dimension 64 (rotate-half), never into 1
    e0 = np.zeros(128)
    e0[0] = 1.0
    r = O.rope(e0, 1.0, 1e6)
    np.testing.assert_allclose(r[0], math.cos(1.0), rtol=1e-15)
    np.testing.assert_allclose(r[64], math.sin(1.0), rtol=1e-15)
    assert np.count_nonzero(r) == 2
    e64 = np.zeros(128)
    e64[64] = 1.0
    r = O.rope(e64, 1.0, 1e6)
    np.testing.assert_allclose(r[0], -math.sin(1.0), rtol=1e-15)
    np.testing.assert_allclose(r[64], math.cos(1.0), rtol=1e-15)


def test_rope_frequencies_closed_form():
    # pair j rotates by p * theta^(-2j/128): j=0 -> p rad, j=32 -> p/1000 at theta=1e6,
    # j=16 -> p * 1e6^(-1/4) = p / 31.6227766...
    p = 777.0
    for j, w in ((0, 1.0), (32, 1e-3), (16, 1.0 / 31.622776601683793)):
        e = np.zeros(128)
        e[j] = 1.0
        r = O.rope(e, p, 1e6)
        np.testing.assert_allclose([r[j], r[j + 64]], [math.cos(p * w), math.sin(p * w)],
                                   rtol=1e-12, atol=1e-13)


def test_rope_relative_position_identity():
    q = RNG.standard_normal(128)
    k = RNG.standard_normal(128)
    for p, pp in ((10, 3), (4000, 3999), (57, 200)):
        lhs = O.rope(q, p, 1e6) @ O.rope(k, pp, 1e6)
        rhs = O.rope(q, p - pp, 1e6) @ k
        np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-10)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def test_attention_brute_force_tiny():
    # H=2 query heads sharing H_kv=1 head, d=4, L=3; softmax written out with loops
    q = RNG.standard_normal((2, 4))
    K = RNG.standard_normal((3, 1, 4))
    V = RNG.standard_normal((3, 1, 4))
    o = O.attend(q, K, V)
    for h in range(2):
        s = []
        for j in range(3):
            acc = 0.0
            for i in range(4):
                acc += q[h, i] * K[j, 0, i]
            s.append(acc / 2.0)
        w = [math.exp(v) for v in s]
        z = sum(w)
        for i in range(4):
            ref = sum(w[j] / z * V[j, 0, i] for j in range(3))
            assert abs(o[h, i] - ref) < 1e-14


def test_attention_two_keys_is_logistic():
    q = RNG.standard_normal((1, 8))
    K = RNG.standard_normal((2, 1, 8))
    V = RNG.standard_normal((2, 1, 8))
    s0 = q[0] @ K[0, 0] / math.sqrt(8)
    s1 = q[0] @ K[1, 0] / math.sqrt(8)
    a = 1.0 / (1.0 + math.exp(-(s0 - s1)))
    np.testing.assert_allclose(O.attend(q, K, V)[0], a * V[0, 0] + (1 - a) * V[1, 0], rtol=1e-13)


def test_attention_degenerate_cases():
    q = RNG.standard_normal((4, 16))
    V = RNG.standard_normal((5, 2, 16))
    # L = 1: output is v
    K1 = RNG.standard_normal((1, 2, 16))
    o = O.attend(q, K1, V[:1])
    np.testing.assert_allclose(o, V[0, [0, 0, 1, 1]], rtol=1e-15)
    # identical keys: mean of V
    Kid = np.repeat(RNG.standard_normal((1, 2, 16)), 5, axis=0)
    o = O.attend(q, Kid, V)
    np.testing.assert_allclose(o, V.mean(axis=0)[[0, 0, 1, 1]], rtol=1e-12)
    # q = 0: mean of V
    o = O.attend(np.zeros((4, 16)), RNG.standard_normal((5, 2, 16)), V)
    np.testing.assert_allclose(o, V.mean(axis=0)[[0, 0, 1, 1]], rtol=1e-12)


def test_gqa_equals_mha_with_duplicated_kv():
    q = RNG.standard_normal((16, 128))
    K = RNG.standard_normal((9, 8, 128))
    V = RNG.standard_normal((9, 8, 128))
    gqa = O.attend(q, K, V)
    idx = np.arange(16) // 2  # consecutive grouping: heads 2i, 2i+1 read KV head i
    mha = O.attend(q, K[:, idx, :], V[:, idx, :])
    np.testing.assert_allclose(gqa, mha, rtol=1e-14)
    # and per head it is single-head attention on the right KV head
    for h in (0, 1, 7, 15):
        one = O.attend(q[h:h + 1], K[:, h // 2:h // 2 + 1], V[:, h // 2:h // 2 + 1])
        np.testing.assert_allclose(gqa[h], one[0], rtol=1e-14)


def test_causal_prefix_unchanged_by_appended_tokens():
    S, H, Hk, d = 7, 4, 2, 16
    Q = RNG.standard_normal((S + 3, H, d))
    K = RNG.standard_normal((S + 3, Hk, d))
    V = RNG.standard_normal((S + 3, Hk, d))
    a = O.attention_full(Q[:S], K[:S], V[:S], causal=True)
    b = O.attention_full(Q, K, V, causal=True)
    np.testing.assert_allclose(a, b[:S], rtol=1e-14)
    # while bidirectional attention of the prefix does change
    c = O.attention_full(Q, K, V, causal=False)
    assert np.max(np.abs(c[:S] - a)) > 1e-3


# ---------------------------------------------------------------------------
# Whole layer: decode = recompute, bidirectional dependence, special cases
# ---------------------------------------------------------------------------

def test_decode_steps_equal_causal_recompute():
    dims = small_dims()
    rng = np.random.default_rng(5)
    layers = [rand_layer(dims, rng) for _ in range(2)]
    S = 6
    X = rng.standard_normal((S, dims.hidden))
    full = O.backbone_full(X, layers, dims, causal=True)
    cache = O.KVCache(2, 1)
    for p in range(S):
        out = O.decode_step(X[p:p + 1], [p], cache, layers, dims)
        np.testing.assert_allclose(out[0], full[p], rtol=1e-11, atol=1e-12)


def test_decode_batch_streams_are_independent():
    dims = small_dims()
    rng = np.random.default_rng(6)
    layers = [rand_layer(dims, rng)]
    X = rng.standard_normal((3, dims.hidden))
    cache = O.KVCache(1, 3)
    pre = [rng.standard_normal((n, 2, dims.n_kv_heads, dims.head_dim)) for n in (2, 5, 0)]
    for b, p in enumerate(pre):
        if p.shape[0]:
            cache.set(0, b, p[:, 0], p[:, 1])
    out = O.decode_step(X, [2, 5, 0], cache, layers, dims)
    for b, p in enumerate(pre):
        c1 = O.KVCache(1, 1)
        if p.shape[0]:
            c1.set(0, 0, p[:, 0], p[:, 1])
        one = O.decode_step(X[b:b + 1], [p.shape[0]], c1, layers, dims)
        np.testing.assert_allclose(out[b], one[0], rtol=1e-12, atol=1e-13)


def test_maskgit_attention_is_bidirectional():
    dims = small_dims()
    rng = np.random.default_rng(7)
    layers = [rand_layer(dims, rng)]
    X = rng.standard_normal((5, dims.hidden))
    Y = X.copy()
    Y[-1] += 1.0
    a = O.backbone_full(X, layers, dims, causal=False)
    b = O.backbone_full(Y, layers, dims, causal=False)
    assert np.max(np.abs(a[0] - b[0])) > 1e-4  # the last token reaches position 0
    a = O.backbone_full(X, layers, dims, causal=True)
    b = O.backbone_full(Y, layers, dims, causal=True)
    np.testing.assert_array_equal(a[0], b[0])


def test_first_token_layer_closed_form():
    # At position 0 with an empty cache: RoPE is the identity and softmax over one key
    # is 1, so o_h = v_{h//2}; with W_down = 0 the layer is x + W_o [v_0, v_0, v_1, ...].
    dims = small_dims()
    rng = np.random.default_rng(8)
    L = rand_layer(dims, rng, zero=("w_down",))
    x = rng.standard_normal((1, dims.hidden))
    out = O.decode_step(x, [0], O.KVCache(1, 1), [L], dims)
    h = x[0] / math.sqrt(np.mean(x[0] ** 2) + dims.eps) * L.attn_norm
    v = (L.wv @ h).reshape(dims.n_kv_heads, dims.head_dim)
    o = np.concatenate([v[hq // 2] for hq in range(dims.n_heads)])
    np.testing.assert_allclose(out[0], x[0] + L.wo @ o, rtol=1e-12, atol=1e-13)


def test_swiglu_special_cases():
    assert O.silu(0.0) == 0.0
    np.testing.assert_allclose(O.silu(1.0), 0.7310585786300049, rtol=1e-15)  # 1/(1+e^-1)
    np.testing.assert_allclose(O.silu(-1.0), -0.2689414213699951, rtol=1e-15)
    np.testing.assert_allclose(O.silu(40.0), 40.0, rtol=1e-15)
    dims = small_dims()
    rng = np.random.default_rng(9)
    # W_gate = 0 -> silu(0) = 0 -> MLP contributes nothing: x2 = x1
    L = rand_layer(dims, rng, zero=("w_gate",))
    x = rng.standard_normal((2, dims.hidden))
    o = rng.standard_normal((2, dims.n_heads, dims.head_dim))
    post = O.post_attention(x, o, L, dims)
    np.testing.assert_array_equal(post["x2"], post["x1"])
    # W_o = 0 -> x1 = x
    L = rand_layer(dims, rng, zero=("wo",))
    post = O.post_attention(x, o, L, dims)
    np.testing.assert_array_equal(post["x1"], x)
    # gate and up are not swapped: with W_up = 0 the MLP is zero, with a one-hot gate
    # and up the MLP output is silu(g) * u through W_down
    L = rand_layer(dims, rng)
    L.w_gate[:] = 0.0
    L.w_up[:] = 0.0
    L.w_gate[0, 0] = 1.0
    L.w_up[0, 1] = 1.0
    L.w_down[:] = 0.0
    L.w_down[3, 0] = 1.0
    post = O.post_attention(x, o, L, dims)
    h2 = post["h2"]
    np.testing.assert_allclose(post["x2"][:, 3] - post["x1"][:, 3],
                               h2[:, 0] / (1 + np.exp(-h2[:, 0])) * h2[:, 1], rtol=1e-14)


# ---------------------------------------------------------------------------
# Embedding
# ---------------------------------------------------------------------------

def test_codebook_embed_sums_offset_rows():
    V, K, D = 5, 3, 4
    table = RNG.standard_normal((K * V, D))
    codes = np.array([[0, 4, 2], [3, 3, 3]])
    e = O.codebook_embed(codes, table, V)
    np.testing.assert_array_equal(e[0], table[0] + table[1 * 5 + 4] + table[2 * 5 + 2])
    np.testing.assert_array_equal(e[1], table[3] + table[8] + table[13])
    # K = 1 is a plain lookup
    np.testing.assert_array_equal(O.codebook_embed(codes[:, :1], table, V), table[[0, 3]])


def test_codebook_embed_bf16_sum_is_exact_in_fp64():
    from workload import gen
    vals = gen.round_bf16(RNG.standard_normal((16, 64)).astype(np.float32) * 0.02)
    codes = np.arange(16)[None, :] * 0  # code 0 of each of 16 codebooks
    table = np.zeros((16 * 2, 64), np.float32)
    table[np.arange(16) * 2] = vals
    e = O.codebook_embed(codes, table, 2)
    # Python's math.fsum is the correctly rounded sum
    for j in range(64):
        assert e[0, j] == math.fsum(float(v) for v in vals[:, j])


def test_hybrid_embed_text_then_audio_with_mask_row():
    V, K, D = 4, 2, 3
    audio = RNG.standard_normal((K * V, D))
    text = RNG.standard_normal((10, D))
    codes_kt = np.array([[1, 3], [3, 0]])  # [K][T]; id 3 plays the mask id
    e = O.hybrid_embed(np.array([7, 2]), text, codes_kt, audio, V)
    np.testing.assert_array_equal(e[0], text[7])
    np.testing.assert_array_equal(e[1], text[2])
    np.testing.assert_array_equal(e[2], audio[1] + audio[4 + 3])
    np.testing.assert_array_equal(e[3], audio[3] + audio[4 + 0])


# ---------------------------------------------------------------------------
# Heads, scoring, selection, schedule
# ---------------------------------------------------------------------------

def test_head_one_hot_selects_column_and_argmax_groups():
    H = RNG.standard_normal((12, 8))
    x = np.zeros((1, 8))
    x[0, 3] = 2.0
    y, lg = O.head_logits(x, np.ones(8), H, 0.0)
    # rms of x is 2/sqrt(8); y = x / rms = sqrt(8) e_3
    np.testing.assert_allclose(lg[0], math.sqrt(8) * H[:, 3], rtol=1e-14)
    am = O.argmax_groups(np.array([[1.0, 5.0, 5.0, 0.0, 2.0, 2.0]]), 2, 3)
    np.testing.assert_array_equal(am, [[1, 1]])  # ties go to the lower class id


def test_maskgit_scores_properties():
    K, T, V, mask = 3, 5, 7, 6
    lg = RNG.standard_normal((T, K * V)) * 3
    codes = np.array([[6, 1, 6, 6, 2], [6, 6, 6, 0, 6], [3, 6, 6, 6, 6]])
    pred, conf, lp = O.maskgit_scores(lg, codes, K, V, mask, 5.0)
    view = lg.reshape(T, K, V)
    for k in range(K):
        for t in range(T):
            row = view[t, k]
            # softmax probabilities over all V classes sum to one
            z = sum(math.exp(v) for v in row)
            assert abs(sum(math.exp(v) / z for v in row) - 1.0) < 1e-12
            # pred is the best non-mask class of the raw logits
            assert pred[k, t] == int(np.argmax(row[:mask]))
            if codes[k, t] == mask:
                ref = math.log(math.exp(row[pred[k, t]]) / z) - 5.0 * k
                assert abs(conf[k, t] - ref) < 1e-12
            else:
                assert conf[k, t] == -np.inf
    # shifting all logits of a group by a constant changes nothing
    lg2 = lg.copy()
    lg2[:, V:2 * V] += 11.0
    p2, c2, _ = O.maskgit_scores(lg2, codes, K, V, mask, 5.0)
    np.testing.assert_array_equal(p2, pred)
    np.testing.assert_allclose(c2, conf, rtol=1e-12)


def test_select_top_matches_brute_force_with_ties():
    rng = np.random.default_rng(11)
    for trial in range(20):
        n_el = int(rng.integers(1, 60))
        conf = rng.integers(-3, 4, n_el).astype(float)  # many ties
        conf[rng.random(n_el) < 0.3] = -np.inf
        n = int(rng.integers(0, n_el + 3))
        picked = O.select_top(conf, n)
        finite = [(-conf[i], i) for i in range(n_el) if conf[i] > -np.inf]
        finite.sort()
        ref = [i for _, i in finite[:n]] + [-1] * max(0, n - len(finite))
        np.testing.assert_array_equal(picked, np.array(ref[:n], np.int32))


def test_apply_picks_updates_only_picked():
    codes = np.array([[9, 9, 1], [9, 2, 9]])
    pred = np.array([[4, 5, 6], [7, 8, 0]])
    out = O.apply_picks(codes, pred, np.array([3, 0, -1]))
    np.testing.assert_array_equal(out, [[4, 9, 1], [7, 2, 9]])


def test_unmask_schedule():
    for N, steps in ((3000, 32), (7, 3), (100, 1), (0, 4), (5, 10)):
        s = O.unmask_schedule(N, steps)
        assert len(s) == steps and sum(s) == N and min(s) >= 0
        cum = np.cumsum(s)
        for i in range(steps - 1):
            # every step unmasks at least the cosine fraction of the total
            frac = 1.0 - math.cos(math.pi / 2 * (i + 1) / steps)
            assert cum[i] >= min(N, math.floor(N * frac - 1e-9))
    # two steps of 10: t1 = 1 - cos(pi/4) = 0.29289..., ceil(2.93) = 3 then the rest
    assert O.unmask_schedule(10, 2) == [3, 7]


# ---------------------------------------------------------------------------
# Classifier-free guidance (the first NEXT row)
# ---------------------------------------------------------------------------

def _cfg_setup(rng, n_text=3, n_frames=6, n_cb=2, V=9, mask=8):
    dims = small_dims()
    layers = [rand_layer(dims, rng) for _ in range(2)]
    text_tab = rng.standard_normal((11, dims.hidden))
    tab = rng.standard_normal((n_cb * V, dims.hidden))
    heads = 0.3 * rng.standard_normal((n_cb * V, dims.hidden))
    fnorm = 1.0 + 0.1 * rng.standard_normal(dims.hidden)
    text = rng.integers(0, 11, n_text)
    codes = rng.integers(0, V - 1, (n_cb, n_frames))
    codes[rng.random((n_cb, n_frames)) < 0.5] = mask
    return dims, layers, text_tab, tab, heads, fnorm, text, codes, V, mask


def test_cfg_logits_is_affine_in_the_scale():
    rng = np.random.default_rng(21)
    c, u = rng.standard_normal((4, 9)), rng.standard_normal((4, 9))
    np.testing.assert_array_equal(O.cfg_logits(c, u, 0.0), c)           # no guidance
    np.testing.assert_array_equal(O.cfg_logits(c, c, 3.7), c)           # nothing to contrast
    f0, f1, f3 = (O.cfg_logits(c, u, s) for s in (0.0, 1.0, 3.0))
    np.testing.assert_allclose(f3 - f1, 2.0 * (f1 - f0), rtol=1e-12, atol=1e-12)  # linear in s
    # a large scale follows the contrast c - u: its argmax wins
    big = O.cfg_logits(c, u, 1e6)
    np.testing.assert_array_equal(np.argmax(big, -1), np.argmax(c - u, -1))


def test_cfg_without_context_equals_the_plain_step():
    """No text and a window that covers every frame: the unconditional prompt is the
    conditional one, so guidance cancels for any scale."""
    rng = np.random.default_rng(22)
    dims, layers, text_tab, tab, heads, fnorm, _, codes, V, mask = _cfg_setup(rng)
    plain = O.maskgit_pass([], text_tab, codes, tab, heads, layers, fnorm, dims, V, mask, 5.0, 4)
    for s in (0.0, 2.5):
        guided = O.maskgit_pass_cfg([], text_tab, codes, codes.shape[1], tab, heads, layers, fnorm, dims, V,
                                    mask, 5.0, 4, s)
        for a, b in zip(plain, guided):
            np.testing.assert_array_equal(a, b)


def test_cfg_unconditional_prompt_is_the_window_alone():
    """The unconditional logits depend on the window's tokens only: changing the text or
    the reference frames moves the conditional logits and leaves them alone; they equal
    the logits of a plain step run on the window by itself."""
    rng = np.random.default_rng(23)
    dims, layers, text_tab, tab, heads, fnorm, text, codes, V, mask = _cfg_setup(rng)
    nt = 4
    rec = {}
    out = O.maskgit_pass_cfg(text, text_tab, codes, nt, tab, heads, layers, fnorm, dims, V, mask, 5.0, 3, 2.0, rec)
    text2 = (text + 1) % 11
    codes2 = codes.copy()
    codes2[:, 0] = (codes2[:, 0] + 1) % (V - 1)  # a reference frame, outside the window
    rec2 = {}
    O.maskgit_pass_cfg(text2, text_tab, codes2, nt, tab, heads, layers, fnorm, dims, V, mask, 5.0, 3, 2.0, rec2)
    np.testing.assert_array_equal(rec["logits_u"], rec2["logits_u"])
    assert np.max(np.abs(rec["logits_c"] - rec2["logits_c"])) > 1e-6
    rec3 = {}
    window = codes[:, -nt:]
    O.maskgit_pass([], text_tab, window, tab, heads, layers, fnorm, dims, V, mask, 5.0, 0, rec3)
    np.testing.assert_allclose(rec["logits_u"], rec3["logits"], rtol=1e-12, atol=1e-12)
    # only the window is updated, and only where the guided scores pick
    new_codes, pred, conf, picked = out
    np.testing.assert_array_equal(new_codes[:, :-nt], codes[:, :-nt])
    assert pred.shape == (codes.shape[0], nt) and conf.shape == pred.shape
    np.testing.assert_array_equal(new_codes[:, -nt:], O.apply_picks(window, pred, picked))
    # the scores are those of the guided logits
    p_ref, c_ref, _ = O.maskgit_scores(rec["guided"], window, codes.shape[0], V, mask, 5.0)
    np.testing.assert_array_equal(p_ref, pred)
    np.testing.assert_array_equal(c_ref, conf)


# ---------------------------------------------------------------------------
# Sampler: temperatures, top-k ratio, Gumbel noise (the third NEXT row)
# ---------------------------------------------------------------------------

def test_gumbel_closed_form():
    c = np.array([-3.0, -0.5, 0.0, 0.7, 4.0])
    u = np.exp(-np.exp(-c))  # the Gumbel CDF: G(F(c)) = c
    np.testing.assert_allclose(O.gumbel(u), c, rtol=1e-12, atol=1e-12)
    assert O.gumbel(np.array([math.exp(-1.0)]))[0] == pytest.approx(0.0, abs=1e-15)
    g = O.gumbel(np.linspace(0.01, 0.99, 50))
    assert np.all(np.diff(g) > 0)


def test_gumbel_max_draws_follow_the_tempered_softmax():
    """Gumbel-max: argmax(lp / temp + G(u)) is distributed as softmax(lp / temp).  A wrong
    sign, a multiplied temperature or log(u) in place of -log(-log u) fails this."""
    rng = np.random.default_rng(31)
    lp = np.log(np.array([0.5, 0.2, 0.15, 0.1, 0.05]))
    temp, n = 0.7, 40000
    u = rng.random((n, 5))
    u = np.clip(u, 1e-12, 1 - 1e-12)
    draws = np.argmax(lp / temp + O.gumbel(u), axis=1)
    freq = np.bincount(draws, minlength=5) / n
    p = np.exp(lp / temp)
    p /= p.sum()
    sigma = np.sqrt(p * (1 - p) / n)
    assert np.all(np.abs(freq - p) < 5 * sigma + 1e-9)


def test_keep_top_k_ratio_counts_and_ties():
    rng = np.random.default_rng(32)
    for _ in range(20):
        V = int(rng.integers(1, 40))
        ratio = float(rng.choice([0.1, 0.25, 0.5, 1.0, 0.01]))
        row = rng.integers(-3, 3, V).astype(float)  # many ties
        out = O.keep_top_k_ratio(row[None], ratio)[0]
        k = max(1, math.floor(ratio * V))
        kept = [v for v in range(V) if out[v] > -np.inf]
        assert len(kept) == k
        for v in range(V):  # rank by (value desc, id asc), counted directly
            rank = sum(1 for w in range(V) if row[w] > row[v] or (row[w] == row[v] and w < v))
            assert (v in kept) == (rank < k)
            if v in kept:
                assert out[v] == row[v]


def test_sampler_reduces_to_greedy_scoring():
    rng = np.random.default_rng(33)
    K, T, V, mask = 2, 6, 9, 8
    lg = rng.standard_normal((T, K * V)) * 2
    codes = np.full((K, T), mask)
    codes[0, 1] = 3
    p0, c0, _ = O.maskgit_scores(lg, codes, K, V, mask, 5.0)
    p1, c1, _ = O.sample_scores(lg, codes, K, V, mask, 5.0, 0.0, 0.0, 0.1, None, None)
    np.testing.assert_array_equal(p0, p1)
    np.testing.assert_array_equal(c0, c1)
    # zero noise (u = 1/e) and ratio 1: temperature 1 changes nothing either
    u_c = np.full((K, T, V), math.exp(-1.0))
    p2, c2, _ = O.sample_scores(lg, codes, K, V, mask, 5.0, 1.0, 0.0, 1.0, u_c, None)
    np.testing.assert_array_equal(p0, p2)
    np.testing.assert_allclose(c0, c2, rtol=1e-12, atol=1e-12)
    # position noise shifts every masked score by pos_temp * G(u_pos), nothing else
    u_p = rng.random((K, T)) * 0.98 + 0.01
    p3, c3, _ = O.sample_scores(lg, codes, K, V, mask, 5.0, 0.0, 0.3, 0.1, None, u_p)
    np.testing.assert_array_equal(p0, p3)
    fin = np.isfinite(c0)
    np.testing.assert_allclose(c3[fin] - c0[fin], 0.3 * O.gumbel(u_p)[fin], rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isfinite(c3), fin)


def test_sampler_tempered_score_hand_example():
    """A worked case of the sampler's order of operations (OmniVoice ARCHITECTURE, "MaskGIT
    decoder": log-softmax over all classes, mask class to -inf, keep the top-k ratio,
    divide by the class temperature, add Gumbel noise, score = max - layer index *
    penalty, plus position noise), with values chosen so that each plausible mistake
    changes the answer.  Logits ln[4, 2, 1, 1, 8] (class 4 = mask): the normaliser is 16
    (mask included), so lp = ln[1/4, 1/8, 1/16, 1/16] on the non-mask classes.
    Uniforms are u = exp(-exp(-G)), i.e. Gumbel values G chosen by hand."""
    V, mask = 5, 4
    ln2 = math.log(2.0)
    row = np.log(np.array([4.0, 2.0, 1.0, 1.0, 8.0]))
    lg = np.concatenate([row, row])[None, :]          # T = 1 frame, K = 2 codebooks
    codes = np.full((2, 1), mask)

    def u_of(G):
        return np.exp(-np.exp(-np.asarray(G, np.float64)))

    # codebook 0: G = [0, 0.5, 10, 0, 0]; codebook 1: no noise (G = 0)
    u_c = np.stack([u_of([0.0, 0.5, 10.0, 0.0, 0.0]), u_of([0.0] * 5)])[:, None, :]
    u_p = u_of([[1.0], [0.0]])
    # ratio 0.4 keeps floor(2.0) = 2 classes {0, 1}: class 2 (G = 10) is filtered out.
    # Tempered values (temperature 2): class 0: -ln2 + 0; class 1: -1.5 ln2 + 0.5 = -0.540
    # -> class 1 wins (with unscaled log-probs class 0 would: -2 ln2 > -3 ln2 + 0.5).
    pred, score, _ = O.sample_scores(lg, codes, 2, V, mask, 5.0, 2.0, 0.3, 0.4, u_c, u_p)
    assert pred.tolist() == [[1], [0]]
    assert abs(score[0, 0] - (-1.5 * ln2 + 0.5 + 0.3 * 1.0)) <= 1e-12       # k = 0, position G = 1
    assert abs(score[1, 0] - (-1.0 * ln2 - 5.0)) <= 1e-12                   # k = 1: lp0 / 2 - 5
    # no noise and ratio 1: the greedy choice, score = max lp / temperature - k * penalty
    u0 = np.full((2, 1, V), math.exp(-1.0))
    pred, score, _ = O.sample_scores(lg, codes, 2, V, mask, 5.0, 2.0, 0.0, 1.0, u0, None)
    assert pred.tolist() == [[0], [0]]
    np.testing.assert_allclose(score[:, 0], [-ln2, -ln2 - 5.0], rtol=0, atol=1e-12)
    # ties at the threshold keep the lower class id: ratio 0.6 keeps {0, 1, 2} (classes 2
    # and 3 tie at ln 1/16); class 3 carries G = 10 but is dropped, class 2 (G = 2) wins
    u_t = np.stack([u_of([0.0, 0.0, 2.0, 10.0, 0.0]), u_of([0.0] * 5)])[:, None, :]
    pred, score, _ = O.sample_scores(lg, codes, 2, V, mask, 5.0, 2.0, 0.0, 0.6, u_t, None)
    assert pred[0, 0] == 2
    assert abs(score[0, 0] - (-2.0 * ln2 + 2.0)) <= 1e-12


def test_sampler_picks_inside_the_kept_classes():
    """With class noise the choice is always one of the top floor(ratio * V) non-mask
    classes, never the mask class."""
    rng = np.random.default_rng(34)
    K, T, V, mask = 2, 40, 50, 49
    lg = rng.standard_normal((T, K * V)) * 2
    codes = np.full((K, T), mask)
    u_c = rng.random((K, T, V)) * 0.999 + 0.0005
    pred, conf, lp = O.sample_scores(lg, codes, K, V, mask, 5.0, 1.3, 0.0, 0.1, u_c, None)
    base, _, lp0 = O.maskgit_scores(lg, codes, K, V, mask, 5.0)
    for k in range(K):
        for t in range(T):
            order = sorted(range(V), key=lambda v: (-lp0[k, t, v], v))[:5]  # floor(0.1 * 50)
            assert pred[k, t] in order and pred[k, t] != mask


def test_general_step_reduces_to_the_plain_and_guided_steps():
    rng = np.random.default_rng(35)
    dims, layers, text_tab, tab, heads, fnorm, text, codes, V, mask = _cfg_setup(rng)
    nf = codes.shape[1]
    a = O.maskgit_pass(text, text_tab, codes, tab, heads, layers, fnorm, dims, V, mask, 5.0, 3)
    b = O.maskgit_step(text, text_tab, codes, nf, tab, heads, layers, fnorm, dims, V, mask, 5.0, 3)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    c = O.maskgit_pass_cfg(text, text_tab, codes, 4, tab, heads, layers, fnorm, dims, V, mask, 5.0, 3, 1.5)
    d = O.maskgit_step(text, text_tab, codes, 4, tab, heads, layers, fnorm, dims, V, mask, 5.0, 3, cfg_scale=1.5)
    for x, y in zip(c, d):
        np.testing.assert_array_equal(x, y)


# ---------------------------------------------------------------------------
# Codec RVQ decode (the fourth NEXT row)
# ---------------------------------------------------------------------------

def test_rvq_decode_identity_projection_sums_embeddings():
    """With project_out = [I; 0] and zero bias the decode is the sum of the gathered
    embeddings in the first dim outputs; a bias alone shifts every frame by sum_k b_k."""
    rng = np.random.default_rng(41)
    Q, CB, D, OUT, T = 3, 10, 4, 6, 7
    emb = rng.standard_normal((Q, CB, D))
    w = np.zeros((Q, OUT, D))
    w[:, :D, :] = np.eye(D)
    codes = rng.integers(0, CB, (Q, T))
    out = O.rvq_decode(codes, emb, w, np.zeros((Q, OUT)))
    ref = sum(emb[k][codes[k]] for k in range(Q))
    np.testing.assert_allclose(out[:, :D], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(out[:, D:], 0.0)
    b = rng.standard_normal((Q, OUT))
    out_b = O.rvq_decode(codes, np.zeros_like(emb), w, b)
    np.testing.assert_allclose(out_b, np.tile(b.sum(0), (T, 1)), rtol=1e-12, atol=1e-12)


def test_rvq_decode_frame_by_loops_and_codebook_additivity():
    rng = np.random.default_rng(42)
    Q, CB, D, OUT, T = 4, 12, 5, 9, 6
    emb, w, b = rng.standard_normal((Q, CB, D)), rng.standard_normal((Q, OUT, D)), rng.standard_normal((Q, OUT))
    codes = rng.integers(0, CB, (Q, T))
    out = O.rvq_decode(codes, emb, w, b)
    for t in range(T):  # one frame, plain loops
        for n in range(OUT):
            v = 0.0
            for k in range(Q):
                v += b[k, n] + sum(emb[k, codes[k, t], d] * w[k, n, d] for d in range(D))
            assert abs(out[t, n] - v) < 1e-10
    # decoding codebooks 0..1 and 2..3 separately and adding gives the whole
    a = O.rvq_decode(codes[:2], emb[:2], w[:2], b[:2])
    c = O.rvq_decode(codes[2:], emb[2:], w[2:], b[2:])
    np.testing.assert_allclose(a + c, out, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Causal multi-token prefill (the second NEXT row)
# ---------------------------------------------------------------------------

def test_prefill_equals_token_by_token_decode():
    """A prefill of S tokens after p0 cached ones equals S decode steps of one token each
    (the cached/recompute equivalence of the rightkit-qts synthetic tests), outputs and
    cache contents."""
    rng = np.random.default_rng(51)
    dims = small_dims()
    layers = [rand_layer(dims, rng) for _ in range(2)]
    p0, S = 3, 5
    pre = rng.standard_normal((p0, dims.hidden))
    x = rng.standard_normal((S, dims.hidden))
    c1, c2 = O.KVCache(2, 1), O.KVCache(2, 1)
    for c in (c1, c2):
        O.prefill(pre, 0, c, 0, layers, dims)
    out = O.prefill(x, p0, c1, 0, layers, dims)
    for i in range(S):
        step = O.decode_step(x[i:i + 1], [p0 + i], c2, layers, dims)
        np.testing.assert_allclose(out[i], step[0], rtol=1e-10, atol=1e-12)
    for li in range(2):
        np.testing.assert_allclose(c1.k[li][0], c2.k[li][0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(c1.v[li][0], c2.v[li][0], rtol=1e-12, atol=1e-14)


def test_prefill_from_empty_is_the_causal_full_pass():
    rng = np.random.default_rng(52)
    dims = small_dims()
    layers = [rand_layer(dims, rng) for _ in range(2)]
    x = rng.standard_normal((7, dims.hidden))
    out = O.prefill(x, 0, O.KVCache(2, 1), 0, layers, dims)
    ref = O.backbone_full(x, layers, dims, causal=True)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    # a later token never changes an earlier one
    out2 = O.prefill(np.vstack([x[:4], rng.standard_normal((3, dims.hidden))]), 0, O.KVCache(2, 1), 0, layers,
                     dims)
    np.testing.assert_allclose(out2[:4], out[:4], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# The whole layer stack against an independent implementation of the same
# architecture: the Qwen3 decoder of the `transformers` library (the pages name the
# backbone Qwen3-0.6B), built at small sizes in float64 with the oracle's weights.
# ---------------------------------------------------------------------------

def _library_qwen3(dims, layers, final_gain):
    torch = pytest.importorskip("torch")
    tf = pytest.importorskip("transformers")
    cfg = tf.Qwen3Config(vocab_size=8, hidden_size=dims.hidden, intermediate_size=dims.ffn,
                         num_hidden_layers=len(layers), num_attention_heads=dims.n_heads,
                         num_key_value_heads=dims.n_kv_heads, head_dim=dims.head_dim,
                         rms_norm_eps=dims.eps, rope_theta=dims.theta, max_position_embeddings=64,
                         attention_bias=False, attn_implementation="eager")
    m = tf.Qwen3Model(cfg).double().eval()

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a))

    with torch.no_grad():
        for L, hl in zip(layers, m.layers):
            at = hl.self_attn
            for mod, w in ((at.q_proj, L.wq), (at.k_proj, L.wk), (at.v_proj, L.wv), (at.o_proj, L.wo),
                           (at.q_norm, L.q_norm), (at.k_norm, L.k_norm), (hl.input_layernorm, L.attn_norm),
                           (hl.post_attention_layernorm, L.ffn_norm), (hl.mlp.gate_proj, L.w_gate),
                           (hl.mlp.up_proj, L.w_up), (hl.mlp.down_proj, L.w_down)):
                mod.weight.copy_(t(w))
        m.norm.weight.copy_(t(final_gain))

    def run(x, causal):
        kw = {} if causal else {"attention_mask": torch.zeros(1, 1, x.shape[0], x.shape[0], dtype=torch.float64)}
        with torch.no_grad():
            return m(inputs_embeds=t(x)[None], **kw).last_hidden_state[0].numpy()
    return run


@pytest.mark.parametrize("causal", [True, False])
def test_layer_stack_matches_library_qwen3(causal):
    rng = np.random.default_rng(77)
    dims = small_dims()
    layers = [rand_layer(dims, rng) for _ in range(3)]
    g = 1.0 + 0.1 * rng.standard_normal(dims.hidden)
    run = _library_qwen3(dims, layers, g)
    x = rng.standard_normal((11, dims.hidden))
    ref = O.rms_norm(O.backbone_full(x, layers, dims, causal=causal), g, dims.eps)
    # the library rounds to float32 inside every RMSNorm (it upcasts its input to float32
    # whatever the dtype) and takes the RoPE angles in float32; everything else runs in
    # float64.  Observed ~3e-7 of max |y|; a structural mistake (a dropped term, a wrong
    # sign, index or operand order) gives errors of order one.
    err = np.abs(run(x, causal) - ref).max() / np.abs(ref).max()
    assert err < 3e-6, err
    # position 0 alone (RoPE is the identity there) and two positions
    for n in (1, 2):
        ref_n = O.rms_norm(O.backbone_full(x[:n], layers, dims, causal=causal), g, dims.eps)
        err = np.abs(run(x[:n], causal) - ref_n).max() / np.abs(ref_n).max()
        assert err < 3e-6, (n, err)
