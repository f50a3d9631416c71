"""GPU parity of the HIP path against the oracle at small sizes (several tiles, ragged
tails, degenerate cases).  Every call goes through the C ABI (codec_token_tts_amd.ttsbb).

Tolerances (derived in the design notes):
* fp32 mode: 1e-4 max-abs on every intermediate and the layer output.
* bf16 mode: normwise max-relative max|gpu-ref|/max|ref| <= TOL_LAYER_BF16 on continuous outputs.
* discrete outputs: exact argmax / top-n of the GPU's own scores, and agreement with the
  oracle wherever the oracle's margin exceeds twice the measured score error.
* the codebook embedding: bit-exact (fp64 sum in codebook order, one rounding).
"""
import numpy as np
import pytest

from oracle import backbone as O
from workload import configs as CFG
from workload import device as DEV
from workload import gen
from workload.gen import stream_id

from gpu_setup import (TOL_LAYER_BF16, Model, check_argmax_groups, check_sampler, check_topn, dims_of, normwise, read_tap,
                       torch, widen)

pytestmark = pytest.mark.gpu


def t_i32(a):
    return torch().from_numpy(np.ascontiguousarray(a, np.int32)).to("cuda")


def t_f32(a):
    return torch().from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")


# ---------------------------------------------------------------------------------------
def test_device_inputs_match_host_generator():
    for bf16 in (True, False):
        t = DEV.normal((3, 1001), 5, 77, 0.02, bf16, start=9)
        h = gen.fast_normal(5, 77, (3, 1001), 0.02, start=9, bf16=bf16)
        a = t.cpu().numpy()
        assert np.array_equal(a.view(np.uint16) if bf16 else a, h)
    shape = CFG.Shape(n_layers=2)
    lengths = [5, 33, 0]
    pt, n_pages = CFG.page_table(3, [n + 1 for n in lengths], extra_pages=2)
    pool = DEV.kv_pool(3, shape, 2, lengths, pt, n_pages, True).cpu().numpy().view(np.uint16)
    used = set()
    for l in range(2):
        for b, n in enumerate(lengths):
            k, v = CFG.kv_prefill(3, shape, l, b, n, True)
            for p in range(n):
                pg = pt[b, p // 16]
                used.add(pg)
                assert np.array_equal(pool[l, pg, 0, :, p % 16, :], k[p])
                assert np.array_equal(pool[l, pg, 1, :, p % 16, :], v[p])
    free = [p for p in range(n_pages) if p not in used]
    assert np.all(pool[:, free] == 0)


# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("bf16", [True, False])
def test_codebook_embed_bit_exact(bf16):
    m = Model(CFG.Shape(), 0, bf16)
    T = m.T
    try:
        K, V, R, TV = 16, 2048, 37, 500
        tables_h = CFG.table(0, gen.KIND_CB_TABLE, 0, K * V, 1024, bf16)
        text_h = CFG.table(0, gen.KIND_TEXT_TABLE, 0, TV, 1024, bf16)
        codes = gen.uniform_int(0, stream_id(gen.KIND_CODES, 1), (R, K), V)
        codes[3, :] = V - 1
        codes[4, :] = 0
        is_text = np.zeros(R, np.uint8)
        is_text[[0, 7, 36]] = 1
        text_ids = gen.uniform_int(0, stream_id(gen.KIND_TEXT_IDS, 1), (R,), TV)
        out = torch().empty((R, 1024), dtype=torch().float32, device="cuda")
        T.ttsbb_codebook_embed(m.ctx, R, K, t_i32(codes), DEV.host_to_device(tables_h), V,
                               DEV.host_to_device(is_text), t_i32(text_ids),
                               DEV.host_to_device(text_h), TV, out)
        assert T.ttsbb_sync(m.ctx) == T.OK
        got = out.cpu().numpy()
        ref = O.codebook_embed(codes, widen(tables_h), V)
        ref[is_text == 1] = widen(text_h)[text_ids[is_text == 1]]
        assert np.array_equal(got, ref.astype(np.float32))
        # K = 1 is a lookup; zero rows are a no-op
        out1 = torch().empty((R, 1024), dtype=torch().float32, device="cuda")
        T.ttsbb_codebook_embed(m.ctx, R, 1, t_i32(codes[:, :1]), DEV.host_to_device(tables_h), V,
                               None, None, None, 0, out1)
        assert np.array_equal(out1.cpu().numpy(), widen(tables_h)[codes[:, 0]])
        assert T.ttsbb_codebook_embed(m.ctx, 0, K, None, None, V, None, None, None, 0, None) == T.OK
        # an out-of-range code raises the device flag, reported by ttsbb_sync, then clears
        bad = codes.copy()
        bad[5, 2] = V
        T.ttsbb_codebook_embed(m.ctx, R, K, t_i32(bad), DEV.host_to_device(tables_h), V, None,
                               None, None, 0, out)
        assert T.ttsbb_sync(m.ctx) == T.DEVICE_ERROR
        assert T.ttsbb_sync(m.ctx) == T.OK
    finally:
        m.close()


# ---------------------------------------------------------------------------------------
def run_decode(m: Model, lengths, seed, head=None, tap_layer=None, gpu_tap=True):
    """One decode step of len(lengths) streams; returns GPU results and oracle results.
    With gpu_tap=False the oracle still records tap_layer but the GPU runs untapped (every
    layer on the fused q_len = 1 path)."""
    T = m.T
    shape = m.shape
    B = len(lengths)
    pt, n_pages = CFG.page_table(seed, [n + 1 for n in lengths], extra_pages=3)
    pool = DEV.kv_pool(seed, shape, m.n_layers, lengths, pt, n_pages, m.bf16)
    x_in = gen.fast_normal(seed, stream_id(gen.KIND_X_IN, 0), (B, shape.hidden), 1.0)
    x = t_f32(x_in)
    pos = t_i32(lengths)
    res = {}
    if tap_layer is not None and gpu_tap:
        T.ttsbb_set_tap_layer(m.ctx, tap_layer)
    if head is not None:
        hd_dev, G, V = head[:3]
        am = torch().empty((B, G), dtype=torch().int32, device="cuda")
        lg = torch().empty((B, G * V), dtype=torch().float32, device="cuda")
        T.ttsbb_decode_step(m.ctx, B, x, pos, t_i32(pt), pt.shape[1], pool, n_pages, hd_dev, G, V, am, lg)
    else:
        T.ttsbb_decode_step(m.ctx, B, x, pos, t_i32(pt), pt.shape[1], pool, n_pages)
    assert T.ttsbb_sync(m.ctx) == T.OK
    res["x"] = x.cpu().numpy()
    res["pos"] = pos.cpu().numpy()
    res["pool"] = DEV.bits_to_f32(pool) if m.bf16 else pool.cpu().numpy()
    if head is not None:
        res["argmax"] = am.cpu().numpy()
        res["logits"] = lg.cpu().numpy()
    if tap_layer is not None and gpu_tap:
        taps = {}
        w = dict(h=(T.TAP_H_ATTN, shape.hidden),
                 qkv=(T.TAP_QKV, (shape.n_heads + 2 * shape.n_kv_heads) * shape.head_dim),
                 q=(T.TAP_Q, shape.n_heads * shape.head_dim),
                 o=(T.TAP_ATTN, shape.n_heads * shape.head_dim), x1=(T.TAP_X_MID, shape.hidden),
                 h2=(T.TAP_H_FFN, shape.hidden), m=(T.TAP_MLP, shape.ffn),
                 x2=(T.TAP_X_OUT, shape.hidden), x_in=(T.TAP_X_IN, shape.hidden))
        for k, (tp, cols) in w.items():
            taps[k] = read_tap(m, tp, B, cols)
        res["taps"] = taps
        T.ttsbb_set_tap_layer(m.ctx, -1)

    cache = O.KVCache(m.n_layers, B)
    for l in range(m.n_layers):
        for b, n in enumerate(lengths):
            if n:
                k, v = CFG.kv_prefill(seed, shape, l, b, n, m.bf16)
                cache.set(l, b, widen(k), widen(v))
    rec = {}
    out = O.decode_step(x_in, list(lengths), cache, m.oracle_layers(), dims_of(shape),
                        record_layer=tap_layer, record=rec)
    ref = {"x": out, "rec": rec, "cache": cache, "pt": pt}
    if head is not None:
        y, lg_ref = O.head_logits(out, m.oracle_final_norm(), head[3], shape.eps)
        ref["logits"] = lg_ref
    return res, ref


def rec_as_taps(rec, B):
    return dict(h=rec["h"], qkv=np.concatenate([rec["q_raw"].reshape(B, -1), rec["k_raw"].reshape(B, -1),
                                                 rec["v"].reshape(B, -1)], axis=1),
                q=rec["q"].reshape(B, -1), o=rec["o"].reshape(B, -1), x1=rec["x1"], h2=rec["h2"],
                m=rec["m"], x2=rec["x2"])


def test_decode_fp32_single_layer_kv64():
    """One layer, fp32, batch 1, KV prefilled to 64 (the fp32 single-layer workload)."""
    w = CFG.c1()
    m = Model(w.shape, 1, False, seed=w.seed)
    try:
        res, ref = run_decode(m, [64], w.seed, tap_layer=0)
        assert np.max(np.abs(res["x"] - ref["x"])) <= 1e-4
        taps, rtaps = res["taps"], rec_as_taps(ref["rec"], 1)
        for k in rtaps:
            assert np.max(np.abs(taps[k] - rtaps[k])) <= 1e-4, k
        # K and V of the new token sit at position 64 of the paged pool
        pg = ref["pt"][0, 64 // 16]
        np.testing.assert_allclose(res["pool"][0, pg, 0, :, 0, :], ref["rec"]["k"][0], atol=1e-4)
        np.testing.assert_allclose(res["pool"][0, pg, 1, :, 0, :], ref["rec"]["v"][0], atol=1e-4)
        assert res["pos"].tolist() == [65]
    finally:
        m.close()


@pytest.mark.parametrize("bf16,lengths", [(False, [64]), (False, [0, 5, 16, 17, 40]),
                                          (True, [0, 1, 15, 16, 17, 33, 64, 100, 129])])
def test_decode_step_token_fused(bf16, lengths):
    """No tap: the step token's head norms, RoPE and K/V append run inside the attention
    kernel.  The layer output and the K / V the kernel wrote to each stream's slot at
    position L_b match the oracle (fp32: 1e-4 max-abs; bf16: the layer tolerance)."""
    shape = CFG.Shape(n_layers=1)
    m = Model(shape, 1, bf16, seed=13, gains="random")
    try:
        res, ref = run_decode(m, lengths, 13, tap_layer=0, gpu_tap=False)
        if bf16:
            assert normwise(res["x"], ref["x"]) <= TOL_LAYER_BF16
        else:
            assert np.max(np.abs(res["x"] - ref["x"])) <= 1e-4
        assert res["pos"].tolist() == [n + 1 for n in lengths]
        for b, n in enumerate(lengths):
            pg, slot = ref["pt"][b, n // 16], n % 16
            k_got, v_got = res["pool"][0, pg, 0, :, slot, :], res["pool"][0, pg, 1, :, slot, :]
            k_ref, v_ref = ref["rec"]["k"][b], ref["rec"]["v"][b]
            if bf16:  # bf16 operands of the projection, then bf16 storage
                assert normwise(k_got, k_ref) <= TOL_LAYER_BF16, b
                assert normwise(v_got, v_ref) <= TOL_LAYER_BF16, b
            else:
                np.testing.assert_allclose(k_got, k_ref, atol=1e-4)
                np.testing.assert_allclose(v_got, v_ref, atol=1e-4)
    finally:
        m.close()


@pytest.mark.parametrize("tap", [False, True])
def test_decode_bad_page_and_position_raise_flag(tap):
    """A stream whose slot page id is invalid, or whose position lies past its page-table
    row, raises the device flag (reported once by ttsbb_sync, then cleared) on both the
    fused and the separate step-token path; only the valid streams' slots are written and
    nothing faults."""
    shape = CFG.Shape(n_layers=1)
    m = Model(shape, 1, True, seed=3)
    T = m.T
    try:
        lengths = [20, 40]
        pt, n_pages = CFG.page_table(3, [n + 1 for n in lengths], extra_pages=1)
        pool = DEV.kv_pool(3, shape, 1, lengths, pt, n_pages, True)
        x = t_f32(gen.fast_normal(3, stream_id(gen.KIND_X_IN, 0), (2, shape.hidden), 1.0))
        if tap:
            T.ttsbb_set_tap_layer(m.ctx, 0)

        def changed(before):
            d = (pool != before).any(dim=-1).nonzero().cpu().numpy()  # (layer, page, kv, head, slot)
            return sorted({(int(r[1]), int(r[2]), int(r[4])) for r in d})

        pt_bad = pt.copy()
        pt_bad[0, 20 // 16] = -1  # stream 0's slot page
        before = pool.clone()
        T.ttsbb_decode_step(m.ctx, 2, x.clone(), t_i32(lengths), t_i32(pt_bad), pt.shape[1], pool, n_pages)
        assert T.ttsbb_sync(m.ctx) == T.DEVICE_ERROR
        assert T.ttsbb_sync(m.ctx) == T.OK
        p1 = int(pt[1, 40 // 16])
        assert changed(before) == [(p1, 0, 40 % 16), (p1, 1, 40 % 16)]

        far = [20, 16 * pt.shape[1] + 5]  # stream 1 past its row (max_pages pages of 16)
        before = pool.clone()
        T.ttsbb_decode_step(m.ctx, 2, x.clone(), t_i32(far), t_i32(pt), pt.shape[1], pool, n_pages)
        assert T.ttsbb_sync(m.ctx) == T.DEVICE_ERROR
        assert T.ttsbb_sync(m.ctx) == T.OK
        p0 = int(pt[0, 20 // 16])
        assert changed(before) == [(p0, 0, 20 % 16), (p0, 1, 20 % 16)]
        if tap:
            T.ttsbb_set_tap_layer(m.ctx, -1)
    finally:
        m.close()


def test_decode_fp32_ragged_batch_random_gains():
    shape = CFG.Shape(n_layers=2)
    m = Model(shape, 2, False, seed=11, gains="random")
    try:
        lengths = [0, 5, 16, 17, 40]
        res, ref = run_decode(m, lengths, 11, tap_layer=1)
        assert np.max(np.abs(res["x"] - ref["x"])) <= 1e-4
        rtaps = rec_as_taps(ref["rec"], len(lengths))
        for k in rtaps:
            assert np.max(np.abs(res["taps"][k] - rtaps[k])) <= 1e-4, k
        assert res["pos"].tolist() == [n + 1 for n in lengths]
    finally:
        m.close()


@pytest.mark.parametrize("lengths", [[3, 300, 31], [0, 1, 15, 16, 17, 33, 64, 100, 129, 250, 7],
                                     [(29 * i) % 97 for i in range(9)], [(31 * i) % 160 for i in range(17)],
                                     [(37 * i) % 211 for i in range(40)],
                                     [(53 * i + 5) % 301 for i in range(64)]])
def test_decode_bf16_ragged_with_head(lengths):
    """bf16, 2 layers.  Batch 3 takes the GEMV path; batches 9, 11, 17, 40 and 64 the skinny
    MFMA path with one, two, three (padded to four) and four 16-row tiles, its split-K
    products with the residual update deferred to the next RMSNorm (o and down
    projections) and a ragged head width (3 x 37 columns)."""
    shape = CFG.Shape(n_layers=2)
    m = Model(shape, 2, True, seed=5, gains="random")
    try:
        G, V = 3, 37
        head_h = CFG.table(5, gen.KIND_HEAD, 0, G * V, shape.hidden, True)
        head = (DEV.host_to_device(head_h), G, V, widen(head_h))
        res, ref = run_decode(m, lengths, 5, head=head, tap_layer=0)
        assert normwise(res["x"], ref["x"]) <= TOL_LAYER_BF16
        rtaps = rec_as_taps(ref["rec"], len(lengths))
        for k in rtaps:
            assert normwise(res["taps"][k], rtaps[k]) <= TOL_LAYER_BF16, k
        assert normwise(res["logits"], ref["logits"]) <= TOL_LAYER_BF16
        B = len(lengths)
        check_argmax_groups(res["argmax"], res["logits"].reshape(B, G, V),
                            ref["logits"].reshape(B, G, V))
    finally:
        m.close()


@pytest.mark.parametrize("lengths", [[(29 * i) % 97 for i in range(9)], [(31 * i) % 160 for i in range(17)],
                                     [(37 * i) % 211 for i in range(40)]])
def test_decode_bf16_untapped_fragment_major(lengths):
    """bf16, 2 layers and a head, nothing tapped: batches 9, 17 and 40 run every product
    on the skinny kernel with its operands in the fragment-major layout (one, two, and
    three 16-row tiles padded to four), written by the RMSNorm, the chunk merge and the
    SwiGLU epilogue; outputs, logits and choices against the oracle."""
    shape = CFG.Shape(n_layers=2)
    m = Model(shape, 2, True, seed=5, gains="random")
    try:
        G, V = 3, 37
        head_h = CFG.table(5, gen.KIND_HEAD, 0, G * V, shape.hidden, True)
        head = (DEV.host_to_device(head_h), G, V, widen(head_h))
        res, ref = run_decode(m, lengths, 5, head=head)
        assert normwise(res["x"], ref["x"]) <= TOL_LAYER_BF16
        assert normwise(res["logits"], ref["logits"]) <= TOL_LAYER_BF16
        B = len(lengths)
        check_argmax_groups(res["argmax"], res["logits"].reshape(B, G, V),
                            ref["logits"].reshape(B, G, V))
    finally:
        m.close()


# ---------------------------------------------------------------------------------------
def run_maskgit(m: Model, n_text, n_frames, n_cb, V, mask_id, n_unmask, seed, tap_layer=None,
                text_vocab=500, masked_frac=0.5):
    T = m.T
    shape = m.shape
    text_h = CFG.table(seed, gen.KIND_TEXT_TABLE, 0, text_vocab, shape.hidden, True)
    tab_h = CFG.table(seed, gen.KIND_CB_TABLE, 0, n_cb * V, shape.hidden, True)
    head_h = CFG.table(seed, gen.KIND_HEAD, 0, n_cb * V, shape.hidden, True)
    text_ids = gen.uniform_int(seed, stream_id(gen.KIND_TEXT_IDS, 0), (n_text,), text_vocab)
    codes = gen.uniform_int(seed, stream_id(gen.KIND_CODES, 0), (n_cb, n_frames), V - 1)
    perm = gen.permutation(seed, stream_id(gen.KIND_MASK_PERM, 0), n_cb * n_frames)
    codes.reshape(-1)[perm[:int(masked_frac * n_cb * n_frames)]] = mask_id
    codes_d = t_i32(codes)
    pred = torch().empty((n_cb, n_frames), dtype=torch().int32, device="cuda")
    conf = torch().empty((n_cb, n_frames), dtype=torch().float32, device="cuda")
    picked = torch().empty(max(1, n_unmask), dtype=torch().int32, device="cuda")
    T.ttsbb_set_tap_layer(m.ctx, 0 if tap_layer is None else tap_layer)
    T.ttsbb_maskgit_pass(m.ctx, n_text, t_i32(text_ids), DEV.host_to_device(text_h), text_vocab,
                         n_frames, n_cb, V, mask_id, DEV.host_to_device(tab_h),
                         DEV.host_to_device(head_h), codes_d, n_unmask, 5.0, pred, conf, picked)
    assert T.ttsbb_sync(m.ctx) == T.OK
    res = dict(codes=codes_d.cpu().numpy(), pred=pred.cpu().numpy(), conf=conf.cpu().numpy(),
               picked=picked.cpu().numpy()[:n_unmask],
               logits=read_tap(m, T.TAP_LOGITS, n_frames, n_cb * V),
               head_in=read_tap(m, T.TAP_HEAD_IN, n_frames, shape.hidden))
    S = n_text + n_frames
    if tap_layer is not None:
        res["taps"] = {k: read_tap(m, tp, S, c) for k, (tp, c) in dict(
            x_in=(T.TAP_X_IN, shape.hidden), q=(T.TAP_Q, shape.n_heads * 128),
            k=(T.TAP_K, shape.n_kv_heads * 128), v=(T.TAP_V, shape.n_kv_heads * 128),
            o=(T.TAP_ATTN, shape.n_heads * 128), x1=(T.TAP_X_MID, shape.hidden),
            m=(T.TAP_MLP, shape.ffn), x2=(T.TAP_X_OUT, shape.hidden)).items()}
    T.ttsbb_set_tap_layer(m.ctx, -1)

    rec, lrec = {}, {}
    x0 = O.hybrid_embed(text_ids, widen(text_h), codes, widen(tab_h), V)
    if tap_layer is not None:
        O.backbone_full(x0, m.oracle_layers(), dims_of(shape), causal=False,
                        record_layer=tap_layer, record=lrec)
    new_codes, pred_r, conf_r, picked_r = O.maskgit_pass(
        text_ids, widen(text_h), codes, widen(tab_h), widen(head_h), m.oracle_layers(),
        m.oracle_final_norm(), dims_of(shape), V, mask_id, 5.0, n_unmask, record=rec)
    ref = dict(codes_in=codes, rec=rec, lrec=lrec, conf=conf_r, pred=pred_r, x0=x0)
    return res, ref


def check_maskgit(res, ref, n_cb, n_frames, V, mask_id, n_unmask, tol=2e-2):
    rec = ref["rec"]
    assert normwise(res["logits"], rec["logits"]) <= tol
    g = res["logits"].reshape(n_frames, n_cb, V).transpose(1, 0, 2)
    r = rec["logits"].reshape(n_frames, n_cb, V).transpose(1, 0, 2)
    check_argmax_groups(res["pred"], g, r, exclude=mask_id)
    # confidence: same masked set, and within twice the logit error
    fin = np.isfinite(ref["conf"])
    assert np.array_equal(np.isfinite(res["conf"]), fin)
    delta = np.max(np.abs(res["logits"] - rec["logits"]))
    assert np.max(np.abs(res["conf"][fin] - ref["conf"][fin])) <= 2 * delta + 1e-5
    check_topn(res["picked"], res["conf"], ref["conf"], n_unmask)
    # the update writes pred at the picked positions and nothing else
    assert np.array_equal(res["codes"], O.apply_picks(ref["codes_in"], res["pred"], res["picked"]))


def test_maskgit_zero_layers_head_and_selection():
    """n_layers = 0: embedding -> final norm -> heads -> scores -> selection."""
    m = Model(CFG.Shape(n_layers=0), 0, True, seed=3, gains="random")
    try:
        n_text, n_frames, n_cb, V, mask = 5, 83, 4, 65, 64
        n = 50
        res, ref = run_maskgit(m, n_text, n_frames, n_cb, V, mask, n, 3)
        check_maskgit(res, ref, n_cb, n_frames, V, mask, n, tol=1e-2)
    finally:
        m.close()


@pytest.mark.parametrize("n_text,n_frames,n_unmask", [(13, 57, 40), (0, 64, 150), (70, 3, 6), (1, 64, 20),
                                                    (77, 123, 60), (0, 129, 33)])
def test_maskgit_two_layers(n_text, n_frames, n_unmask):
    """bf16, 2 bidirectional layers, ragged sequence (several key blocks and a tail), heads
    whose width is not a tile multiple; n_unmask beyond the masked count -> -1.  S = 64 runs
    the skinny products and the separate RoPE / V^T kernels; S = 65, 70, 73, 129, 200 the
    LDS-DMA products with the fused q|k|v epilogue (one or two 128-token tiles, a ragged
    last tile), split residual products, and attention with empty key quarters (S <= 96)."""
    m = Model(CFG.Shape(n_layers=2), 2, True, seed=4, gains="random")
    try:
        n_cb, V, mask = 3, 33, 32
        res, ref = run_maskgit(m, n_text, n_frames, n_cb, V, mask, n_unmask, 4, tap_layer=1)
        check_maskgit(res, ref, n_cb, n_frames, V, mask, n_unmask)
        lrec = ref["lrec"]
        S = n_text + n_frames
        for k, rk in dict(x_in=None, q="q", k="k", v="v", o="o", x1="x1", m="m", x2="x2").items():
            if rk is None:
                continue
            assert normwise(res["taps"][k], lrec[rk].reshape(S, -1)) <= TOL_LAYER_BF16, k
        if n_unmask > (ref["codes_in"] == mask).sum():
            assert (res["picked"] == -1).sum() == n_unmask - (ref["codes_in"] == mask).sum()
    finally:
        m.close()



@pytest.mark.parametrize("n_text,n_frames", [(20, 130), (5, 60)])
def test_maskgit_without_gqa(n_text, n_frames):
    """bf16, one bidirectional layer with as many KV heads as query heads: the attention
    kernel's one-head-per-group form (the two waves of a key quarter take two query tiles
    of one head), and the fused q|k|v epilogue with 8 + 8 + 8 heads."""
    m = Model(CFG.Shape(n_layers=1, n_heads=8, n_kv_heads=8), 1, True, seed=11, gains="random")
    try:
        n_cb, V, mask, n_unmask = 3, 33, 32, 40
        res, ref = run_maskgit(m, n_text, n_frames, n_cb, V, mask, n_unmask, 6, tap_layer=0)
        check_maskgit(res, ref, n_cb, n_frames, V, mask, n_unmask)
        S = n_text + n_frames
        for k in ("q", "k", "v", "o", "x1", "m", "x2"):
            assert normwise(res["taps"][k], ref["lrec"][k].reshape(S, -1)) <= TOL_LAYER_BF16, k
    finally:
        m.close()

def test_maskgit_deterministic():
    m = Model(CFG.Shape(n_layers=1), 1, True, seed=9)
    try:
        a, _ = run_maskgit(m, 9, 40, 2, 33, 32, 10, 9)
        b, _ = run_maskgit(m, 9, 40, 2, 33, 32, 10, 9)
        for k in ("codes", "pred", "conf", "picked", "logits"):
            assert np.array_equal(a[k], b[k]), k
    finally:
        m.close()


# ---------------------------------------------------------------------------------------
# Guided MaskGIT step (classifier-free guidance)
# ---------------------------------------------------------------------------------------
def run_maskgit_cfg(m: Model, n_text, n_frames, n_target, n_cb, V, mask_id, n_unmask, cfg_scale, seed,
                    text_vocab=500, masked_frac=0.5):
    T = m.T
    shape = m.shape
    text_h = CFG.table(seed, gen.KIND_TEXT_TABLE, 0, text_vocab, shape.hidden, True)
    tab_h = CFG.table(seed, gen.KIND_CB_TABLE, 0, n_cb * V, shape.hidden, True)
    head_h = CFG.table(seed, gen.KIND_HEAD, 0, n_cb * V, shape.hidden, True)
    text_ids = gen.uniform_int(seed, stream_id(gen.KIND_TEXT_IDS, 0), (n_text,), text_vocab)
    codes = gen.uniform_int(seed, stream_id(gen.KIND_CODES, 0), (n_cb, n_frames), V - 1)
    w0 = n_frames - n_target
    perm = gen.permutation(seed, stream_id(gen.KIND_MASK_PERM, 0), n_cb * n_target)
    win = codes[:, w0:].copy().reshape(-1)
    win[perm[:int(masked_frac * n_cb * n_target)]] = mask_id
    codes[:, w0:] = win.reshape(n_cb, n_target)
    codes_d = t_i32(codes)
    pred = torch().empty((n_cb, n_target), dtype=torch().int32, device="cuda")
    conf = torch().empty((n_cb, n_target), dtype=torch().float32, device="cuda")
    picked = torch().empty(max(1, n_unmask), dtype=torch().int32, device="cuda")
    T.ttsbb_set_tap_layer(m.ctx, 0)
    T.ttsbb_maskgit_pass_cfg(m.ctx, n_text, t_i32(text_ids), DEV.host_to_device(text_h), text_vocab, n_frames,
                             n_target, n_cb, V, mask_id, DEV.host_to_device(tab_h), DEV.host_to_device(head_h),
                             codes_d, n_unmask, 5.0, cfg_scale, pred, conf, picked)
    assert T.ttsbb_sync(m.ctx) == T.OK
    res = dict(codes=codes_d.cpu().numpy(), pred=pred.cpu().numpy(), conf=conf.cpu().numpy(),
               picked=picked.cpu().numpy()[:n_unmask],
               logits_c=read_tap(m, T.TAP_LOGITS, n_target, n_cb * V),
               logits_u=read_tap(m, T.TAP_LOGITS_U, n_target, n_cb * V))
    T.ttsbb_set_tap_layer(m.ctx, -1)
    rec = {}
    O.maskgit_pass_cfg(text_ids, widen(text_h), codes, n_target, widen(tab_h), widen(head_h), m.oracle_layers(),
                       m.oracle_final_norm(), dims_of(shape), V, mask_id, 5.0, n_unmask, cfg_scale, record=rec)
    return res, dict(codes_in=codes, rec=rec, inputs=(text_ids, text_h, tab_h, head_h, codes))


@pytest.mark.parametrize("n_text,n_frames,n_target,n_unmask,scale,max_rows",
                         [(13, 57, 40, 30, 2.0, 1024), (70, 130, 100, 77, 3.0, 1024), (0, 50, 50, 20, 1.5, 1024),
                          (13, 57, 40, 30, 2.0, 100), (70, 130, 100, 77, 3.0, 300), (5, 27, 20, 9, 2.5, 1024)])
def test_maskgit_cfg_two_layers(n_text, n_frames, n_target, n_unmask, scale, max_rows):
    """bf16, 2 layers: both passes' logits against the oracle's, the guided choice and
    scores (discrete parity on the guided logits), the top-n picks and the update of the
    window only.  With room in the workspace the two passes run as one batch of two
    sequences (rows [0, S) and [S rounded up to 64, + n_target): M = 168, 356, 114 and 84,
    the last with a 32-row first sequence followed by 32 padding rows); max_rows 100 and
    300 force two separate passes (M <= 64 products for the first, the LDS-DMA products
    with the fused q|k|v epilogue for the second)."""
    m = Model(CFG.Shape(n_layers=2), 2, True, seed=6, gains="random", max_rows=max_rows)
    try:
        n_cb, V, mask = 3, 33, 32
        res, ref = run_maskgit_cfg(m, n_text, n_frames, n_target, n_cb, V, mask, n_unmask, scale, 6)
        rec = ref["rec"]
        assert normwise(res["logits_c"], rec["logits_c"]) <= TOL_LAYER_BF16
        assert normwise(res["logits_u"], rec["logits_u"]) <= TOL_LAYER_BF16
        g_gpu = O.cfg_logits(res["logits_c"], res["logits_u"], scale)
        gv = g_gpu.reshape(n_target, n_cb, V).transpose(1, 0, 2)
        rv = rec["guided"].reshape(n_target, n_cb, V).transpose(1, 0, 2)
        check_argmax_groups(res["pred"], gv, rv, exclude=mask)
        fin = np.isfinite(rec["conf"])
        assert np.array_equal(np.isfinite(res["conf"]), fin)
        delta = np.max(np.abs(g_gpu - rec["guided"]))
        assert np.max(np.abs(res["conf"][fin] - rec["conf"][fin])) <= 2 * delta + 1e-4
        check_topn(res["picked"], res["conf"], rec["conf"], n_unmask)
        w0 = n_frames - n_target
        codes_in = ref["codes_in"]
        np.testing.assert_array_equal(res["codes"][:, :w0], codes_in[:, :w0])
        np.testing.assert_array_equal(res["codes"][:, w0:], O.apply_picks(codes_in[:, w0:], res["pred"],
                                                                          res["picked"]))
    finally:
        m.close()


def test_maskgit_cfg_without_context_is_the_plain_step():
    """No text and a window covering every frame: the two passes see the same sequence,
    compute bit-identical logits, and the guided step returns exactly the plain step's
    choices, scores, picks and codes, whatever the scale."""
    m = Model(CFG.Shape(n_layers=1), 1, True, seed=8)
    try:
        T = m.T
        n_cb, V, mask, n_frames, n_unmask = 2, 33, 32, 75, 25
        tab_h = CFG.table(8, gen.KIND_CB_TABLE, 0, n_cb * V, m.shape.hidden, True)
        head_h = CFG.table(8, gen.KIND_HEAD, 0, n_cb * V, m.shape.hidden, True)
        codes = gen.uniform_int(8, stream_id(gen.KIND_CODES, 0), (n_cb, n_frames), V - 1)
        codes[:, ::2] = mask
        outs = []
        for cfg in (None, 0.0, 4.0):
            cd = t_i32(codes)
            pred = torch().empty((n_cb, n_frames), dtype=torch().int32, device="cuda")
            conf = torch().empty((n_cb, n_frames), dtype=torch().float32, device="cuda")
            picked = torch().empty(n_unmask, dtype=torch().int32, device="cuda")
            args = (DEV.host_to_device(tab_h), DEV.host_to_device(head_h), cd, n_unmask, 5.0)
            if cfg is None:
                T.ttsbb_maskgit_pass(m.ctx, 0, None, None, 0, n_frames, n_cb, V, mask, *args, pred, conf, picked)
            else:
                T.ttsbb_maskgit_pass_cfg(m.ctx, 0, None, None, 0, n_frames, n_frames, n_cb, V, mask, *args, cfg,
                                         pred, conf, picked)
            assert T.ttsbb_sync(m.ctx) == T.OK
            outs.append([a.cpu().numpy() for a in (cd, pred, conf, picked)])
        for o in outs[1:]:
            for a, b in zip(outs[0], o):
                np.testing.assert_array_equal(a, b)
    finally:
        m.close()


@pytest.mark.parametrize("n_text,n_frames,n_target,cfg_scale,class_temp,pos_temp",
                         [(13, 57, 40, 0.0, 1.0, 0.0), (13, 57, 40, 2.0, 0.7, 0.5), (70, 130, 100, 3.0, 1.5, 1.0),
                          (0, 45, 45, 0.0, 0.0, 2.0)])
def test_maskgit_step_sampler(n_text, n_frames, n_target, cfg_scale, class_temp, pos_temp):
    """The general step with the sampler: top-k ratio filter, class temperature with
    Gumbel noise and position noise from given uniforms, with and without guidance;
    choices and scores in two-stage discrete parity (GPU vs an fp64 emulation on its own
    logits, emulation vs the oracle), picks, and the window update."""
    m = Model(CFG.Shape(n_layers=2), 2, True, seed=12, gains="random")
    try:
        T = m.T
        shape = m.shape
        n_cb, V, mask, n_unmask, ratio, seed, tv = 3, 33, 32, 25, 0.25, 12, 500
        text_h = CFG.table(seed, gen.KIND_TEXT_TABLE, 0, tv, shape.hidden, True)
        tab_h = CFG.table(seed, gen.KIND_CB_TABLE, 0, n_cb * V, shape.hidden, True)
        head_h = CFG.table(seed, gen.KIND_HEAD, 0, n_cb * V, shape.hidden, True)
        text_ids = gen.uniform_int(seed, stream_id(gen.KIND_TEXT_IDS, 0), (n_text,), tv)
        codes = gen.uniform_int(seed, stream_id(gen.KIND_CODES, 0), (n_cb, n_frames), V - 1)
        w0 = n_frames - n_target
        win = codes[:, w0:].copy()
        win[:, ::2] = mask
        win[1, 1::4] = mask
        codes[:, w0:] = win
        u_class = gen.uniform_open01(seed, stream_id(gen.KIND_U_CLASS, 0), (n_cb, n_target, V))
        u_pos = gen.uniform_open01(seed, stream_id(gen.KIND_U_POS, 0), (n_cb, n_target))
        codes_d = t_i32(codes)
        pred = torch().empty((n_cb, n_target), dtype=torch().int32, device="cuda")
        conf = torch().empty((n_cb, n_target), dtype=torch().float32, device="cuda")
        picked = torch().empty(n_unmask, dtype=torch().int32, device="cuda")
        T.ttsbb_set_tap_layer(m.ctx, 0)
        T.ttsbb_maskgit_step(m.ctx, n_text, t_i32(text_ids), DEV.host_to_device(text_h), tv, n_frames, n_target,
                             n_cb, V, mask, DEV.host_to_device(tab_h), DEV.host_to_device(head_h), codes_d, n_unmask,
                             5.0, pred, conf, picked, cfg_scale=cfg_scale, class_temp=class_temp, pos_temp=pos_temp,
                             top_k_ratio=ratio, u_class=t_f32(u_class), u_pos=t_f32(u_pos))
        assert T.ttsbb_sync(m.ctx) == T.OK
        lc = read_tap(m, T.TAP_LOGITS, n_target, n_cb * V)
        guided_gpu = O.cfg_logits(lc, read_tap(m, T.TAP_LOGITS_U, n_target, n_cb * V), cfg_scale) \
            if cfg_scale != 0 else lc
        T.ttsbb_set_tap_layer(m.ctx, -1)
        res_codes, res_pred, res_conf = codes_d.cpu().numpy(), pred.cpu().numpy(), conf.cpu().numpy()
        res_picked = picked.cpu().numpy()
        rec = {}
        O.maskgit_step(text_ids, widen(text_h), codes, n_target, widen(tab_h), widen(head_h), m.oracle_layers(),
                       m.oracle_final_norm(), dims_of(shape), V, mask, 5.0, n_unmask, cfg_scale, class_temp,
                       pos_temp, ratio, u_class.astype(np.float64), u_pos.astype(np.float64), record=rec)
        assert normwise(guided_gpu, rec["guided"]) <= 3 * TOL_LAYER_BF16 * (1 + abs(cfg_scale))
        ex1, ex2 = check_sampler(res_pred, res_conf, guided_gpu, rec["guided"], win, n_cb, V, mask, 5.0,
                                 class_temp, pos_temp, ratio, u_class.astype(np.float64),
                                 u_pos.astype(np.float64))
        # explained exceptions stay rare (fp32 vs fp64 ties; bf16 logit error at the edges)
        assert ex1 <= 2 and ex2 <= max(3, n_cb * n_target // 20), (ex1, ex2)
        # picks: exactly the top-n of the GPU's own scores; the update touches the window only
        check_topn(res_picked, res_conf, res_conf, n_unmask)
        np.testing.assert_array_equal(res_codes[:, :w0], codes[:, :w0])
        np.testing.assert_array_equal(res_codes[:, w0:], O.apply_picks(win, res_pred, res_picked))
    finally:
        m.close()


# ---------------------------------------------------------------------------------------
# Codec RVQ decode
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("n_frames,n_q,cb,dim,out_dim", [(750, 8, 1024, 64, 1024), (37, 3, 100, 48, 200),
                                                         (1, 1, 5, 130, 7)])
def test_rvq_decode(n_frames, n_q, cb, dim, out_dim):
    """fp32 against the oracle to 1e-4 max-abs (the quantizer accuracy the ncnn port reports
    against PyTorch); the first shape is the 8 x 1024 x 64 -> 1024 quantizer of the
    OmniVoice codec over 30 s of frames, the others ragged tiles and a codebook dimension
    that is not a multiple of the 64-wide slices."""
    m = Model(CFG.Shape(n_layers=1), 0, False, seed=13)
    try:
        T = m.T
        seed = 13
        emb = gen.normal_f32(seed, stream_id(gen.KIND_CB_TABLE, 3), (n_q, cb, dim), 1.0)
        w = gen.normal_f32(seed, stream_id(gen.KIND_HEAD, 3), (n_q, out_dim, dim), 0.05)
        b = gen.normal_f32(seed, stream_id(gen.KIND_FINAL_NORM, 3), (n_q, out_dim), 0.1)
        codes = gen.uniform_int(seed, stream_id(gen.KIND_CODES, 3), (n_q, n_frames), cb)
        codes[0, 0] = cb - 1
        codes[-1, -1] = 0
        out = torch().empty((n_frames, out_dim), dtype=torch().float32, device="cuda")
        T.ttsbb_rvq_decode(m.ctx, n_frames, n_q, cb, dim, out_dim, t_i32(codes), t_f32(emb), t_f32(w), t_f32(b), out)
        assert T.ttsbb_sync(m.ctx) == T.OK
        ref = O.rvq_decode(codes, emb, w, b)
        assert np.max(np.abs(out.cpu().numpy() - ref)) <= 1e-4
        # an out-of-range code is clamped and reported, then the flag clears
        bad = codes.copy()
        bad[-1, 0] = cb
        T.ttsbb_rvq_decode(m.ctx, n_frames, n_q, cb, dim, out_dim, t_i32(bad), t_f32(emb), t_f32(w), t_f32(b), out)
        assert T.ttsbb_sync(m.ctx) == T.DEVICE_ERROR
        assert T.ttsbb_sync(m.ctx) == T.OK
    finally:
        m.close()


# ---------------------------------------------------------------------------------------
# Causal prefill of one stream into its paged cache
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("p0,S", [(0, 5), (21, 37), (0, 100), (300, 64)])
def test_prefill_bf16(p0, S):
    """bf16, 2 layers: the prompt's final residual stream, the K/V it leaves in the pool at
    positions p0..p0+S-1, the advanced cache length and the last token's head choice,
    against the oracle's prefill (which the oracle pins equal to token-by-token decode)."""
    shape = CFG.Shape(n_layers=2)
    m = Model(shape, 2, True, seed=17, gains="random")
    try:
        T = m.T
        seed = 17
        pt, n_pages = CFG.page_table(seed, [p0 + S + 1], extra_pages=2)
        pool = DEV.kv_pool(seed, shape, 2, [p0], pt, n_pages, True)
        x_in = gen.fast_normal(seed, stream_id(gen.KIND_X_IN, 1), (S, shape.hidden), 1.0)
        x = t_f32(x_in)
        cl = t_i32(np.array([p0]))
        G, V = 3, 37
        head_h = CFG.table(seed, gen.KIND_HEAD, 0, G * V, shape.hidden, True)
        am = torch().empty(G, dtype=torch().int32, device="cuda")
        lg = torch().empty(G * V, dtype=torch().float32, device="cuda")
        T.ttsbb_prefill(m.ctx, S, x, cl, t_i32(pt), pt.shape[1], pool, n_pages, DEV.host_to_device(head_h), G, V,
                        am, lg)
        assert T.ttsbb_sync(m.ctx) == T.OK
        assert cl.cpu().numpy().tolist() == [p0 + S]
        cache = O.KVCache(2, 1)
        for l in range(2):
            if p0:
                k, v = CFG.kv_prefill(seed, shape, l, 0, p0, True)
                cache.set(l, 0, widen(k), widen(v))
        out = O.prefill(x_in, p0, cache, 0, m.oracle_layers(), dims_of(shape))
        assert normwise(x.cpu().numpy(), out) <= TOL_LAYER_BF16
        pool_h = DEV.bits_to_f32(pool)
        for l in range(2):
            for p in range(p0, p0 + S):
                pg, slot = pt[0, p // 16], p % 16
                assert normwise(pool_h[l, pg, 0, :, slot, :], cache.k[l][0][p]) <= TOL_LAYER_BF16
                assert normwise(pool_h[l, pg, 1, :, slot, :], cache.v[l][0][p]) <= TOL_LAYER_BF16
        _, lg_ref = O.head_logits(out[-1:], m.oracle_final_norm(), widen(head_h), shape.eps)
        lg_gpu = lg.cpu().numpy()
        assert normwise(lg_gpu, lg_ref[0]) <= TOL_LAYER_BF16
        check_argmax_groups(am.cpu().numpy()[None], lg_gpu.reshape(1, G, V), lg_ref.reshape(1, G, V))
    finally:
        m.close()


# ---------------------------------------------------------------------------------------
# Edge cases: empty calls, the longest cache a page table allows, a MaskGIT sequence at
# the workspace's row limit
# ---------------------------------------------------------------------------------------
def test_empty_calls_are_no_ops():
    """Zero streams, zero prompt tokens, zero embedding rows and zero picks succeed and
    leave every output untouched."""
    shape = CFG.Shape(n_layers=1)
    m = Model(shape, 1, True, seed=2)
    T = m.T
    try:
        pt, n_pages = CFG.page_table(2, [17])
        pool = DEV.kv_pool(2, shape, 1, [16], pt, n_pages, True)
        before = pool.clone()
        x = torch().zeros((1, shape.hidden), dtype=torch().float32, device="cuda")
        pos = t_i32([16])
        assert T.ttsbb_decode_step(m.ctx, 0, x, pos, t_i32(pt), pt.shape[1], pool, n_pages) == T.OK
        assert T.ttsbb_prefill(m.ctx, 0, x, pos, t_i32(pt), pt.shape[1], pool, n_pages) == T.OK
        out = torch().full((1, shape.hidden), 7.0, dtype=torch().float32, device="cuda")
        tab = DEV.host_to_device(CFG.table(2, gen.KIND_CB_TABLE, 0, 4 * 8, shape.hidden, True))
        assert T.ttsbb_codebook_embed(m.ctx, 0, 4, t_i32(np.zeros((1, 4))), tab, 8, None, None, None, 0, out) == T.OK
        assert T.ttsbb_sync(m.ctx) == T.OK
        assert pos.cpu().tolist() == [16]
        assert torch().equal(pool, before)
        assert bool((out == 7.0).all())
        # a MaskGIT step that unmasks nothing leaves the codes as they were
        res, ref = run_maskgit(m, 5, 40, 2, 17, 16, 0, 2)
        assert np.array_equal(res["codes"], ref["codes_in"])
    finally:
        m.close()


@pytest.mark.parametrize("bf16", [False, True])
def test_decode_longest_cache(bf16):
    """One stream at the last position max_pos - 1 (8191: 512 pages, 64 chunks of 128 merged
    in one pass of 64) next to a short one."""
    shape = CFG.Shape(n_layers=1)
    m = Model(shape, 1, bf16, seed=17, max_pos=8192)
    try:
        lengths = [8191, 3]
        res, ref = run_decode(m, lengths, 17, tap_layer=0, gpu_tap=False)
        if bf16:
            assert normwise(res["x"], ref["x"]) <= TOL_LAYER_BF16
        else:
            assert np.max(np.abs(res["x"] - ref["x"])) <= 1e-4
        assert res["pos"].tolist() == [8192, 4]
    finally:
        m.close()


@pytest.mark.parametrize("bf16", [False, True])
def test_decode_long_stream_multi_pass_merge(bf16):
    """Six streams, one of them at 16000 positions: 125 chunks of 128 (the work list keeps
    the 128-position chunk at this total), merged in two passes of 64; the others in one
    pass.  Every stream's layer output against the oracle."""
    shape = CFG.Shape(n_layers=1)
    m = Model(shape, 1, bf16, seed=23, max_pos=16384)
    try:
        lengths = [8191, 3, 200, 4097, 1000, 16000]
        res, ref = run_decode(m, lengths, 23, tap_layer=0, gpu_tap=False)
        if bf16:
            assert normwise(res["x"], ref["x"]) <= TOL_LAYER_BF16
        else:
            assert np.max(np.abs(res["x"] - ref["x"])) <= 1e-4
        assert res["pos"].tolist() == [n + 1 for n in lengths]
    finally:
        m.close()


def test_decode_more_streams_than_one_plan_pass():
    """1100 streams (more than the work-list kernel's 1024 threads, so its prefix sum runs
    over two passes), short caches including empty ones (position 0), bf16: every
    stream's layer output against the oracle."""
    shape = CFG.Shape(n_layers=1)
    m = Model(shape, 1, True, seed=29, max_rows=1200, max_pos=256)
    try:
        lengths = [int(v) for v in gen.uniform_int(29, stream_id(gen.KIND_CODES, 1), (1100,), 41)]
        lengths[0], lengths[1099] = 0, 40
        res, ref = run_decode(m, lengths, 29, tap_layer=0, gpu_tap=False)
        assert normwise(res["x"], ref["x"]) <= TOL_LAYER_BF16
        assert res["pos"].tolist() == [n + 1 for n in lengths]
    finally:
        m.close()


def test_maskgit_at_row_limit():
    """S = max_rows = 1024 (24 text tokens + 1000 frames): whole 128-row tiles, no ragged
    tail, 32 key blocks; one layer against the oracle."""
    shape = CFG.Shape(n_layers=1)
    m = Model(shape, 1, True, seed=19, max_rows=1024)
    try:
        n_cb, V, mask = 2, 33, 32
        res, ref = run_maskgit(m, 24, 1000, n_cb, V, mask, 300, 19)
        check_maskgit(res, ref, n_cb, 1000, V, mask, 300)
    finally:
        m.close()
