"""GPU parity of the HIP path against the oracle at small sizes (several tiles, ragged
tails, degenerate cases).  Every call goes through the C ABI (codec_token_tts_amd.ttsbb).

Tolerances (derived in the design notes):
* fp32 mode: 1e-4 max-abs on every intermediate and the layer output.
* bf16 mode: normwise max-relative max|gpu-ref|/max|ref| <= TOL_LAYER_BF16 against the
  oracle, <= TOL_EMUL_BF16 against the bf16-storage emulation (tests/bf16_emulation.py).
* discrete outputs: exact argmax / top-n of the GPU's own scores; bit-exact against the
  oracle on the GPU's own head operand (teacher-forced: only fp32 accumulation order
  between the two); against the emulation wherever its margin exceeds twice the measured
  score error, with such near ties capped.
* the codebook embedding: bit-exact (fp64 sum in codebook order, one rounding).
"""
import numpy as np
import pytest

from oracle import backbone as O
from workload import configs as CFG
from workload import device as DEV
from workload import gen
from workload.gen import stream_id

import bf16_emulation as E
from gpu_setup import (BOUNDARY_FRAC, TOL_EMUL_BF16, TOL_LAYER_BF16, Model, check_argmax_groups, check_head_teacher_forced,
                       check_sampler, check_scores_teacher_forced, check_stack, check_topn, dims_of, normwise,
                       read_tap, torch, widen)

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
        # 21 codebooks: the kernel's second round of codebook loads is ragged (5 of 16)
        K2, V2 = 21, 64
        t2_h = CFG.table(0, gen.KIND_CB_TABLE, 1, K2 * V2, 1024, bf16)
        c2 = gen.uniform_int(0, stream_id(gen.KIND_CODES, 2), (R, K2), V2)
        out2 = torch().empty((R, 1024), dtype=torch().float32, device="cuda")
        T.ttsbb_codebook_embed(m.ctx, R, K2, t_i32(c2), DEV.host_to_device(t2_h), V2, None, None, None, 0, out2)
        assert T.ttsbb_sync(m.ctx) == T.OK
        assert np.array_equal(out2.cpu().numpy(), O.codebook_embed(c2, widen(t2_h), V2).astype(np.float32))
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
    if m.bf16:  # the bf16-storage emulation of the same step
        c16 = O.KVCache(m.n_layers, B)
        for l in range(m.n_layers):
            for b, n in enumerate(lengths):
                if n:
                    c16.set(l, b, cache.k[l][b][:n], cache.v[l][b][:n])
        ref["x_emul"] = E.decode_step(x_in, list(lengths), c16, m.oracle_layers(), dims_of(shape))
        if head is not None:
            ref["logits_emul"] = E.head_logits(ref["x_emul"], m.oracle_final_norm(), head[3], shape.eps)[1]
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
        assert normwise(res["x"], ref["x_emul"]) <= TOL_EMUL_BF16
        B = len(lengths)
        check_argmax_groups(res["argmax"], res["logits"].reshape(B, G, V),
                            ref["logits_emul"].reshape(B, G, V))
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
        check_stack("decode untapped x", res["x"], ref["x_emul"], ref["x"])
        B = len(lengths)
        check_argmax_groups(res["argmax"], res["logits"].reshape(B, G, V),
                            ref["logits_emul"].reshape(B, G, V))
    finally:
        m.close()


@pytest.mark.parametrize("bf16,lengths,tap", [(True, [(13 * i) % 111 for i in range(40)], None),
                                              (True, [(7 * i + 3) % 127 for i in range(64)], 1),
                                              (False, [(11 * i) % 97 for i in range(33)], 0)])
def test_decode_direct_short_caches(bf16, lengths, tap):
    """Caches that fit one attention chunk (33 to 64 streams of at most 8 pages): the
    attention covers each stream whole, reading its position and page ids itself, and
    writes the output rows directly -- no work list, no merge launch.  Outputs (and the
    tapped layer's intermediates) against the oracle -- 1e-4 in fp32 -- and the bf16-storage
    emulation; the positions advance."""
    shape = CFG.Shape(n_layers=2)
    m = Model(shape, 2, bf16, seed=17)
    try:
        res, ref = run_decode(m, lengths, 17, tap_layer=tap)
        if bf16:
            assert normwise(res["x"], ref["x"]) <= TOL_LAYER_BF16
            assert normwise(res["x"], ref["x_emul"]) <= TOL_EMUL_BF16
        else:
            assert np.max(np.abs(res["x"] - ref["x"])) <= 1e-4
        if tap is not None:
            rtaps = rec_as_taps(ref["rec"], len(lengths))
            for k in rtaps:
                if bf16:
                    assert normwise(res["taps"][k], rtaps[k]) <= TOL_LAYER_BF16, k
                else:
                    assert np.max(np.abs(res["taps"][k] - rtaps[k])) <= 1e-4, k
        assert res["pos"].tolist() == [n + 1 for n in lengths]
    finally:
        m.close()


@pytest.mark.parametrize("bf16,tap", [(True, None), (True, 1), (False, None)])
def test_decode_kv_heads_not_a_multiple_of_four(bf16, tap):
    """12 query and 6 KV heads (GQA 2), 2 layers: the q_len = 1 work list's waves take
    (segment, KV head) pairs in the mapping for KV-head counts that are not a multiple of
    four; five ragged streams (one at position 0) in segment mode.  Outputs (and the tapped
    layer's intermediates) against the oracle -- fp32: 1e-4 -- and the bf16-storage
    emulation; the positions advance."""
    shape = CFG.Shape(n_layers=2, n_heads=12, n_kv_heads=6)
    m = Model(shape, 2, bf16, seed=31, gains="random")
    try:
        lengths = [300, 1000, 37, 0, 150]
        res, ref = run_decode(m, lengths, 31, tap_layer=tap)
        if bf16:
            assert normwise(res["x"], ref["x"]) <= TOL_LAYER_BF16
            assert normwise(res["x"], ref["x_emul"]) <= TOL_EMUL_BF16
        else:
            assert np.max(np.abs(res["x"] - ref["x"])) <= 1e-4
        if tap is not None:
            rtaps = rec_as_taps(ref["rec"], len(lengths))
            for k in rtaps:
                assert normwise(res["taps"][k], rtaps[k]) <= TOL_LAYER_BF16, k
        assert res["pos"].tolist() == [n + 1 for n in lengths]
    finally:
        m.close()


@pytest.mark.parametrize("tap", [False, True])
def test_decode_direct_negative_position(tap):
    """Direct mode (40 streams, caches of at most 7 pages) with one stream at position -1:
    the step raises the device flag, that stream's attention output is zero and nothing is
    written to the pool for it, and the other streams match the oracle and the emulation."""
    shape = CFG.Shape(n_layers=1)
    m = Model(shape, 1, True, seed=41)
    T = m.T
    try:
        B, bad = 40, 7
        lengths = [(17 * i + 4) % 100 for i in range(B)]
        lengths[bad] = -1
        pt, n_pages = CFG.page_table(41, [max(n, 0) + 1 for n in lengths], extra_pages=1)
        pool = DEV.kv_pool(41, shape, 1, [max(n, 0) for n in lengths], pt, n_pages, True)
        before = pool.clone()
        x_in = gen.fast_normal(41, stream_id(gen.KIND_X_IN, 0), (B, shape.hidden), 1.0)
        x = t_f32(x_in)
        pos = t_i32(lengths)
        if tap:
            T.ttsbb_set_tap_layer(m.ctx, 0)
        T.ttsbb_decode_step(m.ctx, B, x, pos, t_i32(pt), pt.shape[1], pool, n_pages)
        assert T.ttsbb_sync(m.ctx) == T.DEVICE_ERROR
        assert T.ttsbb_sync(m.ctx) == T.OK
        if tap:
            o = read_tap(m, T.TAP_ATTN, B, shape.n_heads * 128)
            assert np.all(o[bad] == 0)
            T.ttsbb_set_tap_layer(m.ctx, -1)
        xg = x.cpu().numpy()
        assert np.all(np.isfinite(xg))
        assert pos.cpu().numpy()[bad] == 0
        sel = [b for b in range(B) if b != bad]
        d = (pool != before).any(dim=-1).nonzero().cpu().numpy()
        assert sorted({int(r[1]) for r in d}) == sorted({int(pt[b, lengths[b] // 16]) for b in sel})
        c_ex, c_em = O.KVCache(1, len(sel)), O.KVCache(1, len(sel))
        for i, b in enumerate(sel):
            if lengths[b]:
                k, v = CFG.kv_prefill(41, shape, 0, b, lengths[b], True)
                c_ex.set(0, i, widen(k), widen(v))
                c_em.set(0, i, widen(k), widen(v))
        lens = [lengths[b] for b in sel]
        out = O.decode_step(x_in[sel], lens, c_ex, m.oracle_layers(), dims_of(shape))
        out_e = E.decode_step(x_in[sel], lens, c_em, m.oracle_layers(), dims_of(shape))
        assert normwise(xg[sel], out) <= TOL_LAYER_BF16
        assert normwise(xg[sel], out_e) <= TOL_EMUL_BF16
    finally:
        m.close()


# ---------------------------------------------------------------------------------------
def run_maskgit(m: Model, n_text, n_frames, n_cb, V, mask_id, n_unmask, seed, tap_layer=None,
                text_vocab=500, masked_frac=0.5):
    T = m.T
    shape = m.shape
    text_h = CFG.table(seed, gen.KIND_TEXT_TABLE, 0, text_vocab, shape.hidden, m.bf16)
    tab_h = CFG.table(seed, gen.KIND_CB_TABLE, 0, n_cb * V, shape.hidden, m.bf16)
    head_h = CFG.table(seed, gen.KIND_HEAD, 0, n_cb * V, shape.hidden, m.bf16)
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
    l_emul = None
    if m.bf16:
        _, _, l_emul = E.maskgit_logits(text_ids, widen(text_h), codes, widen(tab_h), widen(head_h),
                                        m.oracle_layers(), m.oracle_final_norm(), dims_of(shape), V)
    ref = dict(codes_in=codes, rec=rec, lrec=lrec, conf=conf_r, pred=pred_r, x0=x0, head=widen(head_h),
               l_emul=l_emul)
    return res, ref


def check_maskgit(res, ref, n_cb, n_frames, V, mask_id, n_unmask, tol=2e-2, topn_near=BOUNDARY_FRAC):
    rec = ref["rec"]
    assert normwise(res["logits"], rec["logits"]) <= tol
    check_stack("MaskGIT logits", res["logits"], ref["l_emul"], rec["logits"])
    # the stage on the GPU's own head operand: head, pred, conf and picks bit for bit
    _, l_y = check_head_teacher_forced(res["head_in"], ref["head"], res["logits"], res["pred"].T, n_cb, V,
                                       exclude=mask_id)
    check_scores_teacher_forced(res["pred"], res["conf"], res["picked"], l_y, ref["codes_in"], n_cb, V, mask_id,
                                5.0, n_unmask)
    # free-running against the emulation
    g = res["logits"].reshape(n_frames, n_cb, V).transpose(1, 0, 2)
    r = ref["l_emul"].reshape(n_frames, n_cb, V).transpose(1, 0, 2)
    check_argmax_groups(res["pred"], g, r, exclude=mask_id)
    _, conf_e, _ = O.maskgit_scores(ref["l_emul"], ref["codes_in"], n_cb, V, mask_id, 5.0)
    fin = np.isfinite(conf_e)
    assert np.array_equal(np.isfinite(res["conf"]), fin)
    delta = np.max(np.abs(res["logits"] - ref["l_emul"]))
    assert np.max(np.abs(res["conf"][fin] - conf_e[fin])) <= 2 * delta + 1e-5
    check_topn(res["picked"], res["conf"], conf_e, n_unmask, max_near=topn_near)
    # the update writes pred at the picked positions and nothing else
    assert np.array_equal(res["codes"], O.apply_picks(ref["codes_in"], res["pred"], res["picked"]))


def check_attention_teacher_forced(taps, S, H, Hkv):
    """The bidirectional attention on the GPU's own bf16 q, K, V (the taps): against the
    oracle's softmax attention on those values (normwise <= TOL_EMUL_BF16: the kernel's
    bf16 weights and bf16 output are the only differences) and against the emulation of
    the kernel's accumulation (weights rounded relative to its lazily raised references):
    identical for >= 99% of the elements, and no element further from it than one bf16
    unit of the largest output (2^-7 normwise; an element that is small by cancellation may
    move several of its own units)."""
    q = taps["q"].reshape(S, H, 128)
    k = taps["k"].reshape(S, Hkv, 128)
    v = taps["v"].reshape(S, Hkv, 128)
    o = taps["o"].reshape(S, H * 128)
    exact = O.attention_full(q, k, v, causal=False).reshape(S, -1)
    emul = E.r16(E.flash_attention(q, k, v).reshape(S, -1))
    d = normwise(o, exact)
    same = float(np.mean(o == emul))
    d_emul = normwise(o, emul)
    print("attention on the GPU's q/k/v: vs oracle %.2e, vs emulation %.2e, identical to the emulation %.4f"
          % (d, d_emul, same))
    assert d <= TOL_EMUL_BF16
    assert d_emul <= 2.0 ** -7
    assert same >= 0.99


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
        check_attention_teacher_forced(res["taps"], S, 16, 8)
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
        check_attention_teacher_forced(res["taps"], S, 8, 8)
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
    lc_e, lu_e = cfg_emulation(m, text_ids, text_h, tab_h, head_h, codes, n_target, V)
    return res, dict(codes_in=codes, rec=rec, inputs=(text_ids, text_h, tab_h, head_h, codes), lc_e=lc_e, lu_e=lu_e)


def cfg_emulation(m, text_ids, text_h, tab_h, head_h, codes, n_target, V):
    """The bf16-storage emulation of a guided step's two passes: the conditional logits
    on the window's rows, and the unconditional logits of the window's frames alone."""
    w0 = codes.shape[1] - n_target
    n_text = len(text_ids)
    dims = dims_of(m.shape)
    _, _, lc = E.maskgit_logits(text_ids, widen(text_h), codes, widen(tab_h), widen(head_h), m.oracle_layers(),
                                m.oracle_final_norm(), dims, V)
    _, _, lu = E.maskgit_logits(np.zeros(0, np.int32), widen(text_h), codes[:, w0:], widen(tab_h), widen(head_h),
                                m.oracle_layers(), m.oracle_final_norm(), dims, V)
    return lc[w0:], lu


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
        assert normwise(res["logits_c"], ref["lc_e"]) <= TOL_EMUL_BF16
        assert normwise(res["logits_u"], ref["lu_e"]) <= TOL_EMUL_BF16
        g_gpu = O.cfg_logits(res["logits_c"], res["logits_u"], scale)
        g_emu = O.cfg_logits(ref["lc_e"], ref["lu_e"], scale)
        gv = g_gpu.reshape(n_target, n_cb, V).transpose(1, 0, 2)
        rv = g_emu.reshape(n_target, n_cb, V).transpose(1, 0, 2)
        check_argmax_groups(res["pred"], gv, rv, exclude=mask)
        w0 = n_frames - n_target
        _, conf_e, _ = O.maskgit_scores(g_emu, ref["codes_in"][:, w0:], n_cb, V, mask, 5.0)
        fin = np.isfinite(conf_e)
        assert np.array_equal(np.isfinite(res["conf"]), fin)
        assert np.array_equal(np.isfinite(rec["conf"]), fin)
        delta = np.max(np.abs(g_gpu - g_emu))
        assert np.max(np.abs(res["conf"][fin] - conf_e[fin])) <= 2 * delta + 1e-4
        check_topn(res["picked"], res["conf"], conf_e, n_unmask)
        # K8 / K9 on the GPU's own guided logits: choices and picks bit for bit
        check_argmax_groups(res["pred"], gv, gv, exclude=mask)
        assert np.array_equal(np.asarray(res["picked"]), O.select_top(res["conf"].reshape(-1), n_unmask))
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
        lu_gpu = read_tap(m, T.TAP_LOGITS_U, n_target, n_cb * V) if cfg_scale != 0 else None
        guided_gpu = O.cfg_logits(lc, lu_gpu, cfg_scale) if cfg_scale != 0 else lc
        T.ttsbb_set_tap_layer(m.ctx, -1)
        res_codes, res_pred, res_conf = codes_d.cpu().numpy(), pred.cpu().numpy(), conf.cpu().numpy()
        res_picked = picked.cpu().numpy()
        rec = {}
        O.maskgit_step(text_ids, widen(text_h), codes, n_target, widen(tab_h), widen(head_h), m.oracle_layers(),
                       m.oracle_final_norm(), dims_of(shape), V, mask, 5.0, n_unmask, cfg_scale, class_temp,
                       pos_temp, ratio, u_class.astype(np.float64), u_pos.astype(np.float64), record=rec)
        # each pass against its references (the guided logits follow by linearity)
        lc_e, lu_e = cfg_emulation(m, text_ids, text_h, tab_h, head_h, codes, n_target, V)
        assert normwise(lc, rec["logits_c"]) <= TOL_LAYER_BF16
        assert normwise(lc, lc_e) <= TOL_EMUL_BF16
        if cfg_scale != 0:
            assert normwise(lu_gpu, rec["logits_u"]) <= TOL_LAYER_BF16
            assert normwise(lu_gpu, lu_e) <= TOL_EMUL_BF16
        ex1, ex2 = check_sampler(res_pred, res_conf, guided_gpu, rec["guided"], win, n_cb, V, mask, 5.0,
                                 class_temp, pos_temp, ratio, u_class.astype(np.float64),
                                 u_pos.astype(np.float64))
        # explained exceptions stay rare (fp32 vs fp64 ties; bf16 logit error at the edges)
        assert ex1 <= 2 and ex2 <= max(3, n_cb * n_target // 20), (ex1, ex2)
        # picks: exactly the top-n of the GPU's own scores (K9 on its input), and against
        # the scores the sampler's fp64 emulation gives on the emulated guided logits (the
        # uniforms are the same; boundary near ties capped)
        assert np.array_equal(res_picked, O.select_top(res_conf.reshape(-1), n_unmask))
        g_emu = O.cfg_logits(lc_e, lu_e, cfg_scale) if cfg_scale != 0 else lc_e
        _, conf_emu, _ = O.sample_scores(g_emu, win, n_cb, V, mask, 5.0, class_temp, pos_temp, ratio,
                                         u_class.astype(np.float64), u_pos.astype(np.float64))
        same_choice = res_pred == O.sample_scores(g_emu, win, n_cb, V, mask, 5.0, class_temp, pos_temp, ratio,
                                                  u_class.astype(np.float64), u_pos.astype(np.float64))[0]
        if same_choice.all():
            check_topn(res_picked, res_conf, conf_emu, n_unmask, max_near=0.1)
        np.testing.assert_array_equal(res_codes[:, :w0], codes[:, :w0])
        np.testing.assert_array_equal(res_codes[:, w0:], O.apply_picks(win, res_pred, res_picked))
    finally:
        m.close()


# ---------------------------------------------------------------------------------------
# Codec RVQ decode
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("n_frames,n_q,cb,dim,out_dim", [(750, 8, 1024, 64, 1024), (37, 3, 100, 48, 200),
                                                         (65, 9, 17, 8, 33), (1, 1, 5, 130, 7)])
def test_rvq_decode(n_frames, n_q, cb, dim, out_dim):
    """fp32 against the oracle to 1e-4 max-abs (the quantizer accuracy the ncnn port reports
    against PyTorch); the first shape is the 8 x 1024 x 64 -> 1024 quantizer of the
    OmniVoice codec over 30 s of frames.  The next two take the matrix-core kernel with
    ragged 32 x 32 tiles, fewer codebooks than its four waves, and a codebook count that is
    not a multiple of four; the last (a dimension that is not a multiple of 8) the
    vector kernel."""
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


def test_rvq_decode_unaligned_tables_take_the_vector_kernel():
    """Tables that are not 16-byte aligned (views one float into their buffers) cannot be
    read with the matrix-core kernel's 16-byte loads: the vector kernel runs them, with
    the same result to the fp32 bound."""
    m = Model(CFG.Shape(n_layers=1), 0, False, seed=13)
    try:
        T = m.T
        n_frames, n_q, cb, dim, out_dim = 70, 4, 50, 32, 96
        seed = 14
        emb = gen.normal_f32(seed, stream_id(gen.KIND_CB_TABLE, 3), (n_q, cb, dim), 1.0)
        w = gen.normal_f32(seed, stream_id(gen.KIND_HEAD, 3), (n_q, out_dim, dim), 0.05)
        b = gen.normal_f32(seed, stream_id(gen.KIND_FINAL_NORM, 3), (n_q, out_dim), 0.1)
        codes = gen.uniform_int(seed, stream_id(gen.KIND_CODES, 3), (n_q, n_frames), cb)
        emb_buf = torch().zeros(emb.size + 1, dtype=torch().float32, device="cuda")
        emb_buf[1:] = torch().from_numpy(emb.reshape(-1)).cuda()
        w_buf = torch().zeros(w.size + 1, dtype=torch().float32, device="cuda")
        w_buf[1:] = torch().from_numpy(w.reshape(-1)).cuda()
        emb_v, w_v = emb_buf[1:], w_buf[1:]
        assert emb_v.data_ptr() % 16 != 0 and w_v.data_ptr() % 16 != 0
        out = torch().empty((n_frames, out_dim), dtype=torch().float32, device="cuda")
        T.ttsbb_rvq_decode(m.ctx, n_frames, n_q, cb, dim, out_dim, t_i32(codes), emb_v, w_v, t_f32(b), out)
        assert T.ttsbb_sync(m.ctx) == T.OK
        ref = O.rvq_decode(codes, emb, w, b)
        assert np.max(np.abs(out.cpu().numpy() - ref)) <= 1e-4
    finally:
        m.close()


# ---------------------------------------------------------------------------------------
# Causal prefill of one stream into its paged cache
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("p0,S", [(0, 5), (21, 37), (300, 64), (0, 100), (37, 130), (0, 200), (500, 512),
                                  (2085, 70)])
def test_prefill_bf16(p0, S):
    """bf16, 2 layers: the prompt's final residual stream, the K/V it leaves in the pool at
    positions p0..p0+S-1, the advanced cache length and the last token's head choice,
    against the oracle's prefill (which the oracle pins equal to token-by-token decode).
    Up to 64 tokens the attention is the decode kernel's, token by token; beyond, the
    causal flash kernel over the pool's positions 0..p0+S-1 (query tiles ending below,
    at and past a 32-key block, a prefix that is not block-aligned), whose dense K / V^T
    rows the RoPE kernel writes: the prompt's own, and the cached prefix copied from the
    pool by extra workgroups (2085 positions: 33 groups of 64 over 16 workgroups per KV
    head, so some take three); each is held to the emulation of its own bf16 storage."""
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
        # the emulation of the path the prefill runs on: token by token (causal, so the same
        # values as a prefill) with the decode kernels' bf16 storage, or the causal flash
        # kernel's
        c16 = O.KVCache(2, 1)
        for l in range(2):
            if p0:
                k, v = CFG.kv_prefill(seed, shape, l, 0, p0, True)
                c16.set(l, 0, widen(k), widen(v))
        if S > 64:
            xe_all = E.prefill(x_in, p0, c16, 0, m.oracle_layers(), dims_of(shape))
            print("flash prefill vs emulation %.2e, vs oracle %.2e" % (normwise(x.cpu().numpy(), xe_all),
                                                                       normwise(x.cpu().numpy(), out)))
            assert normwise(x.cpu().numpy(), xe_all) <= TOL_EMUL_BF16
            xe = xe_all[-1:]
        else:
            xe = None
            for i in range(S):
                xe = E.decode_step(x_in[i:i + 1], [p0 + i], c16, m.oracle_layers(), dims_of(shape))
        assert normwise(x.cpu().numpy()[-1:], xe) <= TOL_EMUL_BF16
        _, lg_emu = E.head_logits(xe, m.oracle_final_norm(), widen(head_h), shape.eps)
        check_argmax_groups(am.cpu().numpy()[None], lg_gpu.reshape(1, G, V), lg_emu.reshape(1, G, V))
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


# ---------------------------------------------------------------------------------------
# The MaskGIT workload's shape with one layer: the whole pass, and the attention on the
# GPU's own q / K / V
# ---------------------------------------------------------------------------------------
def test_maskgit_workload_shape_one_layer():
    """S = 950 (200 text tokens + 750 frames), 8 codebooks of 1025 classes, one layer:
    logits against the oracle and the emulation, head / scores / picks bit for bit on the
    GPU's head operand, and the bidirectional attention on the GPU's own q, K, V."""
    w = CFG.c4()
    m = Model(w.shape, 1, True, seed=w.seed)
    try:
        res, ref = run_maskgit(m, 200, 750, 8, 1025, 1024, 4, w.seed, tap_layer=0)
        check_maskgit(res, ref, 8, 750, 1025, 1024, 4)
        check_attention_teacher_forced(res["taps"], 950, 16, 8)
    finally:
        m.close()


# ---------------------------------------------------------------------------------------
# fp32 contexts: every MaskGIT step in fp32 (the reference mode), against the oracle at
# the fp32 bound
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("n_text,n_frames,n_heads,n_kv", [(13, 57, 16, 8), (70, 130, 16, 8), (5, 60, 8, 8)])
def test_maskgit_fp32_layer(n_text, n_frames, n_heads, n_kv):
    """fp32, one bidirectional layer: every tap (q, K, V after the head norms and RoPE,
    the attention output, both residual updates, the SwiGLU output) and the logits within
    1e-4 of the oracle; pred exactly the oracle's argmax except at near ties; conf and the
    picks as the oracle scores the GPU's own head operand."""
    shape = CFG.Shape(n_layers=1, n_heads=n_heads, n_kv_heads=n_kv)
    m = Model(shape, 1, False, seed=51, gains="random")
    try:
        n_cb, V, mask, n_unmask = 3, 129, 128, 50
        res, ref = run_maskgit(m, n_text, n_frames, n_cb, V, mask, n_unmask, 51, tap_layer=0)
        S = n_text + n_frames
        lrec = ref["lrec"]
        for k in ("q", "k", "v", "o", "x1", "m", "x2"):
            d = float(np.max(np.abs(res["taps"][k] - lrec[k].reshape(S, -1))))
            print("fp32 %s: max |d| %.2e" % (k, d))
            assert d <= 1e-4, k
        assert float(np.max(np.abs(res["logits"] - ref["rec"]["logits"]))) <= 1e-4
        _, l_y = check_head_teacher_forced(res["head_in"], ref["head"], res["logits"], res["pred"].T, n_cb, V,
                                          exclude=mask)
        check_scores_teacher_forced(res["pred"], res["conf"], res["picked"], l_y, ref["codes_in"], n_cb, V, mask,
                                    5.0, n_unmask)
        g = res["logits"].reshape(n_frames, n_cb, V).transpose(1, 0, 2)
        r = ref["rec"]["logits"].reshape(n_frames, n_cb, V).transpose(1, 0, 2)
        check_argmax_groups(res["pred"], g, r, exclude=mask)
        fin = np.isfinite(ref["conf"])
        assert np.array_equal(np.isfinite(res["conf"]), fin)
        assert float(np.max(np.abs(res["conf"][fin] - ref["conf"][fin]))) <= 2e-4
        check_topn(res["picked"], res["conf"], ref["conf"], n_unmask)
    finally:
        m.close()


def test_maskgit_fp32_guided_two_sequences():
    """fp32 guided step: the two prompts batched as two sequences through the fp32
    attention kernel give the oracle's logits of both passes (1e-4), its guided scores
    and its picks."""
    shape = CFG.Shape(n_layers=1)
    m = Model(shape, 1, False, seed=53, gains="random")
    T = m.T
    try:
        n_text, n_frames, n_target, n_cb, V, mask, n_unmask, scale = 9, 70, 40, 2, 65, 64, 20, 2.0
        seed = 53
        text_h = CFG.table(seed, gen.KIND_TEXT_TABLE, 0, 100, shape.hidden, False)
        tab_h = CFG.table(seed, gen.KIND_CB_TABLE, 0, n_cb * V, shape.hidden, False)
        head_h = CFG.table(seed, gen.KIND_HEAD, 0, n_cb * V, shape.hidden, False)
        text_ids = gen.uniform_int(seed, stream_id(gen.KIND_TEXT_IDS, 0), (n_text,), 100)
        codes = gen.uniform_int(seed, stream_id(gen.KIND_CODES, 0), (n_cb, n_frames), V - 1)
        codes[:, n_frames - n_target::2] = mask
        cd = t_i32(codes)
        pred = torch().empty((n_cb, n_target), dtype=torch().int32, device="cuda")
        conf = torch().empty((n_cb, n_target), dtype=torch().float32, device="cuda")
        picked = torch().empty(n_unmask, dtype=torch().int32, device="cuda")
        T.ttsbb_set_tap_layer(m.ctx, 0)
        T.ttsbb_maskgit_pass_cfg(m.ctx, n_text, t_i32(text_ids), DEV.host_to_device(text_h), 100, n_frames,
                                 n_target, n_cb, V, mask, DEV.host_to_device(tab_h), DEV.host_to_device(head_h), cd,
                                 n_unmask, 5.0, scale, pred, conf, picked)
        assert T.ttsbb_sync(m.ctx) == T.OK
        lg_c = read_tap(m, T.TAP_LOGITS, n_target, n_cb * V)
        lg_u = read_tap(m, T.TAP_LOGITS_U, n_target, n_cb * V)
        T.ttsbb_set_tap_layer(m.ctx, -1)
        layers, fn, dims = m.oracle_layers(), m.oracle_final_norm(), dims_of(shape)
        w0 = n_frames - n_target
        f64 = lambda a: np.asarray(a, np.float64)
        x = O.hybrid_embed(text_ids, f64(text_h), codes, f64(tab_h), V)
        xc = O.backbone_full(x, layers, dims, causal=False)
        _, lc = O.head_logits(xc[n_text + w0:], fn, f64(head_h), dims.eps)
        xu = O.hybrid_embed(np.zeros(0, np.int64), f64(text_h), codes[:, w0:], f64(tab_h), V)
        xu = O.backbone_full(xu, layers, dims, causal=False)
        _, lu = O.head_logits(xu, fn, f64(head_h), dims.eps)
        assert float(np.max(np.abs(lg_c - lc))) <= 1e-4
        assert float(np.max(np.abs(lg_u - lu))) <= 1e-4
        gl = lc + scale * (lc - lu)
        _, conf_r, _ = O.maskgit_scores(gl, codes[:, w0:], n_cb, V, mask, 5.0)
        fin = np.isfinite(conf_r)
        c = conf.cpu().numpy()
        assert np.array_equal(np.isfinite(c), fin)
        assert float(np.max(np.abs(c[fin] - conf_r[fin]))) <= 1e-3
        check_topn(picked.cpu().numpy(), c, conf_r, n_unmask)
    finally:
        m.close()


# ---------------------------------------------------------------------------------------
# The fused head (windows of more than 64 frames, codebooks of >= 128 classes): scores
# from the head product's per-tile statistics, logits never stored
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("n_frames,n_cb,V,mask", [(65, 3, 128, 5), (200, 2, 129, 0), (130, 4, 300, 299),
                                                  (257, 1, 1025, 1024), (100, 8, 1025, 512)])
def test_maskgit_fused_head_scores(n_frames, n_cb, V, mask):
    """Codebooks exactly one 128-column tile wide, one column over (a tile holding two
    codebooks at every boundary), several tiles per codebook with a ragged last one, the
    mask class first, last and inside; ragged 128-row tiles.  pred is the argmax of the
    GPU's own (tapped) logits bit for bit, and pred, conf and the picks hold on the
    oracle's logits of the GPU's head operand.  (With no layers the class distributions
    are nearly uniform, so the best scores of all frames lie within the GPU-to-emulation
    distance of each other: the boundary count of the free-running pick check is not
    capped; the teacher-forced check pins the picks exactly.)"""
    m = Model(CFG.Shape(n_layers=0), 0, True, seed=41, gains="random")
    try:
        n = max(1, n_cb * n_frames // 3)
        res, ref = run_maskgit(m, 7, n_frames, n_cb, V, mask, n, 41)
        check_maskgit(res, ref, n_cb, n_frames, V, mask, n, tol=1e-2, topn_near=None)
    finally:
        m.close()


@pytest.mark.parametrize("mask", [0, 200])
def test_maskgit_fused_head_ties_and_nonfinite(mask):
    """Codebook 0: every class has the same head row, so all its logits are equal: the
    choice is the lowest class that is not the mask (the tie crosses lanes and tiles) and
    the score is -log(V) exactly up to fp32 rounding.  Codebook 1: NaN head rows: the
    lowest non-mask class, score -inf, the device flag.  Codebook 2: ordinary."""
    m = Model(CFG.Shape(n_layers=0), 0, True, seed=43)
    T = m.T
    try:
        n_frames, n_cb, V, n = 90, 3, 260, 40
        tab_h = CFG.table(43, gen.KIND_CB_TABLE, 0, n_cb * V, 1024, True)
        head_h = CFG.table(43, gen.KIND_HEAD, 0, n_cb * V, 1024, True)
        head_h[:V] = head_h[3]
        head_h[V:2 * V] = 0x7FC0  # bf16 quiet NaN
        codes = gen.uniform_int(43, stream_id(gen.KIND_CODES, 0), (n_cb, n_frames), V - 1)
        codes[codes == mask] = (mask + 1) % V
        codes[:, ::2] = mask
        cd = t_i32(codes)
        pred = torch().empty((n_cb, n_frames), dtype=torch().int32, device="cuda")
        conf = torch().empty((n_cb, n_frames), dtype=torch().float32, device="cuda")
        picked = torch().empty(n, dtype=torch().int32, device="cuda")
        T.ttsbb_maskgit_pass(m.ctx, 0, None, None, 0, n_frames, n_cb, V, mask, DEV.host_to_device(tab_h),
                             DEV.host_to_device(head_h), cd, n, 0.0, pred, conf, picked)
        assert T.ttsbb_sync(m.ctx) == T.DEVICE_ERROR
        assert T.ttsbb_sync(m.ctx) == T.OK
        p, c, pk = pred.cpu().numpy(), conf.cpu().numpy(), picked.cpu().numpy()
        low = 1 if mask == 0 else 0
        assert np.all(p[0] == low) and np.all(p[1] == low)
        masked0 = codes[0] == mask
        assert np.all(np.abs(c[0][masked0] + np.log(V)) <= 1e-5)
        assert np.all(c[0][~masked0] == -np.inf) and np.all(c[1] == -np.inf)
        assert np.array_equal(np.isfinite(c[2]), codes[2] == mask)
        assert np.array_equal(pk, O.select_top(c.reshape(-1), n))
        assert np.array_equal(cd.cpu().numpy(), O.apply_picks(codes, p, pk))
    finally:
        m.close()


# ---------------------------------------------------------------------------------------
# Invalid inputs met on the device
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("tap", [False, True])
def test_decode_negative_position_is_flagged_and_isolated(tap):
    """A stream whose position is negative gets no attention work: the step raises the
    device flag, the chunk merge gives that stream a zero attention output without
    reading any partial, every output stays finite, nothing is written to the pool for it,
    and the other streams match the oracle and the emulation."""
    shape = CFG.Shape(n_layers=1)
    m = Model(shape, 1, True, seed=31)
    T = m.T
    try:
        lengths = [40, -1, 17]
        pt, n_pages = CFG.page_table(31, [41, 1, 18], extra_pages=1)
        pool = DEV.kv_pool(31, shape, 1, [40, 0, 17], pt, n_pages, True)
        before = pool.clone()
        x_in = gen.fast_normal(31, stream_id(gen.KIND_X_IN, 0), (3, shape.hidden), 1.0)
        x = t_f32(x_in)
        pos = t_i32(lengths)
        if tap:
            T.ttsbb_set_tap_layer(m.ctx, 0)
        T.ttsbb_decode_step(m.ctx, 3, x, pos, t_i32(pt), pt.shape[1], pool, n_pages)
        assert T.ttsbb_sync(m.ctx) == T.DEVICE_ERROR
        assert T.ttsbb_sync(m.ctx) == T.OK
        if tap:
            o = read_tap(m, T.TAP_ATTN, 3, shape.n_heads * 128)
            assert np.all(o[1] == 0)
            T.ttsbb_set_tap_layer(m.ctx, -1)
        xg = x.cpu().numpy()
        assert np.all(np.isfinite(xg))
        assert pos.cpu().numpy().tolist() == [41, 0, 18]
        # only the two valid streams' slots changed
        d = (pool != before).any(dim=-1).nonzero().cpu().numpy()
        assert sorted({int(r[1]) for r in d}) == sorted({int(pt[0, 40 // 16]), int(pt[2, 17 // 16])})
        sel = [0, 2]
        c_ex, c_em = O.KVCache(1, 2), O.KVCache(1, 2)
        for i, b in enumerate(sel):
            k, v = CFG.kv_prefill(31, shape, 0, b, lengths[b], True)
            c_ex.set(0, i, widen(k), widen(v))
            c_em.set(0, i, widen(k), widen(v))
        out = O.decode_step(x_in[sel], [40, 17], c_ex, m.oracle_layers(), dims_of(shape))
        out_e = E.decode_step(x_in[sel], [40, 17], c_em, m.oracle_layers(), dims_of(shape))
        assert normwise(xg[sel], out) <= TOL_LAYER_BF16
        assert normwise(xg[sel], out_e) <= TOL_EMUL_BF16
    finally:
        m.close()


def test_nonfinite_head_groups_raise_flag():
    """A head group without an order: decode, a group whose head rows are NaN gets class 0
    and raises the flag while the other groups keep the argmax of their own logits;
    MaskGIT, a codebook whose head rows are NaN predicts the lowest non-mask class, scores
    -inf (so it is never unmasked) and raises the flag, while the other codebook is scored
    and selected as usual."""
    shape = CFG.Shape(n_layers=1)
    m = Model(shape, 1, True, seed=37)
    T = m.T
    try:
        G, V = 3, 37
        head_h = CFG.table(37, gen.KIND_HEAD, 0, G * V, shape.hidden, True)
        head_h[V:2 * V] = 0x7FC0  # bf16 quiet NaN
        lengths = [5, 20]
        pt, n_pages = CFG.page_table(37, [6, 21])
        pool = DEV.kv_pool(37, shape, 1, lengths, pt, n_pages, True)
        x = t_f32(gen.fast_normal(37, stream_id(gen.KIND_X_IN, 0), (2, shape.hidden), 1.0))
        am = torch().empty((2, G), dtype=torch().int32, device="cuda")
        lg = torch().empty((2, G * V), dtype=torch().float32, device="cuda")
        T.ttsbb_decode_step(m.ctx, 2, x, t_i32(lengths), t_i32(pt), pt.shape[1], pool, n_pages,
                            DEV.host_to_device(head_h), G, V, am, lg)
        assert T.ttsbb_sync(m.ctx) == T.DEVICE_ERROR
        assert T.ttsbb_sync(m.ctx) == T.OK
        a, l = am.cpu().numpy(), lg.cpu().numpy().reshape(2, G, V)
        assert np.all(np.isnan(l[:, 1])) and np.all(a[:, 1] == 0)
        assert np.array_equal(a[:, [0, 2]], np.argmax(l[:, [0, 2]], axis=-1))
    finally:
        m.close()
    m = Model(CFG.Shape(n_layers=0), 0, True, seed=37)
    T = m.T
    try:
        n_frames, n_cb, V, mask, n = 30, 2, 17, 16, 12
        tab_h = CFG.table(37, gen.KIND_CB_TABLE, 0, n_cb * V, 1024, True)
        head_h = CFG.table(37, gen.KIND_HEAD, 0, n_cb * V, 1024, True)
        head_h[V:2 * V] = 0x7FC0
        codes = gen.uniform_int(37, stream_id(gen.KIND_CODES, 0), (n_cb, n_frames), V - 1)
        codes[:, ::2] = mask
        cd = t_i32(codes)
        pred = torch().empty((n_cb, n_frames), dtype=torch().int32, device="cuda")
        conf = torch().empty((n_cb, n_frames), dtype=torch().float32, device="cuda")
        picked = torch().empty(n, dtype=torch().int32, device="cuda")
        T.ttsbb_maskgit_pass(m.ctx, 0, None, None, 0, n_frames, n_cb, V, mask, DEV.host_to_device(tab_h),
                             DEV.host_to_device(head_h), cd, n, 5.0, pred, conf, picked)
        assert T.ttsbb_sync(m.ctx) == T.DEVICE_ERROR
        assert T.ttsbb_sync(m.ctx) == T.OK
        p, c, pk = pred.cpu().numpy(), conf.cpu().numpy(), picked.cpu().numpy()
        assert np.all(p[1] == 0) and np.all(c[1] == -np.inf)
        assert np.array_equal(np.isfinite(c[0]), codes[0] == mask)
        assert np.array_equal(pk, O.select_top(c.reshape(-1), n))
        assert np.all((pk >= 0) & (pk < n_frames))  # codebook 0 only (15 masked >= 12 picks)
        assert np.array_equal(cd.cpu().numpy(), O.apply_picks(codes, p, pk))
    finally:
        m.close()


# ---------------------------------------------------------------------------------------
# The sampler's Philox4x32-10 stream on the device
# ---------------------------------------------------------------------------------------
def test_philox_known_answers_on_device():
    """The library's generator reproduces the Random123 known-answer vectors of
    Philox4x32-10 (Salmon et al., SC'11) and the host definition over a range of blocks."""
    m = Model(CFG.Shape(n_layers=0), 0, True, seed=1)
    T = m.T
    try:
        kat = [
            ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
            ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
            ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
             (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
        ]
        out = torch().zeros(4, dtype=torch().int32, device="cuda")
        for ctr, key, want in kat:
            T.ttsbb_philox_words(m.ctx, key[0] | (key[1] << 32), ctr[0] | (ctr[1] << 32), ctr[2], ctr[3], 1, out)
            assert T.ttsbb_sync(m.ctx) == T.OK
            assert tuple(int(v) & 0xFFFFFFFF for v in out.cpu().numpy()) == want
        n, b0, seed = 1000, (1 << 32) - 300, 0x1234_5678_9ABC_DEF0
        big = torch().zeros(4 * n, dtype=torch().int32, device="cuda")
        T.ttsbb_philox_words(m.ctx, seed, b0, 1, 0, n, big)
        blk = np.arange(b0, b0 + n, dtype=np.uint64)
        ref = gen.philox4x32_10(blk & np.uint64(0xFFFFFFFF), blk >> np.uint64(32), np.ones(n, np.uint64),
                                np.zeros(n, np.uint64), seed & 0xFFFFFFFF, seed >> 32)
        assert np.array_equal(big.cpu().numpy().view(np.uint32).reshape(n, 4), np.stack(ref, 1).astype(np.uint32))
    finally:
        m.close()


def sampler_uniforms(seed, base, n_cb, n_target, V):
    """The sampler's draws as the header defines them, from the host definition of
    Philox4x32-10 (workload.gen): class noise in domain 1, position noise in domain 2."""
    def draws(dom, n):
        e = np.arange(n, dtype=np.uint64)
        blk = np.uint64(base) + (e >> np.uint64(2))
        o = gen.philox4x32_10(blk & np.uint64(0xFFFFFFFF), blk >> np.uint64(32), np.full(n, dom, np.uint64),
                              np.zeros(n, np.uint64), seed & 0xFFFFFFFF, seed >> 32)
        w = np.stack(o, 1)[np.arange(n), (e & np.uint64(3)).astype(np.int64)]
        return gen.open01_of_words(w)
    return (draws(1, n_cb * n_target * V).reshape(n_cb, n_target, V), draws(2, n_cb * n_target).reshape(n_cb, n_target))


def test_sampler_draws_its_uniforms_on_the_device():
    """A sampled, guided step with no uniform arrays draws them from the Philox stream:
    its choices, scores, picks and codes equal bit for bit those of the same step given
    the arrays computed on the host from the header's definition; the device counter
    advances by ceil(n_cb * n_target * V / 4) per call, so a second call draws the next
    blocks (equal to the step given those arrays)."""
    m = Model(CFG.Shape(n_layers=2), 2, True, seed=12, gains="random")
    T = m.T
    try:
        shape = m.shape
        n_text, n_frames, n_target, n_cb, V, mask, n_unmask, seed, tv = 13, 57, 40, 3, 33, 32, 25, 12, 500
        text_h = CFG.table(seed, gen.KIND_TEXT_TABLE, 0, tv, shape.hidden, True)
        tab_h = CFG.table(seed, gen.KIND_CB_TABLE, 0, n_cb * V, shape.hidden, True)
        head_h = CFG.table(seed, gen.KIND_HEAD, 0, n_cb * V, shape.hidden, True)
        text_ids = gen.uniform_int(seed, stream_id(gen.KIND_TEXT_IDS, 0), (n_text,), tv)
        codes = gen.uniform_int(seed, stream_id(gen.KIND_CODES, 0), (n_cb, n_frames), V - 1)
        codes[:, n_frames - n_target::2] = mask
        dev = [DEV.host_to_device(a) for a in (text_h, tab_h, head_h)]
        rng_seed, base = 0xC0FFEE_1234_5678, 77
        per_call = (n_cb * n_target * V + 3) // 4
        counter = torch().tensor([base], dtype=torch().int64, device="cuda")

        def step(codes_in, u_class=None, u_pos=None):
            cd = t_i32(codes_in)
            out = [torch().empty((n_cb, n_target), dtype=torch().int32, device="cuda"),
                   torch().empty((n_cb, n_target), dtype=torch().float32, device="cuda"),
                   torch().empty(n_unmask, dtype=torch().int32, device="cuda")]
            T.ttsbb_maskgit_step(m.ctx, n_text, t_i32(text_ids), dev[0], tv, n_frames, n_target, n_cb, V, mask,
                                 dev[1], dev[2], cd, n_unmask, 5.0, *out, cfg_scale=2.0, class_temp=0.8,
                                 pos_temp=1.5, top_k_ratio=0.25,
                                 u_class=None if u_class is None else t_f32(u_class),
                                 u_pos=None if u_pos is None else t_f32(u_pos), rng_seed=rng_seed,
                                 rng_counter=counter)
            assert T.ttsbb_sync(m.ctx) == T.OK
            return [cd.cpu().numpy()] + [o.cpu().numpy() for o in out]

        drawn = step(codes)
        assert int(counter.cpu().item()) == base + per_call
        given = step(codes, *sampler_uniforms(rng_seed, base, n_cb, n_target, V))
        assert int(counter.cpu().item()) == base + per_call  # arrays given: nothing drawn
        for a, b in zip(drawn, given):
            assert np.array_equal(a, b)
        drawn2 = step(drawn[0])
        given2 = step(drawn[0], *sampler_uniforms(rng_seed, base + per_call, n_cb, n_target, V))
        for a, b in zip(drawn2, given2):
            assert np.array_equal(a, b)
        assert int(counter.cpu().item()) == base + 2 * per_call
        # a missing counter is an argument error when something must be drawn
        st = T.ttsbb_maskgit_step(m.ctx, n_text, t_i32(text_ids), dev[0], tv, n_frames, n_target, n_cb, V, mask,
                                  dev[1], dev[2], t_i32(codes), n_unmask, 5.0, *[torch().empty(1, device="cuda")] * 3,
                                  class_temp=1.0, check=False)
        assert st == T.INVALID_ARG
    finally:
        m.close()
