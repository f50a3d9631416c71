"""GPU parity at the five workloads' full sizes, in the launch configuration the benchmark
uses, against the oracle on sampled outputs (whole streams, frames, steps) it can compute.

* single layer, fp32, KV 64: every output (1e-4 max-abs);
* 28-layer batch-1 decode, KV 1000, 148 steps: all 148 GPU steps run; the oracle follows
  the first steps exactly (codes are drawn up front, so the trajectory does not depend on
  the argmax); every step's argmax is checked against the GPU's own logits;
* 5-layer code predictor, 256 frames x 15 steps with on-device argmax feedback: the
  oracle follows sampled frames, code by code, until a near tie (if any) lets them part;
* MaskGIT pass, S = 950, 28 layers: logits, predictions, confidences, picks;
* 64-stream paged decode, KV U[200, 4000]: sampled streams through all 28 layers.
"""
import numpy as np
import pytest

from oracle import backbone as O
from workload import configs as CFG
from workload import device as DEV
from workload import gen
from workload.gen import stream_id

from gpu_setup import (TOL_STACK_BF16, Model, check_argmax_groups, check_topn, dims_of, normwise, read_tap,
                       torch, widen)

pytestmark = pytest.mark.gpu


def t_i32(a):
    return torch().from_numpy(np.ascontiguousarray(a, np.int32)).to("cuda")


def t_f32(a):
    return torch().from_numpy(np.ascontiguousarray(a, np.float32)).to("cuda")


def oracle_cache(m, seed, lengths, streams):
    cache = O.KVCache(m.n_layers, len(streams))
    for l in range(m.n_layers):
        for i, b in enumerate(streams):
            if lengths[b]:
                k, v = CFG.kv_prefill(seed, m.shape, l, b, int(lengths[b]), m.bf16)
                cache.set(l, i, widen(k), widen(v))
    return cache


def test_c2_decode_batch1_148_steps():
    w = CFG.c2()
    e = w.extra
    m = Model(w.shape, 28, True, seed=w.seed, max_pos=2048, max_head_cols=4096)
    T = m.T
    try:
        L0, steps, K, V = e["prefill"][0], e["steps"], e["n_cb"], e["cb_vocab"]
        pt, n_pages = CFG.page_table(w.seed, [L0 + steps + 1])
        pool = DEV.kv_pool(w.seed, w.shape, 28, [L0], pt, n_pages, True)
        tables_h = CFG.table(w.seed, gen.KIND_CB_TABLE, 0, K * V, 1024, True)
        head_h = CFG.table(w.seed, gen.KIND_HEAD, 0, e["head_vocab"], 1024, True)
        tables, head = DEV.host_to_device(tables_h), DEV.host_to_device(head_h)
        codes = np.stack([gen.uniform_int(w.seed, stream_id(gen.KIND_CODES, s), (1, K), V) for s in range(steps)])
        codes_d = t_i32(codes)
        pos = t_i32([L0])
        pt_d = t_i32(pt)
        x = torch().empty((1, 1024), dtype=torch().float32, device="cuda")
        am = torch().empty((steps, 1), dtype=torch().int32, device="cuda")
        lg = torch().empty((steps, e["head_vocab"]), dtype=torch().float32, device="cuda")
        xs = []
        for s in range(steps):
            T.ttsbb_codebook_embed(m.ctx, 1, K, codes_d[s], tables, V, None, None, None, 0, x)
            T.ttsbb_decode_step(m.ctx, 1, x, pos, pt_d, pt.shape[1], pool, n_pages, head, 1, e["head_vocab"],
                                am[s], lg[s])
            if s < 4:
                xs.append(x.clone())
        assert T.ttsbb_sync(m.ctx) == T.OK
        assert pos.cpu().numpy().tolist() == [L0 + steps]
        am_h, lg_h = am.cpu().numpy(), lg.cpu().numpy()
        assert np.all(np.isfinite(lg_h))
        assert np.array_equal(am_h[:, 0], np.argmax(lg_h, axis=1))  # every step: own-logit argmax
        # oracle: the first 4 steps exactly
        cache = oracle_cache(m, w.seed, [L0], [0])
        for s in range(4):
            xo = O.codebook_embed(codes[s], widen(tables_h), V)
            out = O.decode_step(xo, [L0 + s], cache, m.oracle_layers(), dims_of(w.shape))
            assert normwise(xs[s].cpu().numpy(), out) <= TOL_STACK_BF16, s
            _, lref = O.head_logits(out, m.oracle_final_norm(), widen(head_h), 1e-6)
            assert normwise(lg_h[s:s + 1], lref) <= TOL_STACK_BF16
            check_argmax_groups(am_h[s:s + 1], lg_h[s:s + 1, None, :], lref[:, None, :])
    finally:
        m.close()


def test_c3_code_predictor_256_frames():
    w = CFG.c3()
    e = w.extra
    F, steps, V = e["batch"], e["steps"], e["cb_vocab"]
    m = Model(w.shape, 5, True, seed=w.seed, max_rows=256, max_pos=64, max_head_cols=V)
    T = m.T
    try:
        pt, n_pages = CFG.page_table(w.seed, [16] * F)
        pool = DEV.kv_pool(w.seed, w.shape, 5, [0] * F, pt, n_pages, True)
        tabs_h = [CFG.table(w.seed, gen.KIND_CB_TABLE, s, V, 1024, True) for s in range(steps)]
        heads_h = [CFG.table(w.seed, gen.KIND_HEAD, s, V, 1024, True) for s in range(steps)]
        tabs = [DEV.host_to_device(t) for t in tabs_h]
        heads = [DEV.host_to_device(t) for t in heads_h]
        hidden = gen.fast_normal(w.seed, stream_id(gen.KIND_X_IN, 0), (F, 1024), 1.0)
        c0 = gen.uniform_int(w.seed, stream_id(gen.KIND_CODES, 0), (F,), V)
        pos, pt_d = t_i32([0] * F), t_i32(pt)
        x = t_f32(hidden)
        T.ttsbb_decode_step(m.ctx, F, x, pos, pt_d, 1, pool, n_pages)  # 1-token prefill, output unused
        codes = torch().empty((steps + 1, F, 1), dtype=torch().int32, device="cuda")
        codes[0, :, 0] = t_i32(c0)
        lg = torch().empty((steps, F, V), dtype=torch().float32, device="cuda")
        for s in range(1, steps + 1):  # step s embeds code s-1 with table s-1, head s-1 -> code s
            T.ttsbb_codebook_embed(m.ctx, F, 1, codes[s - 1], tabs[s - 1], V, None, None, None, 0, x)
            T.ttsbb_decode_step(m.ctx, F, x, pos, pt_d, 1, pool, n_pages, heads[s - 1], 1, V, codes[s], lg[s - 1])
        assert T.ttsbb_sync(m.ctx) == T.OK
        codes_h, lg_h = codes.cpu().numpy()[:, :, 0], lg.cpu().numpy()
        assert pos.cpu().numpy().tolist() == [steps + 1] * F
        for s in range(steps):
            assert np.array_equal(codes_h[s + 1], np.argmax(lg_h[s], axis=1))
        # oracle on sampled frames, free-running with its own argmax
        sample = [0, 1, 77, 255]
        dims = dims_of(w.shape)
        cache = O.KVCache(5, len(sample))
        O.decode_step(hidden[sample], [0] * len(sample), cache, m.oracle_layers(), dims)
        prev = c0[sample].astype(np.int64)
        alive = np.ones(len(sample), bool)
        for s in range(1, steps + 1):
            xo = widen(tabs_h[s - 1])[prev]
            out = O.decode_step(xo, [s] * len(sample), cache, m.oracle_layers(), dims)
            _, lref = O.head_logits(out, m.oracle_final_norm(), widen(heads_h[s - 1]), 1e-6)
            g = lg_h[s - 1][sample]
            for i in range(len(sample)):
                if not alive[i]:
                    continue
                assert normwise(g[i], lref[i]) <= TOL_STACK_BF16, (s, i)
                check_argmax_groups(codes_h[s][sample][i:i + 1], g[i:i + 1, None, :], lref[i:i + 1, None, :])
                if codes_h[s][sample][i] != np.argmax(lref[i]):
                    alive[i] = False  # parted at a near tie (checked above); stop following it
            prev = np.where(alive, codes_h[s][sample], np.argmax(lref, axis=1))
        assert alive.sum() >= 2
    finally:
        m.close()


def test_c4_maskgit_full_pass():
    w = CFG.c4()
    e = w.extra
    m = Model(w.shape, 28, True, seed=w.seed)
    T = m.T
    try:
        n_text, n_frames, n_cb, V, mask = e["n_text"], e["n_frames"], e["n_cb"], e["cb_vocab"], e["mask_id"]
        text_d = DEV.table(w.seed, gen.KIND_TEXT_TABLE, 0, e["text_vocab"], 1024, True)
        tab_h = CFG.table(w.seed, gen.KIND_CB_TABLE, 0, n_cb * V, 1024, True)
        head_h = CFG.table(w.seed, gen.KIND_HEAD, 0, n_cb * V, 1024, True)
        text_ids = CFG.maskgit_text_ids(w)
        codes = CFG.maskgit_codes(w)
        n_unmask = T.ttsbb_unmask_schedule(int((codes == mask).sum()), e["n_steps"])[0]
        codes_d = t_i32(codes)
        pred = torch().empty((n_cb, n_frames), dtype=torch().int32, device="cuda")
        conf = torch().empty((n_cb, n_frames), dtype=torch().float32, device="cuda")
        picked = torch().empty(n_unmask, dtype=torch().int32, device="cuda")
        T.ttsbb_set_tap_layer(m.ctx, 27)
        T.ttsbb_maskgit_pass(m.ctx, n_text, t_i32(text_ids), text_d, e["text_vocab"], n_frames, n_cb, V, mask,
                             DEV.host_to_device(tab_h), DEV.host_to_device(head_h), codes_d, n_unmask,
                             e["layer_penalty"], pred, conf, picked)
        assert T.ttsbb_sync(m.ctx) == T.OK
        logits = read_tap(m, T.TAP_LOGITS, n_frames, n_cb * V)
        x_out = read_tap(m, T.TAP_X_OUT, n_text + n_frames, 1024)
        text_tab = CFG.LazyTable(w.seed, gen.KIND_TEXT_TABLE, 0, e["text_vocab"], 1024, True)
        rec = {}
        O.maskgit_pass(text_ids, text_tab, codes, widen(tab_h), widen(head_h), m.oracle_layers(),
                       m.oracle_final_norm(), dims_of(w.shape), V, mask, e["layer_penalty"], n_unmask, record=rec)
        assert normwise(x_out, rec["x"]) <= TOL_STACK_BF16
        assert normwise(logits, rec["logits"]) <= TOL_STACK_BF16
        g = logits.reshape(n_frames, n_cb, V).transpose(1, 0, 2)
        r = rec["logits"].reshape(n_frames, n_cb, V).transpose(1, 0, 2)
        check_argmax_groups(pred.cpu().numpy(), g, r, exclude=mask)
        cg = conf.cpu().numpy()
        fin = np.isfinite(rec["conf"])
        assert np.array_equal(np.isfinite(cg), fin)
        assert np.max(np.abs(cg[fin] - rec["conf"][fin])) <= 2 * np.max(np.abs(logits - rec["logits"])) + 1e-5
        check_topn(picked.cpu().numpy(), cg, rec["conf"], n_unmask)
        assert np.array_equal(codes_d.cpu().numpy(), O.apply_picks(codes, pred.cpu().numpy(), picked.cpu().numpy()))
    finally:
        m.close()


def test_c5_paged_decode_64_streams():
    w = CFG.c5()
    e = w.extra
    m = Model(w.shape, 28, True, seed=w.seed)
    T = m.T
    try:
        B, K, V = e["batch"], e["n_cb"], e["cb_vocab"]
        lengths = CFG.c5_lengths(w)
        pt, n_pages = CFG.page_table(w.seed, [int(n) + 2 for n in lengths])
        pool = DEV.kv_pool(w.seed, w.shape, 28, lengths, pt, n_pages, True)
        tab_h = CFG.table(w.seed, gen.KIND_CB_TABLE, 0, K * V, 1024, True)
        head_h = CFG.table(w.seed, gen.KIND_HEAD, 0, K * V, 1024, True)
        codes = gen.uniform_int(w.seed, stream_id(gen.KIND_CODES, 0), (B, K), V)
        x = torch().empty((B, 1024), dtype=torch().float32, device="cuda")
        am = torch().empty((B, K), dtype=torch().int32, device="cuda")
        lg = torch().empty((B, K * V), dtype=torch().float32, device="cuda")
        pos = t_i32(lengths)
        T.ttsbb_codebook_embed(m.ctx, B, K, t_i32(codes), DEV.host_to_device(tab_h), V, None, None, None, 0, x)
        T.ttsbb_decode_step(m.ctx, B, x, pos, t_i32(pt), pt.shape[1], pool, n_pages, DEV.host_to_device(head_h),
                            K, V, am, lg)
        assert T.ttsbb_sync(m.ctx) == T.OK
        x_h, am_h, lg_h = x.cpu().numpy(), am.cpu().numpy(), lg.cpu().numpy()
        assert pos.cpu().numpy().tolist() == [int(n) + 1 for n in lengths]
        # the longest and the shortest stream, one in between, and the last stream (the
        # last items of the work list)
        sample = [int(np.argmax(lengths)), int(np.argmin(lengths)), 5, len(lengths) - 1]
        cache = oracle_cache(m, w.seed, lengths, sample)
        xo = O.codebook_embed(codes[sample], widen(tab_h), V)
        out = O.decode_step(xo, [int(lengths[b]) for b in sample], cache, m.oracle_layers(), dims_of(w.shape))
        _, lref = O.head_logits(out, m.oracle_final_norm(), widen(head_h), 1e-6)
        assert normwise(x_h[sample], out) <= TOL_STACK_BF16
        assert normwise(lg_h[sample], lref) <= TOL_STACK_BF16
        check_argmax_groups(am_h[sample], lg_h[sample].reshape(-1, K, V), lref.reshape(-1, K, V))
        # every stream: the argmax is that of its own logits
        check_argmax_groups(am_h, lg_h.reshape(B, K, V), lg_h.reshape(B, K, V))
    finally:
        m.close()
