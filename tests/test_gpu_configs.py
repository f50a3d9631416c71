"""GPU parity at the five workloads' full sizes, in the launch configuration the benchmark
uses, against the oracle and the bf16-storage emulation on sampled outputs (whole streams,
frames, steps) they can compute.

* single layer, fp32, KV 64: every output (1e-4 max-abs) -- test_gpu_parity.py;
* 28-layer batch-1 decode, KV 1000, 148 steps: all 148 GPU steps run; the references
  follow the first steps exactly (codes are drawn up front, so the trajectory does not
  depend on the argmax); one more step with the head operand tapped checks the head and
  its argmax bit for bit against the oracle on that operand;
* 5-layer code predictor, 256 frames x 15 steps with on-device argmax feedback: sampled
  frames follow the GPU's own codes (teacher-forced inputs) through the references;
* MaskGIT pass, S = 950, 28 layers: layer output and logits, then prediction, confidence
  and selection on the GPU's own head operand;
* the 32-step MaskGIT generation at S = 950, 8 x 1025 with 2 layers: every step's
  scoring and selection on the GPU's head operand, and the unmask sets of several steps
  against the emulation run on the same codes;
* 64-stream paged decode, KV U[200, 4000]: sampled streams through all 28 layers, and
  one untapped layer for all 64 streams.

Every deep stack is also checked layer by layer: the step is run again with one layer
tapped, and that layer's output on the GPU's own input to it is compared with the oracle's
and the emulation's layer on the same input (check_layer).

Tolerances: see gpu_setup (one layer: TOL_LAYER_BF16 against the oracle, TOL_EMUL_BF16
against the emulation; a free-running stack: bounds from the emulation's own distance to
the oracle).
"""
import numpy as np
import pytest

from oracle import backbone as O
from workload import configs as CFG
from workload import device as DEV
from workload import gen
from workload.gen import stream_id

import bf16_emulation as E
from gpu_setup import (TOL_LAYER_BF16, TOL_EMUL_BF16, Model, check_argmax_groups, check_head_teacher_forced,
                       check_layer, check_scores_teacher_forced, check_stack, check_topn, dims_of, normwise, read_tap,
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


def layer_cache(m, seed, lengths, streams, layer):
    """The prefilled cache of one layer for the given streams (a 1-layer KVCache)."""
    c = O.KVCache(1, len(streams))
    for i, b in enumerate(streams):
        if lengths[b]:
            k, v = CFG.kv_prefill(seed, m.shape, layer, b, int(lengths[b]), m.bf16)
            c.set(0, i, widen(k), widen(v))
    return c


def check_decode_layers(m, name, run_step, layers, seed, lengths, pos, rows):
    """Run the decode step again with each of `layers` tapped (run_step() repeats it from
    the same state) and check that layer on the GPU's own input against the oracle's and
    the emulation's layer over the prefilled cache."""
    T = m.T
    dims = dims_of(m.shape)
    streams = list(range(len(lengths)))
    for l in layers:
        T.ttsbb_set_tap_layer(m.ctx, l)
        run_step()
        assert T.ttsbb_sync(m.ctx) == T.OK
        x_in = read_tap(m, T.TAP_X_IN, rows, m.shape.hidden)
        x_out = read_tap(m, T.TAP_X_OUT, rows, m.shape.hidden)
        L = m.oracle_layers()[l]
        ex = O.decode_layer(x_in, pos, layer_cache(m, seed, lengths, streams, l), 0, L, dims)
        em = E.decode_layer(x_in, pos, layer_cache(m, seed, lengths, streams, l), 0, L, dims)
        check_layer("%s layer %d" % (name, l), x_out, em, ex)
    T.ttsbb_set_tap_layer(m.ctx, -1)


def test_c2_decode_batch1_148_steps():
    w = CFG.c2()
    e = w.extra
    m = Model(w.shape, 28, True, seed=w.seed, max_pos=2048, max_head_cols=4096)
    T = m.T
    try:
        L0, steps, K, V = e["prefill"][0], e["steps"], e["n_cb"], e["cb_vocab"]
        HV = e["head_vocab"]
        pt, n_pages = CFG.page_table(w.seed, [L0 + steps + 2])
        pool = DEV.kv_pool(w.seed, w.shape, 28, [L0], pt, n_pages, True)
        tables_h = CFG.table(w.seed, gen.KIND_CB_TABLE, 0, K * V, 1024, True)
        head_h = CFG.table(w.seed, gen.KIND_HEAD, 0, HV, 1024, True)
        tables, head = DEV.host_to_device(tables_h), DEV.host_to_device(head_h)
        codes = np.stack([gen.uniform_int(w.seed, stream_id(gen.KIND_CODES, s), (1, K), V) for s in range(steps + 1)])
        codes_d = t_i32(codes)
        pos = t_i32([L0])
        pt_d = t_i32(pt)
        x = torch().empty((1, 1024), dtype=torch().float32, device="cuda")
        am = torch().empty((steps + 1, 1), dtype=torch().int32, device="cuda")
        lg = torch().empty((steps + 1, HV), dtype=torch().float32, device="cuda")
        # layer by layer on the first step (run again from the same state each time)
        def first_step():
            pos.fill_(L0)
            T.ttsbb_codebook_embed(m.ctx, 1, K, codes_d[0], tables, V, None, None, None, 0, x)
            T.ttsbb_decode_step(m.ctx, 1, x, pos, pt_d, pt.shape[1], pool, n_pages, head, 1, HV, am[0], lg[0])
        check_decode_layers(m, "C2", first_step, (0, 13, 27), w.seed, [L0], [L0], 1)
        pos.fill_(L0)
        xs = []
        for s in range(steps):
            T.ttsbb_codebook_embed(m.ctx, 1, K, codes_d[s], tables, V, None, None, None, 0, x)
            T.ttsbb_decode_step(m.ctx, 1, x, pos, pt_d, pt.shape[1], pool, n_pages, head, 1, HV, am[s], lg[s])
            if s < 4:
                xs.append(x.clone())
        assert T.ttsbb_sync(m.ctx) == T.OK
        assert pos.cpu().numpy().tolist() == [L0 + steps]
        am_h, lg_h = am.cpu().numpy(), lg.cpu().numpy()
        assert np.all(np.isfinite(lg_h[:steps]))
        assert np.array_equal(am_h[:steps, 0], np.argmax(lg_h[:steps], axis=1))  # every step: own-logit argmax
        # the references: the first 4 steps exactly
        c_exact = oracle_cache(m, w.seed, [L0], [0])
        c_emul = oracle_cache(m, w.seed, [L0], [0])
        dims = dims_of(w.shape)
        for s in range(4):
            xo = O.codebook_embed(codes[s], widen(tables_h), V)
            out = O.decode_step(xo, [L0 + s], c_exact, m.oracle_layers(), dims)
            out_e = E.decode_step(xo, [L0 + s], c_emul, m.oracle_layers(), dims)
            check_stack("C2 step %d x" % s, xs[s].cpu().numpy(), out_e, out)
            _, lref = O.head_logits(out, m.oracle_final_norm(), widen(head_h), 1e-6)
            _, lemu = E.head_logits(out_e, m.oracle_final_norm(), widen(head_h), 1e-6)
            check_stack("C2 step %d logits" % s, lg_h[s:s + 1], lemu, lref)
            check_argmax_groups(am_h[s:s + 1], lg_h[s:s + 1, None, :], lemu[:, None, :], max_near=None)
        # one more step with the head operand tapped: the head and the argmax on it
        T.ttsbb_set_tap_layer(m.ctx, 27)
        T.ttsbb_codebook_embed(m.ctx, 1, K, codes_d[steps], tables, V, None, None, None, 0, x)
        T.ttsbb_decode_step(m.ctx, 1, x, pos, pt_d, pt.shape[1], pool, n_pages, head, 1, HV, am[steps], lg[steps])
        assert T.ttsbb_sync(m.ctx) == T.OK
        y = read_tap(m, T.TAP_HEAD_IN, 1, 1024)
        check_head_teacher_forced(y, widen(head_h), lg[steps:].cpu().numpy(), am[steps:].cpu().numpy(), 1, HV)
        T.ttsbb_set_tap_layer(m.ctx, -1)
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

        def prefill_step():  # the 1-token prefill at position 0, from the same state
            pos.fill_(0)
            x.copy_(t_f32(hidden))
            T.ttsbb_decode_step(m.ctx, F, x, pos, pt_d, 1, pool, n_pages)
        check_decode_layers(m, "C3", prefill_step, (0, 4), w.seed, [0] * F, [0] * F, F)
        prefill_step()  # output unused
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
        # sampled frames through the references, fed the GPU's own codes (its argmax is
        # checked against the emulation at every step, so the inputs are the same)
        sample = [0, 1, 77, 255]
        dims = dims_of(w.shape)
        c_exact, c_emul = O.KVCache(5, len(sample)), O.KVCache(5, len(sample))
        O.decode_step(hidden[sample], [0] * len(sample), c_exact, m.oracle_layers(), dims)
        E.decode_step(hidden[sample], [0] * len(sample), c_emul, m.oracle_layers(), dims)
        for s in range(1, steps + 1):
            xo = widen(tabs_h[s - 1])[codes_h[s - 1][sample]]
            out = O.decode_step(xo, [s] * len(sample), c_exact, m.oracle_layers(), dims)
            out_e = E.decode_step(xo, [s] * len(sample), c_emul, m.oracle_layers(), dims)
            _, lref = O.head_logits(out, m.oracle_final_norm(), widen(heads_h[s - 1]), 1e-6)
            _, lemu = E.head_logits(out_e, m.oracle_final_norm(), widen(heads_h[s - 1]), 1e-6)
            g = lg_h[s - 1][sample]
            check_stack("C3 step %d logits" % s, g, lemu, lref)
            check_argmax_groups(codes_h[s][sample], g[:, None, :], lemu[:, None, :], max_near=None)
    finally:
        m.close()


def maskgit_inputs(w, n_layers=28):
    e = w.extra
    n_cb, V = e["n_cb"], e["cb_vocab"]
    text_d = DEV.table(w.seed, gen.KIND_TEXT_TABLE, 0, e["text_vocab"], 1024, True)
    tab_h = CFG.table(w.seed, gen.KIND_CB_TABLE, 0, n_cb * V, 1024, True)
    head_h = CFG.table(w.seed, gen.KIND_HEAD, 0, n_cb * V, 1024, True)
    text_tab = CFG.LazyTable(w.seed, gen.KIND_TEXT_TABLE, 0, e["text_vocab"], 1024, True)
    return text_d, tab_h, head_h, text_tab, CFG.maskgit_text_ids(w), CFG.maskgit_codes(w)


def test_c4_maskgit_full_pass():
    w = CFG.c4()
    e = w.extra
    m = Model(w.shape, 28, True, seed=w.seed)
    T = m.T
    try:
        n_text, n_frames, n_cb, V, mask = e["n_text"], e["n_frames"], e["n_cb"], e["cb_vocab"], e["mask_id"]
        text_d, tab_h, head_h, text_tab, text_ids, codes = maskgit_inputs(w)
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
        x_in27 = read_tap(m, T.TAP_X_IN, n_text + n_frames, 1024)
        y = read_tap(m, T.TAP_HEAD_IN, n_frames, 1024)
        pred_h, conf_h, picked_h = pred.cpu().numpy(), conf.cpu().numpy(), picked.cpu().numpy()
        # the stage: head, scores and selection on the GPU's own head operand, bit for bit
        _, lref_y = check_head_teacher_forced(y, widen(head_h), logits, pred_h.T, n_cb, V, exclude=mask)
        check_scores_teacher_forced(pred_h, conf_h, picked_h, lref_y, codes, n_cb, V, mask, e["layer_penalty"],
                                    n_unmask)
        assert np.array_equal(codes_d.cpu().numpy(), O.apply_picks(codes, pred_h, picked_h))
        # layer by layer, on the GPU's own input to each checked layer
        for l in (0, 13):
            T.ttsbb_set_tap_layer(m.ctx, l)
            T.ttsbb_maskgit_pass(m.ctx, n_text, t_i32(text_ids), text_d, e["text_vocab"], n_frames, n_cb, V, mask,
                                 DEV.host_to_device(tab_h), DEV.host_to_device(head_h), t_i32(codes), n_unmask,
                                 e["layer_penalty"], pred, conf, picked)
            assert T.ttsbb_sync(m.ctx) == T.OK
            xi = read_tap(m, T.TAP_X_IN, n_text + n_frames, 1024)
            xo = read_tap(m, T.TAP_X_OUT, n_text + n_frames, 1024)
            L = [m.oracle_layers()[l]]
            check_layer("C4 layer %d" % l, xo, E.backbone_full(xi, L, dims_of(w.shape)),
                        O.backbone_full(xi, L, dims_of(w.shape)))
        T.ttsbb_set_tap_layer(m.ctx, -1)
        L = [m.oracle_layers()[27]]
        check_layer("C4 layer 27", x_out, E.backbone_full(x_in27, L, dims_of(w.shape)),
                    O.backbone_full(x_in27, L, dims_of(w.shape)))
        # the whole pass against the references
        x_ex = O.backbone_full(O.hybrid_embed(text_ids, text_tab, codes, widen(tab_h), V), m.oracle_layers(),
                               dims_of(w.shape))
        _, l_ex = O.head_logits(x_ex[n_text:], m.oracle_final_norm(), widen(head_h), 1e-6)
        x_em, _, l_em = E.maskgit_logits(text_ids, text_tab, codes, widen(tab_h), widen(head_h), m.oracle_layers(),
                                         m.oracle_final_norm(), dims_of(w.shape), V)
        check_stack("C4 x", x_out, x_em, x_ex)
        check_stack("C4 logits", logits, l_em, l_ex)
        assert normwise(logits, l_ex) <= TOL_LAYER_BF16
        g = logits.reshape(n_frames, n_cb, V).transpose(1, 0, 2)
        r = l_em.reshape(n_frames, n_cb, V).transpose(1, 0, 2)
        check_argmax_groups(pred_h, g, r, exclude=mask)
        _, conf_em, _ = O.maskgit_scores(l_em, codes, n_cb, V, mask, e["layer_penalty"])
        check_topn(picked_h, conf_h, conf_em, n_unmask)
    finally:
        m.close()


def test_c4_maskgit_32_step_generation_two_layers():
    """The full generation loop at the MaskGIT workload's shape (S = 950, 8 x 1025, 3000
    masked, 32 cosine-schedule steps) with 2 layers: each step's codes feed the next.
    Every step: head, scores and selection bit for bit on the GPU's own head operand (so
    the unmask set is exactly the top-n of the GPU's confidences) and the update applied
    to exactly the picked positions.  Steps 0-3, 8, 16, 24 and 31: the unmask set equals
    the emulation's on the same codes except at logged boundary near ties.  At the end no
    position is masked."""
    w = CFG.c4()
    e = w.extra
    m = Model(w.shape, 2, True, seed=w.seed)
    T = m.T
    try:
        n_text, n_frames, n_cb, V, mask = e["n_text"], e["n_frames"], e["n_cb"], e["cb_vocab"], e["mask_id"]
        text_d, tab_h, head_h, text_tab, text_ids, codes0 = maskgit_inputs(w)
        sched = T.ttsbb_unmask_schedule(int((codes0 == mask).sum()), e["n_steps"])
        assert sched == O.unmask_schedule(int((codes0 == mask).sum()), e["n_steps"])
        codes_d = t_i32(codes0)
        tab_d, head_d, ids_d = DEV.host_to_device(tab_h), DEV.host_to_device(head_h), t_i32(text_ids)
        pred = torch().empty((n_cb, n_frames), dtype=torch().int32, device="cuda")
        conf = torch().empty((n_cb, n_frames), dtype=torch().float32, device="cuda")
        picked = torch().empty(max(sched), dtype=torch().int32, device="cuda")
        T.ttsbb_set_tap_layer(m.ctx, 1)
        dims = dims_of(w.shape)
        near_total = 0
        for step, n in enumerate(sched):
            before = codes_d.cpu().numpy()
            T.ttsbb_maskgit_pass(m.ctx, n_text, ids_d, text_d, e["text_vocab"], n_frames, n_cb, V, mask, tab_d,
                                 head_d, codes_d, n, e["layer_penalty"], pred, conf, picked)
            assert T.ttsbb_sync(m.ctx) == T.OK
            logits = read_tap(m, T.TAP_LOGITS, n_frames, n_cb * V)
            y = read_tap(m, T.TAP_HEAD_IN, n_frames, 1024)
            pred_h, conf_h, picked_h = pred.cpu().numpy(), conf.cpu().numpy(), picked.cpu().numpy()[:n]
            _, lref_y = check_head_teacher_forced(y, widen(head_h), logits, pred_h.T, n_cb, V, exclude=mask)
            check_scores_teacher_forced(pred_h, conf_h, picked_h, lref_y, before, n_cb, V, mask,
                                        e["layer_penalty"], n)
            after = codes_d.cpu().numpy()
            assert np.array_equal(after, O.apply_picks(before, pred_h, picked_h)), step
            assert int((after == mask).sum()) == int((before == mask).sum()) - n, step
            if step in (0, 1, 2, 3, 8, 16, 24, 31):
                _, _, l_em = E.maskgit_logits(text_ids, text_tab, before, widen(tab_h), widen(head_h),
                                              m.oracle_layers(), m.oracle_final_norm(), dims, V)
                x_ex = O.backbone_full(O.hybrid_embed(text_ids, text_tab, before, widen(tab_h), V),
                                       m.oracle_layers(), dims)
                _, l_ex = O.head_logits(x_ex[n_text:], m.oracle_final_norm(), widen(head_h), 1e-6)
                check_stack("C4 2 layers, step %d logits" % step, logits, l_em, l_ex)
                _, conf_em, _ = O.maskgit_scores(l_em, before, n_cb, V, mask, e["layer_penalty"])
                nb = check_topn(picked_h, conf_h, conf_em, n)
                near_total += nb
                print("step %2d: n_unmask %4d, boundary near ties vs emulation %d" % (step, n, nb))
        assert int((codes_d.cpu().numpy() == mask).sum()) == 0
        print("near ties over the checked steps: %d" % near_total)
        T.ttsbb_set_tap_layer(m.ctx, -1)
    finally:
        m.close()


def test_c4_maskgit_fp32_32_steps_two_layers():
    """fp32 context, the MaskGIT workload's shape (S = 950, 8 x 1025, 3000 masked, 32
    cosine-schedule steps) with 2 layers, the GPU's codes feeding each next step.  At every
    step the oracle runs the same step in fp64 on the same codes: the logits agree within
    1e-4, pred equals the oracle's argmax except at near ties, and the unmask set equals
    the oracle's except at boundary near ties (both counted, and bounded).  Whether the
    loop stays identical to the oracle's own free-running loop is reported, not asserted:
    with 6000 groups per step, an fp32 near tie somewhere in 32 steps is expected."""
    w = CFG.c4()
    e = w.extra
    m = Model(w.shape, 2, False, seed=w.seed)
    T = m.T
    try:
        n_text, n_frames, n_cb, V, mask = e["n_text"], e["n_frames"], e["n_cb"], e["cb_vocab"], e["mask_id"]
        pen = e["layer_penalty"]
        text_h = CFG.table(w.seed, gen.KIND_TEXT_TABLE, 0, e["text_vocab"], 1024, False)
        tab_h = CFG.table(w.seed, gen.KIND_CB_TABLE, 0, n_cb * V, 1024, False)
        head_h = CFG.table(w.seed, gen.KIND_HEAD, 0, n_cb * V, 1024, False)
        text_ids, codes0 = CFG.maskgit_text_ids(w), CFG.maskgit_codes(w)
        sched = T.ttsbb_unmask_schedule(int((codes0 == mask).sum()), e["n_steps"])
        codes_d = t_i32(codes0)
        text_d, tab_d, head_d, ids_d = (DEV.host_to_device(text_h), DEV.host_to_device(tab_h),
                                        DEV.host_to_device(head_h), t_i32(text_ids))
        pred = torch().empty((n_cb, n_frames), dtype=torch().int32, device="cuda")
        conf = torch().empty((n_cb, n_frames), dtype=torch().float32, device="cuda")
        picked = torch().empty(max(sched), dtype=torch().int32, device="cuda")
        T.ttsbb_set_tap_layer(m.ctx, 1)
        layers, fn, dims = m.oracle_layers(), m.oracle_final_norm(), dims_of(w.shape)
        f64 = lambda a: np.asarray(a, np.float64)
        codes_free = codes0.copy()
        same_as_free = -1
        near_pred = near_pick = 0
        for step, n in enumerate(sched):
            before = codes_d.cpu().numpy()
            T.ttsbb_maskgit_pass(m.ctx, n_text, ids_d, text_d, e["text_vocab"], n_frames, n_cb, V, mask, tab_d,
                                 head_d, codes_d, n, pen, pred, conf, picked)
            assert T.ttsbb_sync(m.ctx) == T.OK
            logits = read_tap(m, T.TAP_LOGITS, n_frames, n_cb * V)
            pred_h, conf_h, picked_h = pred.cpu().numpy(), conf.cpu().numpy(), picked.cpu().numpy()[:n]
            rec = {}
            _, pred_r, conf_r, _ = O.maskgit_pass(text_ids, f64(text_h), before, f64(tab_h), f64(head_h), layers, fn,
                                                  dims, V, mask, pen, n, record=rec)
            dl = float(np.max(np.abs(logits - rec["logits"])))
            assert dl <= 1e-4, (step, dl)
            g = logits.reshape(n_frames, n_cb, V).transpose(1, 0, 2)
            r = rec["logits"].reshape(n_frames, n_cb, V).transpose(1, 0, 2)
            near_pred += check_argmax_groups(pred_h, g, r, exclude=mask)
            near_pick += check_topn(picked_h, conf_h, conf_r, n)
            after = codes_d.cpu().numpy()
            assert np.array_equal(after, O.apply_picks(before, pred_h, picked_h)), step
            if same_as_free == step - 1:
                codes_free = O.apply_picks(codes_free, pred_r, O.select_top(conf_r.reshape(-1), n))
                if np.array_equal(after, codes_free):
                    same_as_free = step
            print("step %2d: n_unmask %4d, max |dlogit| %.1e" % (step, n, dl))
        assert int((codes_d.cpu().numpy() == mask).sum()) == 0
        print("argmax near ties %d, selection boundary near ties %d; identical to the oracle's free-running "
              "loop through step %d of %d" % (near_pred, near_pick, same_as_free, len(sched) - 1))
        # (check_topn counts the threshold element itself: at least one per step)
        assert near_pred <= len(sched) and near_pick <= 2 * len(sched)
        T.ttsbb_set_tap_layer(m.ctx, -1)
    finally:
        m.close()


def c5_setup(m, w):
    e = w.extra
    B, K, V = e["batch"], e["n_cb"], e["cb_vocab"]
    lengths = CFG.c5_lengths(w)
    pt, n_pages = CFG.page_table(w.seed, [int(n) + 2 for n in lengths])
    pool = DEV.kv_pool(w.seed, w.shape, m.n_layers, lengths, pt, n_pages, True)
    tab_h = CFG.table(w.seed, gen.KIND_CB_TABLE, 0, K * V, 1024, True)
    head_h = CFG.table(w.seed, gen.KIND_HEAD, 0, K * V, 1024, True)
    codes = gen.uniform_int(w.seed, stream_id(gen.KIND_CODES, 0), (B, K), V)
    return B, K, V, lengths, pt, n_pages, pool, tab_h, head_h, codes


def test_c5_paged_decode_64_streams():
    w = CFG.c5()
    m = Model(w.shape, 28, True, seed=w.seed)
    T = m.T
    try:
        B, K, V, lengths, pt, n_pages, pool, tab_h, head_h, codes = c5_setup(m, w)
        x = torch().empty((B, 1024), dtype=torch().float32, device="cuda")
        am = torch().empty((B, K), dtype=torch().int32, device="cuda")
        lg = torch().empty((B, K * V), dtype=torch().float32, device="cuda")
        pos = t_i32(lengths)
        tab_d, head_d, pt_d = DEV.host_to_device(tab_h), DEV.host_to_device(head_h), t_i32(pt)

        def step():
            pos.copy_(t_i32(lengths))
            T.ttsbb_codebook_embed(m.ctx, B, K, t_i32(codes), tab_d, V, None, None, None, 0, x)
            T.ttsbb_decode_step(m.ctx, B, x, pos, pt_d, pt.shape[1], pool, n_pages, head_d, K, V, am, lg)
        check_decode_layers(m, "C5", step, (0, 27), w.seed, lengths, [int(n) for n in lengths], B)
        step()
        assert T.ttsbb_sync(m.ctx) == T.OK
        x_h, am_h, lg_h = x.cpu().numpy(), am.cpu().numpy(), lg.cpu().numpy()
        assert pos.cpu().numpy().tolist() == [int(n) + 1 for n in lengths]
        # the longest and the shortest stream, one in between, and the last stream (the
        # last items of the work list)
        sample = [int(np.argmax(lengths)), int(np.argmin(lengths)), 5, len(lengths) - 1]
        xo = O.codebook_embed(codes[sample], widen(tab_h), V)
        dims = dims_of(w.shape)
        out = O.decode_step(xo, [int(lengths[b]) for b in sample], oracle_cache(m, w.seed, lengths, sample),
                            m.oracle_layers(), dims)
        out_e = E.decode_step(xo, [int(lengths[b]) for b in sample], oracle_cache(m, w.seed, lengths, sample),
                              m.oracle_layers(), dims)
        _, lref = O.head_logits(out, m.oracle_final_norm(), widen(head_h), 1e-6)
        _, lemu = E.head_logits(out_e, m.oracle_final_norm(), widen(head_h), 1e-6)
        check_stack("C5 x", x_h[sample], out_e, out)
        check_stack("C5 logits", lg_h[sample], lemu, lref)
        check_argmax_groups(am_h[sample], lg_h[sample].reshape(-1, K, V), lemu.reshape(-1, K, V), max_near=None)
        # every stream: the argmax is that of its own logits
        check_argmax_groups(am_h, lg_h.reshape(B, K, V), lg_h.reshape(B, K, V))
    finally:
        m.close()


def test_c5_one_layer_all_64_streams():
    """The paged workload's 64 streams through one layer on the production path (fused
    step token, balanced work list, fragment-major operands; nothing tapped), every stream
    against the oracle (the layer bound) and the emulation; then the same step with the
    head operand tapped: head and per-codebook argmax bit for bit on it."""
    w = CFG.c5()
    m = Model(w.shape, 1, True, seed=w.seed)
    T = m.T
    try:
        B, K, V, lengths, pt, n_pages, pool, tab_h, head_h, codes = c5_setup(m, w)
        head_d, tab_d, pt_d = DEV.host_to_device(head_h), DEV.host_to_device(tab_h), t_i32(pt)
        pool0 = pool.clone()
        x = torch().empty((B, 1024), dtype=torch().float32, device="cuda")
        am = torch().empty((B, K), dtype=torch().int32, device="cuda")
        lg = torch().empty((B, K * V), dtype=torch().float32, device="cuda")
        T.ttsbb_codebook_embed(m.ctx, B, K, t_i32(codes), tab_d, V, None, None, None, 0, x)
        x_in = x.cpu().numpy()
        T.ttsbb_decode_step(m.ctx, B, x, t_i32(lengths), pt_d, pt.shape[1], pool, n_pages, head_d, K, V, am, lg)
        assert T.ttsbb_sync(m.ctx) == T.OK
        x_h, am_h, lg_h = x.cpu().numpy(), am.cpu().numpy(), lg.cpu().numpy()
        dims = dims_of(w.shape)
        streams = list(range(B))
        out = O.decode_step(x_in, [int(n) for n in lengths], oracle_cache(m, w.seed, lengths, streams),
                            m.oracle_layers(), dims)
        out_e = E.decode_step(x_in, [int(n) for n in lengths], oracle_cache(m, w.seed, lengths, streams),
                              m.oracle_layers(), dims)
        check_layer("C5 all 64 streams, untapped", x_h, out_e, out)
        _, lemu = E.head_logits(out_e, m.oracle_final_norm(), widen(head_h), 1e-6)
        check_argmax_groups(am_h, lg_h.reshape(B, K, V), lemu.reshape(B, K, V))
        # the same step with the head operand tapped (pool restored: the step rewrites the
        # same slots)
        pool.copy_(pool0)
        x2 = t_f32(x_in)
        T.ttsbb_set_tap_layer(m.ctx, 0)
        T.ttsbb_decode_step(m.ctx, B, x2, t_i32(lengths), pt_d, pt.shape[1], pool, n_pages, head_d, K, V, am, lg)
        assert T.ttsbb_sync(m.ctx) == T.OK
        y = read_tap(m, T.TAP_HEAD_IN, B, 1024)
        T.ttsbb_set_tap_layer(m.ctx, -1)
        # the tapped path (separate step-token kernel) agrees with the fused one up to the
        # bf16 rounding flips that fp32 differences cause (the one-layer emulation bound)
        assert normwise(x2.cpu().numpy(), x_h) <= TOL_EMUL_BF16
        check_head_teacher_forced(y, widen(head_h), lg.cpu().numpy(), am.cpu().numpy(), K, V)
    finally:
        m.close()
