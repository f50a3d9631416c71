#!/usr/bin/env python3
"""Benchmark of the TTS backbone hot path on one MI355X.

Default workload ("c5c4"): one step is
  * one batched decode iteration: 64 streams, 28 layers, bf16, paged KV cache with
    16-token pages and per-stream lengths U[200, 4000] (seed 7): embedding of 8 summed
    codebooks (1025 x 1024 tables) -> 28 layers (q_len = 1) -> final norm -> 8 x 1025
    heads -> argmax; and
  * one MaskGIT pass: 200 text tokens + 750 frames x 8 codebooks (half masked), 28
    bidirectional layers, 8 x 1025 heads, scores, top-n unmasking on a cosine schedule
    (32 steps; codes are restored every 32 passes).
Inputs are seeded synthetic tensors resident in HBM before the timed region.  `value` is
decode tokens/s (64 tokens per step over the decode part of the step); MaskGIT frames/s
and MFMA utilisation, and decode-attention HBM GB/s are reported beside it, with per-kernel
rates: each MaskGIT product and the flash attention in TF/s and against the bf16 MFMA peak,
the decode projections as weight-streaming GB/s, the embeddings in GB/s.

Further figures, each timed on its own after the step: a guided and a guided + sampled
MaskGIT step, one whole 32-step MaskGIT generation, a 200-token causal prefill, the codec
RVQ decode of 750 frames, the 5-layer code predictor, and the
batch-1 decode loop (16 x 2048 codebooks, 3072 head, KV 1000, 148 steps) run eagerly and as
one captured HIP graph.  The single fp32 layer is a parity-test case only.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-graph] [--no-extras]
                    [--copy-calibration MIB]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "decode tokens/s + attn HBM GB/s; MaskGIT frames/s + MFMA util (% peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------
# Setup helpers
# ---------------------------------------------------------------------------------------

def make_ctx(T, torch, shape, n_layers, bf16, seed, max_rows, max_pos, max_head_cols, DEV, CFG):
    dev = [DEV.layer_weights(seed, shape, l, bf16) for l in range(n_layers)]
    fn = DEV.host_to_device(CFG.final_norm(seed, shape))
    cfg = T.ttsbb_default_config()
    cfg.n_layers = n_layers
    cfg.dtype = T.BF16 if bf16 else T.F32
    cfg.max_rows, cfg.max_pos, cfg.max_head_cols = max_rows, max_pos, max_head_cols
    layers = [T.make_layer(*[d[k] for k in ("attn_norm", "q_norm", "k_norm", "ffn_norm", "wq", "wk",
                                             "wv", "wo", "w_gate", "w_up", "w_down")]) for d in dev]
    ctx = T.ttsbb_create(cfg, layers, fn, torch.cuda.current_stream().cuda_stream)
    return ctx, (dev, fn)


class DecodeC5:
    """64-stream paged decode iteration with 8 summed codebooks and 8 x 1025 heads."""

    def __init__(self, T, torch, total_steps):
        from workload import configs as CFG, device as DEV, gen
        self.T, self.torch = T, torch
        w = CFG.c5()
        self.w = w
        e = w.extra
        self.B, self.K, self.V = e["batch"], e["n_cb"], e["cb_vocab"]
        self.lengths = CFG.c5_lengths(w)
        room = [int(n) + total_steps + 1 for n in self.lengths]
        # 13 spare pages beyond the streams' (a 200-token prefill stream of its own)
        self.pt, self.n_pages = CFG.page_table(w.seed, room, extra_pages=13)
        self.ctx, self.keep = make_ctx(T, torch, w.shape, 28, True, w.seed, 1024, 8192, 8200, DEV, CFG)
        self.pool = DEV.kv_pool(w.seed, w.shape, 28, self.lengths, self.pt, self.n_pages, True)
        self.pt_d = torch.from_numpy(self.pt).cuda()
        self.tables = DEV.table(w.seed, gen.KIND_CB_TABLE, 0, self.K * self.V, 1024, True)
        self.heads = DEV.table(w.seed, gen.KIND_HEAD, 0, self.K * self.V, 1024, True)
        codes = np.stack([gen.uniform_int(w.seed, gen.stream_id(gen.KIND_CODES, s), (self.B, self.K), self.V)
                          for s in range(total_steps)])
        self.codes = torch.from_numpy(codes).cuda()
        self.pos = torch.from_numpy(self.lengths.astype(np.int32)).cuda()
        self.x = torch.empty((self.B, 1024), dtype=torch.float32, device="cuda")
        self.am = torch.empty((self.B, self.K), dtype=torch.int32, device="cuda")

    def step(self, s):
        T = self.T
        T.ttsbb_codebook_embed(self.ctx, self.B, self.K, self.codes[s], self.tables, self.V, None, None,
                               None, 0, self.x)
        T.ttsbb_decode_step(self.ctx, self.B, self.x, self.pos, self.pt_d, self.pt.shape[1], self.pool,
                            self.n_pages, self.heads, self.K, self.V, self.am)

    def attn_bytes(self, steps_done_before, n_steps):
        """Algorithmic bytes of one decode-attention launch averaged over the timed steps:
        K and V (bf16) of every earlier cached position once; the step token's raw q, k, v
        (fp32) in and its K, V (bf16) out to the slot (the kernel prepares the token);
        o (bf16) out."""
        L = self.lengths.astype(np.int64)
        mean_len = float(np.mean([(L + s).sum() for s in range(steps_done_before,
                                                               steps_done_before + n_steps)]))
        kv = mean_len * 8 * 128 * 2 * 2
        token = self.B * (16 + 2 * 8) * 128 * 4 + self.B * 8 * 128 * 2 * 2
        return kv + token + self.B * 16 * 128 * 2


class MaskgitC4:
    def __init__(self, T, torch):
        from workload import configs as CFG, device as DEV, gen
        self.T, self.torch = T, torch
        w = CFG.c4()
        e = w.extra
        self.e = e
        # 2048 rows: a guided step runs its two sequences (950 + 750 rows) as one batch
        self.ctx, self.keep = make_ctx(T, torch, w.shape, 28, True, w.seed, 2048, 8192, 8200, DEV, CFG)
        self.text_table = DEV.table(w.seed, gen.KIND_TEXT_TABLE, 0, e["text_vocab"], 1024, True)
        self.tables = DEV.table(w.seed, gen.KIND_CB_TABLE, 0, e["n_cb"] * e["cb_vocab"], 1024, True)
        self.heads = DEV.table(w.seed, gen.KIND_HEAD, 0, e["n_cb"] * e["cb_vocab"], 1024, True)
        self.text_ids = torch.from_numpy(CFG.maskgit_text_ids(w)).cuda()
        self.codes0 = torch.from_numpy(CFG.maskgit_codes(w)).cuda()
        self.codes = self.codes0.clone()
        n_masked = int((CFG.maskgit_codes(w) == e["mask_id"]).sum())
        self.sched = T.ttsbb_unmask_schedule(n_masked, e["n_steps"])
        shp = (e["n_cb"], e["n_frames"])
        self.pred = torch.empty(shp, dtype=torch.int32, device="cuda")
        self.conf = torch.empty(shp, dtype=torch.float32, device="cuda")
        self.picked = torch.empty(max(self.sched), dtype=torch.int32, device="cuda")

    def step(self, s):
        e = self.e
        i = s % e["n_steps"]
        if i == 0:
            self.codes.copy_(self.codes0)
        self.T.ttsbb_maskgit_pass(self.ctx, e["n_text"], self.text_ids, self.text_table, e["text_vocab"],
                                  e["n_frames"], e["n_cb"], e["cb_vocab"], e["mask_id"], self.tables,
                                  self.heads, self.codes, self.sched[i], e["layer_penalty"], self.pred,
                                  self.conf, self.picked)

    def step_cfg(self, s, cfg_scale=2.0):
        """The same step with classifier-free guidance: the conditional prompt (200 text
        tokens + 750 frames) and the 750-frame window alone, guided scores."""
        e = self.e
        i = s % e["n_steps"]
        if i == 0:
            self.codes.copy_(self.codes0)
        self.T.ttsbb_maskgit_pass_cfg(self.ctx, e["n_text"], self.text_ids, self.text_table, e["text_vocab"],
                                      e["n_frames"], e["n_frames"], e["n_cb"], e["cb_vocab"], e["mask_id"],
                                      self.tables, self.heads, self.codes, self.sched[i], e["layer_penalty"],
                                      cfg_scale, self.pred, self.conf, self.picked)

    def step_sampled(self, s, cfg_scale=2.0, class_temp=1.0, pos_temp=1.0):
        """The general step: guidance plus the sampler (top-k ratio 0.1, class and
        position temperatures); the Gumbel uniforms are drawn on the device from the
        library's Philox4x32-10 stream, its counter threaded through the calls."""
        e = self.e
        i = s % e["n_steps"]
        if i == 0:
            self.codes.copy_(self.codes0)
        if not hasattr(self, "rng_counter"):
            self.rng_counter = self.torch.zeros(1, dtype=self.torch.int64, device="cuda")
        self.T.ttsbb_maskgit_step(self.ctx, e["n_text"], self.text_ids, self.text_table, e["text_vocab"],
                                  e["n_frames"], e["n_frames"], e["n_cb"], e["cb_vocab"], e["mask_id"], self.tables,
                                  self.heads, self.codes, self.sched[i], e["layer_penalty"], self.pred, self.conf,
                                  self.picked, cfg_scale=cfg_scale, class_temp=class_temp, pos_temp=pos_temp,
                                  top_k_ratio=0.1, rng_seed=42, rng_counter=self.rng_counter)

    def flops(self):
        """Algorithmic flops of one pass: projections, attention, heads."""
        e = self.e
        S = e["n_text"] + e["n_frames"]
        per_tok_layer = 2 * (1024 * 4096 + 2048 * 1024 + 1024 * 6144 + 3072 * 1024)
        gemm = S * per_tok_layer * 28
        attn = 4 * 16 * 128 * S * S * 28
        head = 2 * e["n_frames"] * 1024 * e["n_cb"] * e["cb_vocab"]
        return gemm, attn, head


# ---------------------------------------------------------------------------------------
# CPU baseline: the oracle, untuned, on a bounded sample of the same workload
# ---------------------------------------------------------------------------------------

def cpu_baseline(n_streams=2, n_steps=24):
    from oracle import backbone as O
    from workload import configs as CFG, gen
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    w = CFG.c5()
    e = w.extra
    shape = w.shape
    t0 = time.perf_counter()
    layers = []
    for l in range(28):
        h = CFG.layer_weights(w.seed, shape, l, True)
        layers.append(O.Layer.from_arrays({k: (gen.bf16_bits_to_f32(v) if v.dtype == np.uint16 else v)
                                           for k, v in h.items()}))
    lengths = CFG.c5_lengths(w)[:n_streams]
    cache = O.KVCache(28, n_streams)
    for l in range(28):
        for b in range(n_streams):
            k, v = CFG.kv_prefill(w.seed, shape, l, b, int(lengths[b]), True)
            cache.set(l, b, gen.bf16_bits_to_f32(k), gen.bf16_bits_to_f32(v))
    table = CFG.LazyTable(w.seed, gen.KIND_CB_TABLE, 0, e["n_cb"] * e["cb_vocab"], 1024, True)
    heads = CFG.LazyTable(w.seed, gen.KIND_HEAD, 0, e["n_cb"] * e["cb_vocab"], 1024, True)
    head_full = heads[np.arange(e["n_cb"] * e["cb_vocab"])]
    codes = [gen.uniform_int(w.seed, gen.stream_id(gen.KIND_CODES, s), (e["batch"], e["n_cb"]), e["cb_vocab"])
             for s in range(n_steps)]
    fn = CFG.final_norm(w.seed, shape).astype(np.float64)
    setup = time.perf_counter() - t0
    t1 = time.perf_counter()
    pos = [int(n) for n in lengths]
    for s in range(n_steps):  # the same steps as the GPU decode: embed, 28 layers, head, argmax
        x = O.codebook_embed(codes[s][:n_streams], table, e["cb_vocab"])
        out = O.decode_step(x, pos, cache, layers, O.Dims())
        _, lg = O.head_logits(out, fn, head_full, 1e-6)
        O.argmax_groups(lg, e["n_cb"], e["cb_vocab"])
        pos = [p + 1 for p in pos]
    dt = time.perf_counter() - t1
    return {"value": n_streams * n_steps / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": host_cpu_model(),
            "sample": "%d of the 64 streams (KV %s) for %d consecutive full 28-layer decode steps "
                      "(embed, layers, head, argmax), fp64 numpy; input generation (%.1f s) excluded"
                      % (n_streams, lengths.tolist(), n_steps, setup),
            "seconds": dt}


def cpu_baseline_maskgit():
    """Oracle time of one full MaskGIT pass (28 layers, S = 950) -> frames/s of a 32-step run."""
    from oracle import backbone as O
    from workload import configs as CFG, gen
    w = CFG.c4()
    e = w.extra
    layers = []
    for l in range(28):
        h = CFG.layer_weights(w.seed, w.shape, l, True)
        layers.append(O.Layer.from_arrays({k: (gen.bf16_bits_to_f32(v) if v.dtype == np.uint16 else v)
                                           for k, v in h.items()}))
    text = CFG.LazyTable(w.seed, gen.KIND_TEXT_TABLE, 0, e["text_vocab"], 1024, True)
    tab = CFG.LazyTable(w.seed, gen.KIND_CB_TABLE, 0, e["n_cb"] * e["cb_vocab"], 1024, True)
    heads = CFG.LazyTable(w.seed, gen.KIND_HEAD, 0, e["n_cb"] * e["cb_vocab"], 1024, True)
    head_full = heads[np.arange(e["n_cb"] * e["cb_vocab"])]
    codes = CFG.maskgit_codes(w)
    t0 = time.perf_counter()
    O.maskgit_pass(CFG.maskgit_text_ids(w), text, codes, tab, head_full, layers,
                   CFG.final_norm(w.seed, w.shape).astype(np.float64), O.Dims(), e["cb_vocab"],
                   e["mask_id"], e["layer_penalty"], 100)
    dt = time.perf_counter() - t0
    return {"pass_seconds": dt, "frames_per_s": e["n_frames"] / (dt * e["n_steps"])}


# ---------------------------------------------------------------------------------------

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attn_c5_traffic.md")
TRAFFIC_SOURCES = [os.path.join(ROOT, "codec_token_tts_amd", "csrc", f)
                   for f in ("k_rope_decode.hip", "common.h", "kernels.h")]


def host_cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode-attention launch from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy-kernel calibration), or None when there is none or the
    kernel's sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if ":" in line and line.strip().startswith("- "):
                k, v = line.strip()[2:].split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, mib: int):
    """One plain copy of `mib` MiB (workload library copy kernel): the known-traffic
    reference that scales the FETCH_SIZE / WRITE_SIZE counters."""
    from workload import device as DEV
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    DEV.copy(a, b, n)
    torch.cuda.synchronize()
    del a, b


def run_rvq(T, torch, n_frames, iters):
    """Timed codec RVQ decode: 8 codebooks of 1024 x 64 fp32 projected to 1024."""
    from workload import gen
    nq, cb, dim, od = 8, 1024, 64, 1024
    emb = torch.from_numpy(gen.normal_f32(5, gen.stream_id(gen.KIND_CB_TABLE, 9), (nq, cb, dim))).cuda()
    w = torch.from_numpy(gen.normal_f32(5, gen.stream_id(gen.KIND_HEAD, 9), (nq, od, dim), 0.05)).cuda()
    b = torch.from_numpy(gen.normal_f32(5, gen.stream_id(gen.KIND_FINAL_NORM, 9), (nq, od), 0.1)).cuda()
    codes = torch.from_numpy(gen.uniform_int(5, gen.stream_id(gen.KIND_CODES, 9), (nq, n_frames), cb)).cuda()
    out = torch.empty((n_frames, od), dtype=torch.float32, device="cuda")
    cfg = T.ttsbb_default_config()
    cfg.n_layers = 0
    cfg.dtype = T.F32
    ctx = T.ttsbb_create(cfg, [], None, torch.cuda.current_stream().cuda_stream)
    try:
        T.ttsbb_rvq_decode(ctx, n_frames, nq, cb, dim, od, codes, emb, w, b, out)
        torch.cuda.synchronize()
        # the kernel's own duration (events stamped at its start and end): a loop of calls
        # through the binding would time the host's call overhead instead
        T.ttsbb_profile_start(ctx, 1 << T.K_NAMES.index("rvq"))
        for _ in range(iters):
            T.ttsbb_rvq_decode(ctx, n_frames, nq, cb, dim, od, codes, emb, w, b, out)
        ms, n = T.ttsbb_profile_stop(ctx)["rvq"]
        if T.ttsbb_sync(ctx) != T.OK or n != iters:
            raise RuntimeError("device flag raised by the RVQ decode")
        return ms * 1e3 / iters
    finally:
        T.ttsbb_destroy(ctx)


def run_prefill(T, torch, dec, n_tokens, iters):
    """Timed causal prefill of one stream's n_tokens-token prompt through the 28 layers
    (Talker prompt), on the decode context: a fresh stream (cache length 0) on pages of
    its own, reset before each call; head + argmax on the last token."""
    from workload import configs as CFG, gen
    import numpy as np
    pt = np.full((1, dec.pt.shape[1]), -1, np.int32)
    n_need = (n_tokens + 15) // 16
    spare = np.setdiff1d(np.arange(dec.n_pages), dec.pt[dec.pt >= 0])
    if spare.size < n_need:
        raise RuntimeError("not enough spare pages for the prefill stream")
    pt[0, :n_need] = spare[:n_need]
    pt_d = torch.from_numpy(pt).cuda()
    x0 = torch.from_numpy(gen.fast_normal(5, gen.stream_id(gen.KIND_X_IN, 7), (n_tokens, 1024), 1.0)).cuda()
    x = torch.empty_like(x0)
    cl = torch.zeros(1, dtype=torch.int32, device="cuda")
    am = torch.empty(dec.K, dtype=torch.int32, device="cuda")
    T.ttsbb_prefill(dec.ctx, n_tokens, x0.clone(), cl, pt_d, pt.shape[1], dec.pool, dec.n_pages, dec.heads, dec.K,
                    dec.V, am)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total = 0.0
    for _ in range(iters):
        x.copy_(x0)
        cl.zero_()
        e0.record()
        T.ttsbb_prefill(dec.ctx, n_tokens, x, cl, pt_d, pt.shape[1], dec.pool, dec.n_pages, dec.heads, dec.K,
                        dec.V, am)
        e1.record()
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1)
    if T.ttsbb_sync(dec.ctx) != T.OK:
        raise RuntimeError("device flag raised by the prefill")
    return total / iters


def run_c3(T, torch, iters):
    """The 5-layer code predictor: 256 frames in lockstep, a 1-token prefill of the frame's
    hidden state at position 0, then 15 q_len = 1 steps, step s embedding code s-1 with
    table s-1 and choosing code s with head s-1 (greedy, fed back on the device).  One
    frame batch = those 16 calls (and 15 embeddings), ~720 small kernels.  Timed eagerly
    and as one HIP graph of the whole frame batch (torch's stream capture on the context's
    own stream), whose codes must equal the eager run's.  Returns (eager, graph) ms per
    frame batch.
    Roofline (HBM-bound, ~200 flop/B): the 5 layers' bf16 weights (157.3 MB) in each of
    the 16 calls, the 15 heads (4.2 MB each) and the KV of positions 0..s of every frame
    and layer (4 KB each) in call s: 3.29 GB, 0.412 ms at 8 TB/s."""
    from workload import configs as CFG, device as DEV, gen
    w = CFG.c3()
    e = w.extra
    F, steps, V = e["batch"], e["steps"], e["cb_vocab"]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        ctx, keep = make_ctx(T, torch, w.shape, 5, True, w.seed, F, 64, V, DEV, CFG)
    try:
        pt, n_pages = CFG.page_table(w.seed, [16] * F)
        pool = DEV.kv_pool(w.seed, w.shape, 5, [0] * F, pt, n_pages, True)
        pt_d = torch.from_numpy(pt).cuda()
        tabs = [DEV.table(w.seed, gen.KIND_CB_TABLE, s, V, 1024, True) for s in range(steps)]
        heads = [DEV.table(w.seed, gen.KIND_HEAD, s, V, 1024, True) for s in range(steps)]
        hidden = torch.from_numpy(gen.fast_normal(w.seed, gen.stream_id(gen.KIND_X_IN, 0), (F, 1024), 1.0)).cuda()
        c0 = torch.from_numpy(gen.uniform_int(w.seed, gen.stream_id(gen.KIND_CODES, 0), (F,), V)).cuda()
        pos = torch.zeros(F, dtype=torch.int32, device="cuda")
        x = torch.empty((F, 1024), dtype=torch.float32, device="cuda")
        codes = torch.empty((steps + 1, F, 1), dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

        def frame_batch():
            pos.zero_()
            x.copy_(hidden)
            codes[0, :, 0] = c0
            T.ttsbb_decode_step(ctx, F, x, pos, pt_d, 1, pool, n_pages)
            for s in range(1, steps + 1):
                T.ttsbb_codebook_embed(ctx, F, 1, codes[s - 1], tabs[s - 1], V, None, None, None, 0, x)
                T.ttsbb_decode_step(ctx, F, x, pos, pt_d, 1, pool, n_pages, heads[s - 1], 1, V, codes[s])

        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):
            frame_batch()
            side.synchronize()
            e0.record(side)
            for _ in range(iters):
                frame_batch()
            e1.record(side)
            torch.cuda.synchronize()
            eager_ms = e0.elapsed_time(e1) / iters
            codes_eager = codes.clone()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                frame_batch()
            g.replay()  # warm
            e0.record(side)
            for _ in range(iters):
                g.replay()
            e1.record(side)
            torch.cuda.synchronize()
            graph_ms = e0.elapsed_time(e1) / iters
        if not torch.equal(codes, codes_eager):
            raise RuntimeError("graph replay of the code predictor differs from the eager run")
        if T.ttsbb_sync(ctx) != T.OK:
            raise RuntimeError("device flag raised by the code predictor")
        del g
        return eager_ms, graph_ms
    finally:
        torch.cuda.synchronize()
        T.ttsbb_destroy(ctx)


C3_ROOFLINE_BYTES = (16 * 5 * 15728640 * 2 + 15 * 2048 * 1024 * 2
                     + sum(s + 1 for s in range(16)) * 256 * 4096 * 5)


def run_c2_graph(T, torch, dec, n_steps=148):
    """Batch-1 decode loop of the 16-codebook / 3072-head configuration (28 layers, KV
    1000 -> 1148, codes drawn up front): timed eagerly, then captured once as ONE HIP graph
    of all n_steps steps (torch's stream capture on the context's own stream) and timed as
    one replay.  The layer weights are the decode context's; the two runs' argmax
    trajectories must agree."""
    from workload import configs as CFG, device as DEV, gen
    w = CFG.c2()
    e = w.extra
    L0, K, V, HV = e["prefill"][0], e["n_cb"], e["cb_vocab"], e["head_vocab"]
    side = torch.cuda.Stream()
    dev, fn = dec.keep
    cfg = T.ttsbb_default_config()
    cfg.n_layers = len(dev)
    cfg.dtype = T.BF16
    cfg.max_rows, cfg.max_pos, cfg.max_head_cols = 64, 2048, 4096
    layers = [T.make_layer(*[d[k] for k in ("attn_norm", "q_norm", "k_norm", "ffn_norm", "wq", "wk",
                                             "wv", "wo", "w_gate", "w_up", "w_down")]) for d in dev]
    ctx = T.ttsbb_create(cfg, layers, fn, side.cuda_stream)
    try:
        pt, n_pages = CFG.page_table(w.seed, [L0 + n_steps + 1])
        pool = DEV.kv_pool(w.seed, w.shape, len(dev), [L0], pt, n_pages, True)
        pt_d = torch.from_numpy(pt).cuda()
        tables = DEV.table(w.seed, gen.KIND_CB_TABLE, 0, K * V, 1024, True)
        head = DEV.table(w.seed, gen.KIND_HEAD, 0, HV, 1024, True)
        codes = np.stack([gen.uniform_int(w.seed, gen.stream_id(gen.KIND_CODES, s), (1, K), V)
                          for s in range(n_steps)])
        codes_d = torch.from_numpy(codes.astype(np.int32)).cuda()
        pos = torch.tensor([L0], dtype=torch.int32, device="cuda")
        x = torch.empty((1, 1024), dtype=torch.float32, device="cuda")
        am = torch.empty((n_steps, 1), dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()

        def loop():
            for s in range(n_steps):
                T.ttsbb_codebook_embed(ctx, 1, K, codes_d[s], tables, V, None, None, None, 0, x)
                T.ttsbb_decode_step(ctx, 1, x, pos, pt_d, pt.shape[1], pool, n_pages, head, 1, HV, am[s])

        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):
            pos.fill_(L0)
            loop()                                  # warm
            pos.fill_(L0)
            e0.record(side)
            loop()
            e1.record(side)
            torch.cuda.synchronize()
            eager_ms = e0.elapsed_time(e1)
            am_eager = am.clone()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                loop()
            pos.fill_(L0)
            g.replay()                              # warm
            pos.fill_(L0)
            e0.record(side)
            g.replay()
            e1.record(side)
            torch.cuda.synchronize()
            graph_ms = e0.elapsed_time(e1)
        if not torch.equal(am, am_eager) or int(pos.item()) != L0 + n_steps:
            raise RuntimeError("graph replay of the batch-1 decode loop differs from the eager loop")
        if T.ttsbb_sync(ctx) != T.OK:
            raise RuntimeError("device flag raised by the batch-1 decode loop")
        del g
        return eager_ms / n_steps, graph_ms / n_steps
    finally:
        torch.cuda.synchronize()
        T.ttsbb_destroy(ctx)


def run_c5c4(args, T, torch):
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
    total = args.warmup + 2 * args.steps
    log("setup: decode (64 streams, paged KV) ...")
    dec = DecodeC5(T, torch, total)
    log("setup: MaskGIT (S = 950) ...")
    mg = MaskgitC4(T, torch)
    torch.cuda.synchronize()
    for s in range(args.warmup):
        dec.step(s)
        mg.step(s)
    torch.cuda.synchronize()
    if T.ttsbb_sync(dec.ctx) != T.OK or T.ttsbb_sync(mg.ctx) != T.OK:
        raise RuntimeError("device-side index flag raised during warmup")
    log("timed: %d steps" % args.steps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    # The roofline kernel (decode attention) is timed inside the timed region by HIP events
    # that the library records on its own stream around each of its launches.
    T.ttsbb_profile_start(dec.ctx, 1 << T.K_NAMES.index("decode_attn"))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        s = args.warmup + i
        ev[i][0].record()
        dec.step(s)
        ev[i][1].record()
        mg.step(s)
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timed_attn = T.ttsbb_profile_stop(dec.ctx)["decode_attn"]
    dec_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
    mg_ms = sum(b.elapsed_time(c) for _, b, c in ev) / args.steps

    # Per-kernel durations: HIP events recorded by the library on its stream around each
    # launch, over the same number of further steps (events add a little time per launch,
    # so they are kept out of the timed region above).
    log("profiled: %d steps" % args.steps)
    T.ttsbb_profile_start(dec.ctx)
    T.ttsbb_profile_start(mg.ctx)
    for i in range(args.steps):
        s = args.warmup + args.steps + i
        dec.step(s)
        mg.step(s)
    pd = T.ttsbb_profile_stop(dec.ctx)
    pm = T.ttsbb_profile_stop(mg.ctx)

    extras = {}
    if not args.no_extras:
        extras = run_extras(args, T, torch, dec, mg)
    return assemble(args, dec, mg, dec_ms, mg_ms, wall, timed_attn, pd, pm, extras)


def run_extras(args, T, torch, dec, mg):
    """The figures beside the headline workload: guided and sampled MaskGIT steps, a whole
    32-step MaskGIT generation, the causal prefill, the RVQ decode, the code predictor and
    the batch-1 decode loop."""
    # Guided MaskGIT step (classifier-free guidance), timed on its own after the step
    log("timed: %d guided MaskGIT steps" % args.steps)
    mg.step_cfg(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        mg.step_cfg(i)
    e1.record()
    torch.cuda.synchronize()
    cfg_ms = e0.elapsed_time(e1) / args.steps
    log("timed: %d guided + sampled MaskGIT steps" % args.steps)
    mg.step_sampled(0)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        mg.step_sampled(i)
    e1.record()
    torch.cuda.synchronize()
    smp_ms = e0.elapsed_time(e1) / args.steps

    # One whole MaskGIT generation: the 32 cosine-schedule steps from the initial codes,
    # each step's codes feeding the next on the device; at the end no position is masked
    log("timed: one 32-step MaskGIT generation")
    n_steps = mg.e["n_steps"]
    for i in range(n_steps):  # warm
        mg.step(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n_steps):
        mg.step(i)
    e1.record()
    torch.cuda.synchronize()
    gen_ms = e0.elapsed_time(e1)
    if int((mg.codes == mg.e["mask_id"]).sum().item()) != 0:
        raise RuntimeError("positions still masked after the 32-step generation")

    # Causal prefill of a 200-token prompt of one stream (28 layers)
    log("timed: prefill")
    pf_ms = run_prefill(T, torch, dec, 200, args.steps)

    # Codec RVQ decode of the pass's 750 frames (8 codebooks x 1024 x 64 -> 1024, fp32)
    rvq_us = run_rvq(T, torch, mg.e["n_frames"], args.steps)

    # The 5-layer code predictor: 256 frames x (1-token prefill + 15 steps)
    log("timed: code predictor")
    c3_eager_ms, c3_ms = run_c3(T, torch, args.steps)

    # Batch-1 decode loop (16 codebooks, 3072 head, KV 1000, 148 steps): eager vs one graph
    c2_eager_ms = c2_graph_ms = None
    if not args.no_graph:
        log("timed: batch-1 decode loop, eager and as one HIP graph")
        c2_eager_ms, c2_graph_ms = run_c2_graph(T, torch, dec)
    return {
        "maskgit_generation": {"ms": round(gen_ms, 3), "steps": n_steps,
                               "frames_per_s": round(mg.e["n_frames"] / (gen_ms * 1e-3), 1),
                               "note": "one whole generation: 32 cosine-schedule steps (28-layer pass, fused "
                                       "scoring, top-n unmasking) from the 3000-masked codes, each step's codes "
                                       "feeding the next on the device; no position masked at the end"},
        "maskgit_cfg": {"ms_per_pass": round(cfg_ms, 4),
                        "frames_per_s": round(mg.e["n_frames"] / (cfg_ms * 1e-3 * mg.e["n_steps"]), 1),
                        "note": "guided step: conditional 950-token prompt + unconditional 750-frame window, "
                                "cfg_scale 2.0"},
        "prefill": {"ms_per_call": round(pf_ms, 4), "tokens": 200,
                    "tokens_per_s": round(200 / (pf_ms * 1e-3), 1),
                    "note": "causal prefill of one stream's 200-token prompt into fresh pages, 28 layers, "
                            "head + argmax on the last token"},
        "rvq_decode": {"us_per_call": round(rvq_us, 2), "frames": mg.e["n_frames"],
                       "gflops_fp32": round(2.0 * mg.e["n_frames"] * 8 * 64 * 1024 / (rvq_us * 1e-6) / 1e9, 1),
                       "mfma_frac_fp32": round(2.0 * mg.e["n_frames"] * 8 * 64 * 1024 / (rvq_us * 1e-6) / 157.3e12, 4),
                       "note": "codec RVQ decode, 8 x (1024 x 64) codebooks -> 1024, fp32 matrix cores; "
                               "kernel duration from events stamped at its start and end"},
        "maskgit_sampled": {"ms_per_pass": round(smp_ms, 4),
                            "frames_per_s": round(mg.e["n_frames"] / (smp_ms * 1e-3 * mg.e["n_steps"]), 1),
                            "note": "guided + sampled step: cfg_scale 2.0, top-k ratio 0.1, class and position "
                                    "temperature 1.0, Gumbel uniforms drawn on the device (Philox4x32-10)"},
        "code_predictor": {"ms_per_frame_batch": round(c3_ms, 4), "codes_per_s": round(256 * 15 / (c3_ms * 1e-3), 1),
                           "eager_ms_per_frame_batch": round(c3_eager_ms, 4),
                           "roofline_ms": round(C3_ROOFLINE_BYTES / (HBM_PEAK_GBS * 1e9) * 1e3, 4),
                           "frac_of_roofline": round(C3_ROOFLINE_BYTES / (HBM_PEAK_GBS * 1e9) * 1e3 / c3_ms, 4),
                           "note": "5 layers, 256 frames: 1-token prefill + 15 steps, 15 tables and 2048-way heads, "
                                   "argmax fed back on the device; the frame batch captured as one HIP graph "
                                   "(replays produce the eager run's codes); roofline = 3.29 GB of weights, "
                                   "heads and KV at 8 TB/s"},
        "decode_b1_loop": None if c2_graph_ms is None else {
            "eager_ms_per_step": round(c2_eager_ms, 4), "graph_ms_per_step": round(c2_graph_ms, 4),
            "graph_tokens_per_s": round(1.0 / (c2_graph_ms * 1e-3), 1), "steps": 148,
            "note": "batch-1 28-layer decode, 16 x 2048 summed codebooks, 3072 head + argmax, "
                    "KV 1000 -> 1148: eager launches vs the 148 steps captured as one HIP graph"},
    }


def assemble(args, dec, mg, dec_ms, mg_ms, wall, timed_attn, pd, pm, extras):
    attn_ms, attn_n = timed_attn
    attn_avg_ms = attn_ms / max(1, attn_n)
    attn_bytes = dec.attn_bytes(args.warmup, args.steps)
    attn_gbs = attn_bytes / (attn_avg_ms * 1e-3) / 1e9
    gemm, attn_f, head_f = mg.flops()
    mg_mfma_ms = sum(pm[k][0] for k in ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down",
                                        "flash_attn")) / args.steps
    mfma_tflops = (gemm + attn_f) / (mg_mfma_ms * 1e-3) / 1e12
    # per-kernel figures: MaskGIT products and attention against the bf16 MFMA peak; the
    # decode projections against HBM as weight streaming (31.46 MB of bf16 weights per
    # layer, each read once per step); the embeddings against HBM (gathered table rows in,
    # fp32 rows out)
    S = mg.e["n_text"] + mg.e["n_frames"]
    per_kernel_flops = {"gemm_qkv": 2 * S * 4096 * 1024 * 28, "gemm_o": 2 * S * 1024 * 2048 * 28,
                        "gemm_gate_up": 2 * S * 6144 * 1024 * 28, "gemm_down": 2 * S * 1024 * 3072 * 28,
                        "flash_attn": attn_f}
    mg_kernels = {}
    for k, f in per_kernel_flops.items():
        ms = pm[k][0] / args.steps
        if ms > 0:
            mg_kernels[k] = {"tflops": round(f / (ms * 1e-3) / 1e12, 1),
                             "mfma_util": round(f / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    w_bytes = 28 * 2 * (1024 * 4096 + 2048 * 1024 + 1024 * 6144 + 3072 * 1024)
    dec_gemm_ms = sum(pd[k][0] for k in ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down")) / args.steps
    dec_embed_ms = pd["embed"][0] / args.steps
    mg_embed_ms = pm["embed"][0] / args.steps
    dec_embed_bytes = dec.B * (dec.K * 1024 * 2 + 1024 * 4)
    mg_embed_bytes = mg.e["n_frames"] * mg.e["n_cb"] * 1024 * 2 + mg.e["n_text"] * 1024 * 2 + S * 1024 * 4

    res = {
        "metric": METRIC,
        "value": round(dec.B / (dec_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Philox inputs, random weights)",
        "config": {"workload": "c5 paged decode (64 streams, 28 layers, KV U[200,4000], 16-token pages, "
                               "8x1025) + c4 MaskGIT pass (28 layers, S=950, 8x1025)",
                   "global_batch": dec.B, "seq_len": int(dec.lengths.max()), "parallelism": "none (1 GPU)"},
        "decode": {"ms_per_iteration": round(dec_ms, 4), "tokens_per_s": round(dec.B / (dec_ms * 1e-3), 1),
                   "attn_hbm_gbs": round(attn_gbs, 1), "attn_frac_hbm_peak": round(attn_gbs / HBM_PEAK_GBS, 4),
                   "projections_weight_gbs": round(w_bytes / (dec_gemm_ms * 1e-3) / 1e9, 1) if dec_gemm_ms else None,
                   "embed_gbs": round(dec_embed_bytes / (dec_embed_ms * 1e-3) / 1e9, 1) if dec_embed_ms else None},
        "maskgit": {"ms_per_pass": round(mg_ms, 4),
                    "frames_per_s": round(mg.e["n_frames"] / (mg_ms * 1e-3 * mg.e["n_steps"]), 1),
                    "mfma_tflops": round(mfma_tflops, 1),
                    "mfma_util": round(mfma_tflops / BF16_PEAK_TFLOPS, 4),
                    "kernels": mg_kernels,
                    "embed_gbs": round(mg_embed_bytes / (mg_embed_ms * 1e-3) / 1e9, 1) if mg_embed_ms else None},
        "roofline": {"kernel": "decode_attn (split-sequence paged GQA attention)", "bound": "hbm",
                     "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "avg_launch_us": round(attn_avg_ms * 1e3, 3),
                     "algorithmic_bytes_per_launch": int(attn_bytes)},
        "kernels_ms_per_step": {
            "decode": {k: round(v[0] / args.steps, 4) for k, v in pd.items() if v[1]},
            "maskgit": {k: round(v[0] / args.steps, 4) for k, v in pm.items() if v[1]}},
    }
    res.update(extras)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c5c4", choices=["c5c4"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-streams", type=int, default=2)
    ap.add_argument("--cpu-steps", type=int, default=40)
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-captured batch-1 loop (hardware-counter runs: the profiler's "
                         "per-dispatch counter collection does not support stream capture)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline workload (decode step + MaskGIT pass): for counter runs")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run one plain copy of MIB MiB first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each GPU would run its own "
              "streams / utterances with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from codec_token_tts_amd import ttsbb as T
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    T.lib()
    res = run_c5c4(args, T, torch)
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle decode sample ...")
        cb = cpu_baseline(args.cpu_streams, args.cpu_steps)
        log("cpu baseline: oracle MaskGIT pass ...")
        cm = cpu_baseline_maskgit()
        cb["maskgit_frames_per_s"] = round(cm["frames_per_s"], 3)
        cb["maskgit_pass_seconds"] = round(cm["pass_seconds"], 2)
        cb["value"] = round(cb["value"], 3)
        cb["seconds"] = round(cb["seconds"], 2)
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
