"""Helpers of the GPU parity tests: build a ttsbb context over seeded device weights, the
matching oracle layers on the host, and the comparison rules for discrete outputs."""
from __future__ import annotations

import numpy as np

from oracle import backbone as O
from workload import configs as CFG
from workload import device as DEV
from workload import gen


# bf16-mode tolerances (normwise max|gpu - ref| / max|ref|):
# * one layer's output: 2e-2, the bound stated for layer outputs;
# * a 28-layer stack: 3e-2.  Rounding the operands of the four products and the new K/V
#   to bf16 in every layer, and nothing else, already moves the 28-layer output of the
#   batch-1 decode workload by 1.8% (1.95% rms) from the exact result; the bound allows
#   that plus the fp32 accumulation-order differences of the GPU kernels.
TOL_LAYER_BF16 = 2e-2
TOL_STACK_BF16 = 3e-2


def torch():
    import torch as _t
    return _t


def widen(a: np.ndarray) -> np.ndarray:
    return gen.bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


def dims_of(shape: CFG.Shape) -> O.Dims:
    return O.Dims(hidden=shape.hidden, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
                  head_dim=shape.head_dim, ffn=shape.ffn, eps=shape.eps, theta=shape.theta)


class Model:
    """Device weights + ttsbb context, and (lazily) the oracle's fp64 layers."""

    def __init__(self, shape: CFG.Shape, n_layers: int, bf16: bool, seed: int = 0,
                 gains: str = "ones", max_rows: int = 1024, max_pos: int = 8192,
                 max_head_cols: int = 8200, stream=None):
        from codec_token_tts_amd import ttsbb as T
        self.T = T
        self.shape, self.n_layers, self.bf16, self.seed, self.gains = shape, n_layers, bf16, seed, gains
        self.dev = [DEV.layer_weights(seed, shape, l, bf16, gains) for l in range(n_layers)]
        self.final_norm = DEV.host_to_device(CFG.final_norm(seed, shape, gains))
        cfg = T.ttsbb_default_config()
        cfg.n_layers = n_layers
        cfg.hidden, cfg.n_heads, cfg.n_kv_heads = shape.hidden, shape.n_heads, shape.n_kv_heads
        cfg.head_dim, cfg.ffn = shape.head_dim, shape.ffn
        cfg.rms_eps, cfg.rope_theta = shape.eps, shape.theta
        cfg.dtype = T.BF16 if bf16 else T.F32
        cfg.max_rows, cfg.max_pos, cfg.max_head_cols = max_rows, max_pos, max_head_cols
        self.cfg = cfg
        self.layers = [T.make_layer(d["attn_norm"], d["q_norm"], d["k_norm"], d["ffn_norm"],
                                    d["wq"], d["wk"], d["wv"], d["wo"], d["w_gate"], d["w_up"],
                                    d["w_down"]) for d in self.dev]
        if stream is None:
            stream = torch().cuda.current_stream().cuda_stream
        self.ctx = T.ttsbb_create(cfg, self.layers, self.final_norm, stream)
        self._oracle_layers = None

    def oracle_layers(self):
        if self._oracle_layers is None:
            out = []
            for l in range(self.n_layers):
                h = CFG.layer_weights(self.seed, self.shape, l, self.bf16, self.gains)
                out.append(O.Layer.from_arrays({k: widen(v) for k, v in h.items()}))
            self._oracle_layers = out
        return self._oracle_layers

    def oracle_final_norm(self):
        return CFG.final_norm(self.seed, self.shape, self.gains).astype(np.float64)

    def close(self):
        if self.ctx:
            self.T.ttsbb_destroy(self.ctx)
            self.ctx = None


def read_tap(model: Model, tap: int, rows: int, cols: int) -> np.ndarray:
    t = torch().empty(rows * cols, dtype=torch().float32, device="cuda")
    r, c = model.T.ttsbb_read_tap(model.ctx, tap, t, rows * cols)
    assert (r, c) == (rows, cols), (r, c, rows, cols)
    torch().cuda.synchronize()
    return t.cpu().numpy().reshape(rows, cols).astype(np.float64)


def normwise(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / max |ref| over the tensor."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / (den if den > 0 else 1.0))


def check_argmax_groups(gpu_choice: np.ndarray, gpu_logits: np.ndarray, ref_logits: np.ndarray,
                        exclude=None):
    """Discrete parity of a greedy choice.

    1. The GPU's choice is exactly the argmax of the GPU's own logits (ties -> lowest id).
    2. With delta = max |gpu - ref| over the group, the choice equals the reference argmax
       wherever the reference's top-2 gap exceeds 2*delta; elsewhere (a near tie) it must
       be within 2*delta of the reference maximum.
    Returns the number of near-tie groups.  Arrays are [..., V]."""
    g = np.asarray(gpu_logits, np.float64)
    r = np.asarray(ref_logits, np.float64)
    ch = np.asarray(gpu_choice).reshape(g.shape[:-1])
    if exclude is not None:
        g = g.copy()
        r = r.copy()
        g[..., exclude] = -np.inf
        r[..., exclude] = -np.inf
    own = np.argmax(g, axis=-1)
    assert np.array_equal(own, ch), "choice is not the argmax of the GPU's own logits"
    fin = np.isfinite(r)
    diff = np.zeros_like(r)
    diff[fin] = np.abs(g[fin] - r[fin])  # excluded classes are -inf on both sides
    delta = np.max(diff, axis=-1)
    top2 = np.sort(r, axis=-1)[..., -2:]
    gap = top2[..., 1] - top2[..., 0]
    ref_arg = np.argmax(r, axis=-1)
    clear = gap > 2 * delta
    assert np.array_equal(ch[clear], ref_arg[clear]), "argmax differs where the margin is clear"
    chosen = np.take_along_axis(r, ch[..., None], axis=-1)[..., 0]
    assert np.all(chosen >= top2[..., 1] - 2 * delta - 1e-12), "near-tie choice is not near the top"
    return int(np.count_nonzero(~clear))


def check_topn(picked: np.ndarray, conf_gpu: np.ndarray, conf_ref: np.ndarray, n: int):
    """Discrete parity of the top-n selection.

    1. picked is exactly the top-n of the GPU's own scores (decreasing, ties -> lower flat
       index, -1 where fewer than n are finite).
    2. Against the reference, with eps = max |gpu - ref| over finite scores: every element
       whose reference score clears the reference's n-th score by 2*eps is picked, and no
       picked element falls 2*eps below it.  Returns the count of boundary elements."""
    cg = np.asarray(conf_gpu, np.float64).reshape(-1)
    cr = np.asarray(conf_ref, np.float64).reshape(-1)
    order = sorted([(-cg[i], i) for i in range(cg.size) if np.isfinite(cg[i])])
    own = [i for _, i in order[:n]] + [-1] * max(0, n - len(order))
    assert list(np.asarray(picked).reshape(-1)) == own[:n], "picked is not the top-n of the GPU scores"
    assert np.array_equal(np.isfinite(cg), np.isfinite(cr)), "masked positions differ"
    fin = np.isfinite(cr)
    if not fin.any() or n == 0:
        return 0
    eps = float(np.max(np.abs(cg[fin] - cr[fin])))
    ranked = np.sort(cr[fin])[::-1]
    if n > ranked.size:
        return 0
    thr = ranked[n - 1]
    sel = set(int(i) for i in picked if i >= 0)
    must = np.nonzero(fin & (cr > thr + 2 * eps))[0]
    assert all(int(i) in sel for i in must), "a clearly winning position was not picked"
    assert all(cr[i] >= thr - 2 * eps for i in sel), "a clearly losing position was picked"
    return int(np.count_nonzero(fin & (np.abs(cr - thr) <= 2 * eps)))


def check_sampler(gpu_pred, gpu_conf, guided_gpu, guided_ref, window, n_cb, V, mask_id, penalty, class_temp,
                  pos_temp, ratio, u_class, u_pos, eps=2e-3):
    """Discrete parity of the sampler's choices, in two stages.

    1. GPU against an fp64 emulation of the same scoring on the GPU's own guided logits
       (same uniforms): equal choices except where the emulation has a near tie (within
       eps) or the chosen class sits within eps of the top-k threshold; equal scores to
       eps where the choices agree (the difference is fp32 arithmetic).
    2. The emulation against the oracle (guided_ref): equal choices wherever the oracle's
       margin exceeds twice the perturbed-value error, else the choice is within that
       margin of the oracle's best or at the threshold boundary.
    Returns (stage-1 exceptions, stage-2 exceptions)."""
    T = guided_gpu.shape[0]
    pe, ce, lpe = O.sample_scores(guided_gpu, window, n_cb, V, mask_id, penalty, class_temp, pos_temp, ratio,
                                  u_class, u_pos)
    pr, cr, lpr = O.sample_scores(guided_ref, window, n_cb, V, mask_id, penalty, class_temp, pos_temp, ratio,
                                  u_class, u_pos)
    _, _, lp0e = O.maskgit_scores(guided_gpu, window, n_cb, V, mask_id, penalty)
    _, _, lp0r = O.maskgit_scores(guided_ref, window, n_cb, V, mask_id, penalty)
    k_keep = max(1, int(np.floor(ratio * V)))
    thr_e = -np.sort(-lp0e, axis=-1)[..., k_keep - 1] if class_temp > 0 else None
    thr_r = -np.sort(-lp0r, axis=-1)[..., k_keep - 1] if class_temp > 0 else None
    gp = np.asarray(gpu_pred)
    ex1 = ex2 = 0
    both = np.isfinite(lpe) & np.isfinite(lpr)
    dl = float(np.max(np.abs(lpe[both] - lpr[both]))) if both.any() else 0.0
    fin0 = np.isfinite(lp0e) & np.isfinite(lp0r)
    d0 = float(np.max(np.abs(lp0e[fin0] - lp0r[fin0]))) if fin0.any() else 0.0
    for k in range(n_cb):
        for t in range(T):
            if gp[k, t] != pe[k, t]:
                # a near tie of the perturbed values, or either choice at the top-k edge
                # (kept on one side, dropped on the other)
                c, e = gp[k, t], pe[k, t]
                near = lpe[k, t, c] >= np.max(lpe[k, t]) - eps
                edge = class_temp > 0 and min(abs(lp0e[k, t, c] - thr_e[k, t]),
                                              abs(lp0e[k, t, e] - thr_e[k, t])) <= eps
                assert near or edge, "GPU choice differs from the emulation without a tie (%d, %d)" % (k, t)
                ex1 += 1
            elif np.isfinite(ce[k, t]):
                assert abs(float(gpu_conf[k, t]) - ce[k, t]) <= eps * (1 + abs(ce[k, t])), (k, t)
            if pe[k, t] != pr[k, t]:
                c, r = pe[k, t], pr[k, t]
                near = lpr[k, t, c] >= np.max(lpr[k, t]) - 2 * dl - 1e-9
                edge = class_temp > 0 and min(abs(lp0r[k, t, c] - thr_r[k, t]),
                                              abs(lp0r[k, t, r] - thr_r[k, t])) <= 2 * d0 + 1e-9
                assert near or edge, "emulated choice differs from the oracle's beyond the margin (%d, %d)" % (k, t)
                ex2 += 1
    assert np.array_equal(np.isfinite(np.asarray(gpu_conf)), np.isfinite(cr))
    return ex1, ex2
