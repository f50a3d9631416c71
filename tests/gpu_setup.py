"""Helpers of the GPU parity tests: build a ttsbb context over seeded device weights, the
matching oracle layers on the host, and the comparison rules for discrete outputs."""
from __future__ import annotations

import numpy as np

from oracle import backbone as O
from workload import configs as CFG
from workload import device as DEV
from workload import gen


# bf16-mode tolerances (normwise max|gpu - ref| / max|ref|):
# * one layer against the exact oracle: 2e-2, the bound stated for layer outputs -- for a
#   stack, each checked layer on the GPU's own input to that layer (teacher-forced);
# * one layer against the bf16-storage emulation (tests/bf16_emulation.py: the same bf16
#   roundings on fp64 arithmetic): 5e-3.  Only fp32-versus-fp64 arithmetic separates the
#   two, and it reaches a bf16 value only where it flips a rounding (one flip of a
#   near-maximal element is already 2^-8..2^-7 normwise);
# * a free-running stack: such flips cascade (a flipped operand moves every output of
#   the next product, which flips more of the next rounding point); even correctly
#   rounded fp32 arithmetic drifts 5e-3 from the emulation over the 28-layer batch-1
#   decode stack (tests/test_bf16_emulation.py), so the GPU is held to at most what an
#   independent draw of the whole bf16 rounding noise would give: sqrt(2) x the
#   emulation's own distance from the oracle ("storage"; 1.89% for that stack), and to
#   (1 + sqrt(2)) x storage from the oracle (triangle inequality); never less than the
#   one-layer bounds.
TOL_LAYER_BF16 = 2e-2
TOL_EMUL_BF16 = 5e-3
# Discrete checks against a reference at a distance delta accept a different choice only
# at a near tie (a margin below 2 delta); for one or two layers, and for the 6000 groups
# of the MaskGIT workload, such groups may be at most NEAR_TIE_FRAC of all (more would
# make the check vacuous), and top-n boundary elements at most BOUNDARY_FRAC of the
# candidates.  Free-running deep stacks of few groups report their agreement instead:
# there delta is 1-2% of the largest logit, and the choices are checked bit for bit on
# the GPU's own head operand (check_head_teacher_forced).
NEAR_TIE_FRAC = 0.15
BOUNDARY_FRAC = 0.15


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


def elementwise(gpu: np.ndarray, ref: np.ndarray, floor: float = 1e-2) -> float:
    """max |gpu - ref| / |ref| over the elements with |ref| >= floor * max |ref| (the
    elementwise relative error; it is ill-posed for elements near zero)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    big = np.abs(ref) >= floor * np.max(np.abs(ref))
    return float(np.max(np.abs(gpu[big] - ref[big]) / np.abs(ref[big]))) if big.any() else 0.0


def check_stack(name: str, gpu, emul, exact):
    """A free-running bf16 stack's output against the emulation and the exact oracle (the
    bounds above, from the emulation's own distance to the oracle).  Prints normwise and
    elementwise figures."""
    d_emul = normwise(gpu, emul)
    d_exact = normwise(gpu, exact)
    storage = normwise(emul, exact)
    print("%s: vs emulation %.2e (elementwise %.2e); vs oracle %.2e (elementwise %.2e); bf16 storage %.2e"
          % (name, d_emul, elementwise(gpu, emul), d_exact, elementwise(gpu, exact), storage))
    assert d_emul <= max(TOL_EMUL_BF16, np.sqrt(2.0) * storage), (name, d_emul, storage)
    assert d_exact <= max(TOL_LAYER_BF16, (1 + np.sqrt(2.0)) * storage), (name, d_exact, storage)
    return d_emul, d_exact


def check_layer(name: str, gpu_out, emul_out, exact_out):
    """One layer on the GPU's own input: the layer bound against the oracle, TOL_EMUL_BF16
    against the emulation."""
    d_emul, d_exact = normwise(gpu_out, emul_out), normwise(gpu_out, exact_out)
    print("%s (teacher-forced layer): vs emulation %.2e, vs oracle %.2e (elementwise %.2e)"
          % (name, d_emul, d_exact, elementwise(gpu_out, exact_out)))
    assert d_emul <= TOL_EMUL_BF16, (name, d_emul)
    assert d_exact <= TOL_LAYER_BF16, (name, d_exact)


def check_head_teacher_forced(y, head, gpu_logits, gpu_choice, n_groups: int, V: int, exclude=None,
                              gap_rel: float = 1e-6, max_frac: float = 1e-3):
    """A head and its greedy choice on the GPU's own head operand y (bf16 values, as the
    GPU read them): the oracle's fp64 head on the same y, so only the order of the fp32
    accumulation separates the logits.  Checks
    * every logit within the order-independent bound of an fp32 sum of K exact products,
      |err| <= (K - 1) 2^-24 sum_i |y_i H_ci| (the bf16 x bf16 products are exact in fp32);
    * the choice equals the oracle's argmax bit for bit, except in a group whose oracle
      top-1 / top-2 gap is below gap_rel * max |logit| of the group (a tie fp32 cannot
      resolve); such groups are at most max_frac of all (at least one is allowed).
    Returns (near-tie groups, oracle logits [rows][n_groups * V])."""
    y = np.asarray(y, np.float64)
    H = np.asarray(head, np.float64)
    ref = y @ H.T
    bound = (y.shape[1] - 1) * 2.0 ** -24 * (np.abs(y) @ np.abs(H).T)
    err = np.abs(np.asarray(gpu_logits, np.float64) - ref)
    assert np.all(err <= bound), "logit beyond the fp32 accumulation bound: %g vs %g" % (
        float(np.max(err - bound)), float(np.max(bound)))
    rows = y.shape[0]
    r = ref.reshape(rows, n_groups, V).copy()
    if exclude is not None:
        r[..., exclude] = -np.inf
    ref_arg = np.argmax(r, axis=-1)
    top2 = np.sort(r, axis=-1)[..., -2:]
    scale = np.max(np.where(np.isfinite(r), np.abs(r), 0.0), axis=-1)
    near = (top2[..., 1] - top2[..., 0]) < gap_rel * scale
    ch = np.asarray(gpu_choice).reshape(rows, n_groups)
    assert not np.any((ch != ref_arg) & ~near), "choice differs from the oracle's at a resolvable gap"
    n_near = int(near.sum())
    print("teacher-forced head: %d groups, %d near ties, max |dlogit| %.2e (bound %.2e)"
          % (near.size, n_near, float(np.max(err)), float(np.max(bound))))
    assert n_near <= max(1, max_frac * near.size), n_near
    return n_near, ref


def check_scores_teacher_forced(gpu_pred, gpu_conf, gpu_picked, ref_logits, codes_kt, n_cb: int, V: int,
                                mask_id: int, penalty: float, n_unmask: int, gap_rel: float = 1e-6,
                                max_frac: float = 1e-3):
    """MaskGIT scoring and selection on the oracle's fp64 logits of the GPU's own head
    operand: pred bit-exact except at oracle near ties (as above), conf within the fp32
    evaluation of the log-softmax (2 max|dlogit| + 2e-5 + 2^-20 |conf|), the same masked
    set, and picked exactly the oracle's top-n of the GPU's own conf (ties: lower flat
    index).  Returns the near-tie count."""
    pred_r, conf_r, lp_r = O.maskgit_scores(ref_logits, codes_kt, n_cb, V, mask_id, penalty)
    T = ref_logits.shape[0]
    lg = np.asarray(ref_logits).reshape(T, n_cb, V).transpose(1, 0, 2).copy()
    lg[..., mask_id] = -np.inf
    top2 = np.sort(lg, axis=-1)[..., -2:]
    scale = np.max(np.where(np.isfinite(lg), np.abs(lg), 0.0), axis=-1)
    near = (top2[..., 1] - top2[..., 0]) < gap_rel * scale
    gp = np.asarray(gpu_pred)
    assert not np.any((gp != pred_r) & ~near), "pred differs from the oracle's at a resolvable gap"
    assert int(near.sum()) <= max(1, max_frac * near.size)
    cg = np.asarray(gpu_conf, np.float64)
    fin = np.isfinite(conf_r)
    assert np.array_equal(np.isfinite(cg), fin), "masked sets differ"
    ok = fin & (gp == pred_r)
    if ok.any():
        d = np.abs(cg[ok] - conf_r[ok])
        assert np.all(d <= 2e-5 + 2.0 ** -20 * np.abs(conf_r[ok])), float(np.max(d))
        print("teacher-forced scores: max |dconf| %.2e" % float(np.max(d)))
    want = O.select_top(cg.reshape(-1), n_unmask)
    assert np.array_equal(np.asarray(gpu_picked).reshape(-1), want), "picked is not the top-n of the GPU's scores"
    return int(near.sum())


def check_argmax_groups(gpu_choice: np.ndarray, gpu_logits: np.ndarray, ref_logits: np.ndarray,
                        exclude=None, max_near: float = NEAR_TIE_FRAC):
    """Discrete parity of a greedy choice.

    1. The GPU's choice is exactly the argmax of the GPU's own logits (ties -> lowest id).
    2. With delta = max |gpu - ref| over the group, the choice equals the reference argmax
       wherever the reference's top-2 gap exceeds 2*delta; elsewhere (a near tie) it must
       be within 2*delta of the reference maximum.
    3. Near-tie groups are at most max_near of all groups (max_near = None: not capped;
       only for a reference that is the GPU's own logits).
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
    n_near = int(np.count_nonzero(~clear))
    if max_near is not None:
        assert n_near <= max(1, max_near * clear.size), "near ties: %d of %d groups" % (n_near, clear.size)
    if clear.size > 1:
        print("argmax: %d groups, %d near ties, agreement with the reference %.4f"
              % (clear.size, n_near, float(np.mean(ch == ref_arg))))
    return n_near


def check_topn(picked: np.ndarray, conf_gpu: np.ndarray, conf_ref: np.ndarray, n: int,
               max_near: float = BOUNDARY_FRAC):
    """Discrete parity of the top-n selection.

    1. picked is exactly the top-n of the GPU's own scores (decreasing, ties -> lower flat
       index, -1 where fewer than n are finite).
    2. Against the reference, with eps = max |gpu - ref| over finite scores: every element
       whose reference score clears the reference's n-th score by 2*eps is picked, and no
       picked element falls 2*eps below it.
    3. Boundary elements (within 2*eps of that score) are at most max_near of the
       finite candidates (at least 2).  Returns their count."""
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
    n_near = int(np.count_nonzero(fin & (np.abs(cr - thr) <= 2 * eps)))
    if max_near is not None:
        assert n_near <= max(2, max_near * int(fin.sum())), "boundary elements: %d of %d" % (n_near, int(fin.sum()))
    return n_near


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
