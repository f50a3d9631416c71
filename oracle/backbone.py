"""Oracle for the TTS backbone hot path: plain, slow, fp64 CPU code.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares no
code with the HIP library (``codec_token_tts_amd``) and the HIP library never
imports it.

Every function is the plain definition written out in float64 with numpy; a
matrix product (``@``) and ``argsort`` are the only library primitives used as
steps.  Inputs arrive in whatever precision the caller stored them (fp32 values or
bf16 values widened to fp32); they are widened to float64 exactly and all
arithmetic happens in float64.

Sources (the pages, cited by title and section):
* [OV-IO]   OmniVoice ARCHITECTURE (omnivoice-cpp docs), "Qwen3 0.6B backbone with
            custom IO": hybrid text+audio input embedding, the Qwen3 specifics
            (per-head q/k RMSNorm before RoPE, GQA 16/8, no biases, SwiGLU, RoPE
            theta 1e6), and the (8200, 1024) audio head viewed per codebook.
* [OV-GGUF] same page, "GGUF layout": hyper-parameters and tensor names
            (input_layernorm, post_attention_layernorm, llm.norm, eps 1e-6).
* [OV-MG]   same page, "MaskGIT decoder": log-softmax, mask class to -inf, argmax,
            confidence = max log-prob - layer index * layer penalty, already
            unmasked positions to -inf, top-k over the flattened scores, token
            update; full bidirectional prefill every step.
* [OV-API]  same page, "Public API": sampler defaults (32 steps, layer penalty 5.0).
* [NC-ARCH] ncnn Qwen3-TTS port (Tencent/ncnn discussion 6877), "模型结构拆解":
            Talker 28 layers and Code Predictor 5 layers, 15 autoregressive steps
            per frame, summed codebook embeddings as the next input.
* [NC-ATTN] same page, "单token SDPA问题与host attention": the q_len=1 layer split
            PreRoPE -> half-rotate RoPE + KV append + GQA attention -> PostAttn
            (output projection, MLP, residuals).
* [NC-ROPE] same page, "mRoPE结论": the multi-section RoPE reduces to the plain
            1-D half-rotate RoPE with head_dim 128 and theta 1e6.
* [QTS-T]   rightkit-qts 0.2.0 docs, "Synthetic tests": cached/recompute
            equivalence is the property used to pin the decode path.
* [OV-CODEC] OmniVoice ARCHITECTURE, "Audio tokenizer pipeline": the decode path's RVQ
            decode (per-codebook embedding gather, project_out Linear with bias, sum).
* [NC-CODEC] ncnn Qwen3-TTS port, "Codec Decoder的切分": the codebook lookup and
            projections run before the codec body, projected and summed per frame.

Readings where the pages are silent (each listed in the design notes):
* RMSNorm is x / sqrt(mean(x^2) + eps) * g, eps inside the root, same eps for the
  q/k head norms.
* RoPE pairs dimension j with j + d/2 (rotate-half), omega_j = theta^(-2j/d), the
  angle is position * omega_j computed in float64.
* Attention scale is 1/sqrt(head_dim); query head h reads KV head h // (H/H_kv).
* Decode order: the new token's K/V are appended first, then it attends to
  positions 0..p inclusive.
* The audio embedding is an unweighted sum over codebooks (the pseudo-code's sum).
* The per-codebook head view is logits[k, t, v] = flat[t, k*V + v].
* The confidence is the max log-probability over non-mask classes, with the
  log-softmax normaliser taken over all V classes (mask class included).
* Top-n ties break towards the lower flat index f = k * T + t; argmax ties towards
  the lower class id.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64


def as64(a) -> np.ndarray:
    """Widen fp32 values (or bf16 values already widened to fp32) exactly to fp64."""
    return np.asarray(a, dtype=F64)


# ---------------------------------------------------------------------------
# Elementary steps
# ---------------------------------------------------------------------------

def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.  [OV-GGUF], [OV-IO]."""
    x = as64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * as64(g)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z)), the gate of the SwiGLU MLP.  [OV-IO]."""
    z = as64(z)
    return z / (1.0 + np.exp(-z))


def rope_omega(head_dim: int, theta: float) -> np.ndarray:
    """omega_j = theta^(-2j/d) for j < d/2.  [NC-ROPE], [OV-IO] (theta 1e6)."""
    j = np.arange(head_dim // 2, dtype=F64)
    return np.power(F64(theta), -2.0 * j / head_dim)


def rope(u: np.ndarray, pos, theta: float) -> np.ndarray:
    """Half-rotate RoPE on the last axis at position(s) ``pos``.  [NC-ATTN], [NC-ROPE].

    u has shape [..., d]; pos broadcasts against u.shape[:-1].  Dimension j is
    paired with j + d/2 and the pair is rotated by the angle pos * omega_j."""
    u = as64(u)
    d = u.shape[-1]
    half = d // 2
    ang = np.asarray(pos, dtype=F64)[..., None] * rope_omega(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = u[..., :half], u[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    s = as64(s)
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """GQA attention of the query heads of one token over L cached positions.

    q [H][d], K and V [L][H_kv][d] -> o [H][d].  Query head h reads KV head
    h // (H / H_kv); scores are q.k / sqrt(d); softmax over the L positions.
    [NC-ATTN] (GQA attention of the q_len=1 step), [OV-GGUF] (GQA 2:1)."""
    q, K, V = as64(q), as64(K), as64(V)
    H, d = q.shape
    Hkv = K.shape[1]
    group = H // Hkv
    o = np.empty((H, d), F64)
    for h in range(H):
        kv = h // group
        s = (K[:, kv, :] @ q[h]) / np.sqrt(d)
        p = softmax(s)
        o[h] = p @ V[:, kv, :]
    return o


def attention_full(Q: np.ndarray, K: np.ndarray, V: np.ndarray, causal: bool) -> np.ndarray:
    """Attention of S queries over S keys: Q [S][H][d], K,V [S][H_kv][d] -> [S][H][d].

    causal=False is the bidirectional attention of every MaskGIT step (no mask, no
    cache) [OV-MG]; causal=True is the recompute form of the decode path used to
    pin it [QTS-T]."""
    Q, K, V = as64(Q), as64(K), as64(V)
    S, H, d = Q.shape
    group = H // K.shape[1]
    O = np.empty((S, H, d), F64)
    for h in range(H):
        kv = h // group
        s = (Q[:, h, :] @ K[:, kv, :].T) / np.sqrt(d)
        if causal:
            s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
        O[:, h, :] = softmax(s, axis=-1) @ V[:, kv, :]
    return O


# ---------------------------------------------------------------------------
# Model description
# ---------------------------------------------------------------------------

@dataclass
class Dims:
    hidden: int = 1024
    n_heads: int = 16
    n_kv_heads: int = 8
    head_dim: int = 128
    ffn: int = 3072
    eps: float = 1e-6
    theta: float = 1e6


@dataclass
class Layer:
    """One decoder layer in fp64.  Linear weights are [out][in] (y = W x).  [OV-GGUF]."""
    attn_norm: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    q_norm: np.ndarray
    k_norm: np.ndarray
    wo: np.ndarray
    ffn_norm: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray

    @staticmethod
    def from_arrays(a: Dict[str, np.ndarray]) -> "Layer":
        return Layer(**{k: as64(a[k]) for k in Layer.__dataclass_fields__})


def qkv_heads(x: np.ndarray, L: Layer, dims: Dims, pos) -> Dict[str, np.ndarray]:
    """Pre-attention half of a layer for tokens x [T][hidden] at positions pos [T].

    input_layernorm -> q/k/v projections -> per-head q_norm/k_norm -> RoPE.
    [OV-IO] (per-head RMSNorm on Q and K before RoPE, no bias), [NC-ATTN] (PreRoPE
    outputs Q/K/V, then half-rotate RoPE)."""
    x = as64(x)
    T = x.shape[0]
    h = rms_norm(x, L.attn_norm, dims.eps)
    q = (h @ L.wq.T).reshape(T, dims.n_heads, dims.head_dim)
    k = (h @ L.wk.T).reshape(T, dims.n_kv_heads, dims.head_dim)
    v = (h @ L.wv.T).reshape(T, dims.n_kv_heads, dims.head_dim)
    qn = rms_norm(q, L.q_norm, dims.eps)
    kn = rms_norm(k, L.k_norm, dims.eps)
    p = np.asarray(pos, dtype=F64).reshape(T, 1)
    return dict(h=h, q_raw=q, k_raw=k, v=v, q=rope(qn, p, dims.theta), k=rope(kn, p, dims.theta))


def post_attention(x: np.ndarray, o: np.ndarray, L: Layer, dims: Dims) -> Dict[str, np.ndarray]:
    """Post-attention half: o_proj + residual, post_attention_layernorm, SwiGLU MLP
    down(silu(gate h) * up h) + residual.  [NC-ATTN] (PostAttn), [OV-IO] (SwiGLU)."""
    x = as64(x)
    T = x.shape[0]
    x1 = x + o.reshape(T, -1) @ L.wo.T
    h2 = rms_norm(x1, L.ffn_norm, dims.eps)
    m = silu(h2 @ L.w_gate.T) * (h2 @ L.w_up.T)
    x2 = x1 + m @ L.w_down.T
    return dict(x1=x1, h2=h2, m=m, x2=x2)


# ---------------------------------------------------------------------------
# Decode mode: q_len = 1 per stream, KV cache appended
# ---------------------------------------------------------------------------

class KVCache:
    """Per-layer, per-stream cache of rotated K and raw V, each [L][H_kv][d] fp64."""

    def __init__(self, n_layers: int, n_streams: int):
        self.k = [[None] * n_streams for _ in range(n_layers)]
        self.v = [[None] * n_streams for _ in range(n_layers)]

    def set(self, layer: int, b: int, k: np.ndarray, v: np.ndarray):
        self.k[layer][b] = as64(k)
        self.v[layer][b] = as64(v)

    def length(self, layer: int, b: int) -> int:
        kk = self.k[layer][b]
        return 0 if kk is None else kk.shape[0]


def decode_layer(x: np.ndarray, pos: Sequence[int], cache: KVCache, li: int, L: Layer,
                 dims: Dims, record: Optional[Dict] = None) -> np.ndarray:
    """One layer of the q_len=1 decode step for B independent streams.

    Stream b's token sits at position pos[b] (= tokens already cached); its rotated
    K and V are appended to the cache, then it attends to positions 0..pos[b].
    [NC-ATTN] (RoPE + KV append + GQA attention per layer)."""
    x = as64(x)
    B = x.shape[0]
    st = qkv_heads(x, L, dims, pos)
    o = np.empty((B, dims.n_heads, dims.head_dim), F64)
    for b in range(B):
        if cache.length(li, b) != pos[b]:
            raise ValueError("cache length of stream %d is %d, position is %d"
                             % (b, cache.length(li, b), pos[b]))
        kb = st["k"][b][None] if cache.k[li][b] is None else \
            np.concatenate([cache.k[li][b], st["k"][b][None]], axis=0)
        vb = st["v"][b][None] if cache.v[li][b] is None else \
            np.concatenate([cache.v[li][b], st["v"][b][None]], axis=0)
        cache.set(li, b, kb, vb)
        o[b] = attend(st["q"][b], kb, vb)
    post = post_attention(x, o, L, dims)
    if record is not None:
        record.update(st)
        record["o"] = o
        record.update(post)
    return post["x2"]


def prefill_layer(x: np.ndarray, p0: int, cache: KVCache, b: int, li: int, L: Layer, dims: Dims) -> np.ndarray:
    """One layer of a causal multi-token prefill of stream b: S tokens at positions
    p0..p0+S-1 (p0 = tokens already cached).  All S rotated K and V are appended, then
    token i attends to positions 0..p0+i.  [NC-ATTN] (RoPE + KV append + GQA attention),
    [OV-MG] (the Talker prompt is a prefill; causal, unlike the MaskGIT passes)."""
    x = as64(x)
    S = x.shape[0]
    if cache.length(li, b) != p0:
        raise ValueError("cache length of stream %d is %d, p0 is %d" % (b, cache.length(li, b), p0))
    st = qkv_heads(x, L, dims, np.arange(p0, p0 + S))
    kb = st["k"] if cache.k[li][b] is None else np.concatenate([cache.k[li][b], st["k"]], axis=0)
    vb = st["v"] if cache.v[li][b] is None else np.concatenate([cache.v[li][b], st["v"]], axis=0)
    cache.set(li, b, kb, vb)
    o = np.empty((S, dims.n_heads, dims.head_dim), F64)
    for i in range(S):
        o[i] = attend(st["q"][i], kb[:p0 + i + 1], vb[:p0 + i + 1])
    return post_attention(x, o, L, dims)["x2"]


def prefill(x: np.ndarray, p0: int, cache: KVCache, b: int, layers: List[Layer], dims: Dims) -> np.ndarray:
    """All layers of a causal prefill of S tokens of stream b; returns the residual stream."""
    for li, L in enumerate(layers):
        x = prefill_layer(x, p0, cache, b, li, L, dims)
    return x


def decode_step(x: np.ndarray, pos: Sequence[int], cache: KVCache, layers: List[Layer],
                dims: Dims, record_layer: Optional[int] = None,
                record: Optional[Dict] = None) -> np.ndarray:
    """All layers of one decode step; returns the residual stream after the last layer."""
    for li, L in enumerate(layers):
        x = decode_layer(x, pos, cache, li, L, dims,
                         record if (record is not None and li == record_layer) else None)
    return x


def head_logits(x: np.ndarray, final_norm: np.ndarray, head: np.ndarray, eps: float):
    """Final RMSNorm (llm.norm) then a bias-free head: y = norm(x); logits = y H^T.
    [OV-GGUF] (llm.norm), [OV-IO] (audio_heads Linear, no bias), [NC-ARCH]
    (Talker first-codebook head, predictor heads)."""
    y = rms_norm(x, final_norm, eps)
    return y, y @ as64(head).T


def argmax_groups(logits: np.ndarray, n_groups: int, group_vocab: int) -> np.ndarray:
    """Greedy choice per group of ``group_vocab`` classes; ties to the lower class id."""
    lg = as64(logits).reshape(logits.shape[0], n_groups, group_vocab)
    return np.argmax(lg, axis=-1).astype(np.int32)  # numpy returns the first maximum


# ---------------------------------------------------------------------------
# Input embedding
# ---------------------------------------------------------------------------

def codebook_embed(codes: np.ndarray, tables, cb_vocab: int) -> np.ndarray:
    """Sum over codebooks k of row k*V + code[., k] of the flattened table.

    codes [R][K] int; tables indexable by row ids (the flattened [K*V][hidden]
    table).  [OV-IO] (offsets = arange(K) * 1025, sum over codebooks), [NC-ARCH]
    (the 16 codebook embeddings are summed into the next Talker input)."""
    codes = np.asarray(codes, dtype=np.int64)
    R, K = codes.shape
    out = None
    for k in range(K):
        rows = as64(tables[k * cb_vocab + codes[:, k]])
        out = rows if out is None else out + rows
    return out


def hybrid_embed(text_ids: np.ndarray, text_table, codes_kt: np.ndarray, audio_table,
                 cb_vocab: int) -> np.ndarray:
    """MaskGIT input: text rows take the text embedding, audio frames take the codebook
    sum (``where(audio_mask, audio_emb, text_emb)``).  [OV-IO].

    text_ids [n_text]; codes_kt [K][n_frames] (mask id included as a code)."""
    text = as64(text_table[np.asarray(text_ids, dtype=np.int64)])
    audio = codebook_embed(np.asarray(codes_kt).T, audio_table, cb_vocab)
    return np.concatenate([text, audio], axis=0)


# ---------------------------------------------------------------------------
# MaskGIT mode: full bidirectional pass, per-codebook heads, scoring and selection
# ---------------------------------------------------------------------------

def backbone_full(x: np.ndarray, layers: List[Layer], dims: Dims, causal: bool = False,
                  record_layer: Optional[int] = None, record: Optional[Dict] = None):
    """All layers over a whole sequence at positions 0..S-1 with no cache.  [OV-MG]."""
    x = as64(x)
    S = x.shape[0]
    pos = np.arange(S)
    for li, L in enumerate(layers):
        st = qkv_heads(x, L, dims, pos)
        o = attention_full(st["q"], st["k"], st["v"], causal)
        post = post_attention(x, o, L, dims)
        if record is not None and li == record_layer:
            record.update(st)
            record["o"] = o
            record.update(post)
        x = post["x2"]
    return x


def maskgit_scores(logits_flat: np.ndarray, codes_kt: np.ndarray, n_cb: int, cb_vocab: int,
                   mask_id: int, layer_penalty: float):
    """Per-codebook log-softmax, mask class excluded, argmax and confidence.  [OV-MG].

    logits_flat [T][K*V] -> view [K][T][V] (logits[k, t, v] = flat[t, k*V + v]).
    lp = logits - logsumexp over all V classes; lp[mask] = -inf; pred = argmax lp;
    conf = max lp - k * layer_penalty; conf = -inf where the code is already set."""
    T = logits_flat.shape[0]
    lg = as64(logits_flat).reshape(T, n_cb, cb_vocab).transpose(1, 0, 2)
    m = np.max(lg, axis=-1, keepdims=True)
    lse = m + np.log(np.sum(np.exp(lg - m), axis=-1, keepdims=True))
    lp = lg - lse
    lp[:, :, mask_id] = -np.inf
    pred = np.argmax(lp, axis=-1).astype(np.int32)
    best = np.max(lp, axis=-1)
    conf = best - np.arange(n_cb, dtype=F64)[:, None] * layer_penalty
    conf = np.where(np.asarray(codes_kt) == mask_id, conf, -np.inf)
    return pred, conf, lp


def select_top(conf_flat: np.ndarray, n: int) -> np.ndarray:
    """The n highest scores of the flattened [K*T] array, in decreasing order, ties to
    the lower flat index; entries at -inf are never picked (their slot holds -1).
    [OV-MG] (topk over score.flatten())."""
    conf_flat = as64(conf_flat).reshape(-1)
    order = np.argsort(-conf_flat, kind="stable")  # stable: equal scores keep index order
    picked = np.full(n, -1, np.int32)
    for r in range(min(n, order.size)):
        f = order[r]
        if conf_flat[f] > -np.inf:
            picked[r] = f
    return picked


def apply_picks(codes_kt: np.ndarray, pred: np.ndarray, picked: np.ndarray) -> np.ndarray:
    """tokens[topk_idx] = pred[topk_idx] on the flattened codes.  [OV-MG]."""
    c = np.array(codes_kt, dtype=np.int32).reshape(-1)
    p = np.asarray(pred).reshape(-1)
    for f in picked:
        if f >= 0:
            c[f] = p[f]
    return c.reshape(np.asarray(codes_kt).shape)


def cfg_logits(cond: np.ndarray, uncond: np.ndarray, cfg_scale: float) -> np.ndarray:
    """Classifier-free guidance on the logits, before the log-softmax:
    c + s * (c - u).  [OV-MG] (CFG: log_softmax(c + cfg_scale * (c - u)))."""
    c = as64(cond)
    return c + float(cfg_scale) * (c - as64(uncond))


def gumbel(u: np.ndarray) -> np.ndarray:
    """Standard Gumbel variate from a uniform in (0, 1): -log(-log u).  [OV-MG]
    (gumbel_sample; the uniforms are the caller's, drawn from its Philox stream)."""
    return -np.log(-np.log(as64(u)))


def keep_top_k_ratio(lp: np.ndarray, ratio: float) -> np.ndarray:
    """Keep the floor(ratio * V) (at least 1) largest entries of each row, ties to the lower
    class id; the others become -inf.  [OV-MG] (keep_top_k_ratio(log_probs, 0.1))."""
    lp = np.ascontiguousarray(as64(lp))
    V = lp.shape[-1]
    k = max(1, int(np.floor(ratio * V)))
    out = np.full(lp.shape, -np.inf)  # C-contiguous, so the row view below writes into it
    flat = lp.reshape(-1, V)
    of = out.reshape(-1, V)
    for r in range(flat.shape[0]):
        order = sorted(range(V), key=lambda v: (-flat[r, v], v))  # larger first, then lower id
        for v in order[:k]:
            of[r, v] = flat[r, v]
    return out


def sample_scores(logits_flat: np.ndarray, codes_kt: np.ndarray, n_cb: int, cb_vocab: int, mask_id: int,
                  layer_penalty: float, class_temp: float, pos_temp: float, top_k_ratio: float,
                  u_class: Optional[np.ndarray], u_pos: Optional[np.ndarray]):
    """Scoring with the sampler's temperatures.  [OV-MG], in the listing's order, each step
    acting on the log-probs in place:
      lp = log_softmax(logits) over all V classes; lp[mask] = -inf;
      if class_temp > 0: lp = keep_top_k_ratio(lp, ratio); lp = lp / class_temp + G(u_class);
      pred = argmax lp; score = max lp - k * layer_penalty;
      if pos_temp > 0: score += pos_temp * G(u_pos);
      score = -inf where the code is already set.
    u_class [K][T][V] and u_pos [K][T] are uniforms in (0, 1); G(u) = -log(-log u)."""
    T = logits_flat.shape[0]
    lg = as64(logits_flat).reshape(T, n_cb, cb_vocab).transpose(1, 0, 2)
    m = np.max(lg, axis=-1, keepdims=True)
    lp = lg - (m + np.log(np.sum(np.exp(lg - m), axis=-1, keepdims=True)))
    lp[:, :, mask_id] = -np.inf
    if class_temp > 0:
        lp = keep_top_k_ratio(lp, top_k_ratio)
        lp = lp / class_temp + gumbel(u_class)  # -inf stays -inf
    pred = np.argmax(lp, axis=-1).astype(np.int32)
    score = np.max(lp, axis=-1) - np.arange(n_cb, dtype=F64)[:, None] * layer_penalty
    if pos_temp > 0:
        score = score + pos_temp * gumbel(u_pos)
    score = np.where(np.asarray(codes_kt) == mask_id, score, -np.inf)
    return pred, score, lp


def unmask_schedule(n_total: int, n_steps: int) -> List[int]:
    """How many positions each step unmasks.  [OV-MG] gives the form
    ceil(N * (t[i+1] - t[i])) over a time grid; the grid used here is the cosine
    schedule t_i = 1 - cos(pi/2 * i / n_steps) (the MaskGIT paper's, which the page
    cites in its glossary).  Each count is capped at what is still masked and the
    last step takes the remainder, so the counts sum to N."""
    t = [1.0 - np.cos(0.5 * np.pi * i / n_steps) for i in range(n_steps + 1)]
    out, left = [], n_total
    for i in range(n_steps):
        if i == n_steps - 1:
            n = left
        else:
            n = min(left, int(np.ceil(n_total * (t[i + 1] - t[i]))))
        out.append(n)
        left -= n
    return out


def maskgit_pass(text_ids, text_table, codes_kt, audio_table, audio_heads, layers: List[Layer],
                 final_norm, dims: Dims, cb_vocab: int, mask_id: int, layer_penalty: float,
                 n_unmask: int, record: Optional[Dict] = None):
    """One MaskGIT step: embed, full bidirectional backbone, final norm on the audio
    window, per-codebook heads, scoring, top-n selection, token update.  [OV-IO],
    [OV-MG] (each step is a full prefill; logits are read on the audio window only,
    as the page's inner-loop narrowing does)."""
    codes_kt = np.asarray(codes_kt, dtype=np.int32)
    n_cb, T = codes_kt.shape
    n_text = len(text_ids)
    x = hybrid_embed(text_ids, text_table, codes_kt, audio_table, cb_vocab)
    x = backbone_full(x, layers, dims, causal=False)
    y, logits = head_logits(x[n_text:], final_norm, audio_heads, dims.eps)
    pred, conf, _ = maskgit_scores(logits, codes_kt, n_cb, cb_vocab, mask_id, layer_penalty)
    picked = select_top(conf.reshape(-1), n_unmask)
    new_codes = apply_picks(codes_kt, pred, picked)
    if record is not None:
        record.update(x=x, y=y, logits=logits, pred=pred, conf=conf, picked=picked)
    return new_codes, pred, conf, picked


def maskgit_pass_cfg(text_ids, text_table, codes_kt, n_target: int, audio_table, audio_heads,
                     layers: List[Layer], final_norm, dims: Dims, cb_vocab: int, mask_id: int,
                     layer_penalty: float, n_unmask: int, cfg_scale: float,
                     record: Optional[Dict] = None):
    """One MaskGIT step with classifier-free guidance.  [OV-MG]:
    * the conditional prompt is the full sequence (text rows, then every audio frame,
      the last n_target of which are the target window); its logits are read on the
      window (the last n_target positions);
    * the unconditional prompt is the target window's tokens alone (no text, no
      reference frames), at positions 0..n_target-1; its logits are read on all of it;
    * guided logits c + s (c - u), then the scoring, selection and token update of the
      plain step, all restricted to the window.
    codes_kt [K][n_frames] is updated in place on the window only; pred / conf are
    [K][n_target] and picked indexes the flattened window (k * n_target + t)."""
    codes_kt = np.asarray(codes_kt, dtype=np.int32)
    n_cb, n_frames = codes_kt.shape
    n_text = len(text_ids)
    w0 = n_frames - n_target
    window = codes_kt[:, w0:]
    xc = backbone_full(hybrid_embed(text_ids, text_table, codes_kt, audio_table, cb_vocab), layers, dims)
    _, lc = head_logits(xc[n_text + w0:], final_norm, audio_heads, dims.eps)
    xu = backbone_full(codebook_embed(window.T, audio_table, cb_vocab), layers, dims)
    _, lu = head_logits(xu, final_norm, audio_heads, dims.eps)
    guided = cfg_logits(lc, lu, cfg_scale)
    pred, conf, _ = maskgit_scores(guided, window, n_cb, cb_vocab, mask_id, layer_penalty)
    picked = select_top(conf.reshape(-1), n_unmask)
    new_codes = codes_kt.copy()
    new_codes[:, w0:] = apply_picks(window, pred, picked)
    if record is not None:
        record.update(logits_c=lc, logits_u=lu, guided=guided, pred=pred, conf=conf, picked=picked)
    return new_codes, pred, conf, picked


def maskgit_step(text_ids, text_table, codes_kt, n_target: int, audio_table, audio_heads,
                 layers: List[Layer], final_norm, dims: Dims, cb_vocab: int, mask_id: int,
                 layer_penalty: float, n_unmask: int, cfg_scale: float = 0.0, class_temp: float = 0.0,
                 pos_temp: float = 0.0, top_k_ratio: float = 0.1, u_class=None, u_pos=None,
                 record: Optional[Dict] = None):
    """One MaskGIT step in the general form of [OV-MG]: the conditional prompt (with an
    unconditional pass on the target window and guided logits when cfg_scale != 0),
    the sampler's scoring (temperatures, top-k ratio, Gumbel noise from the given
    uniforms), top-n selection and the update of the window.  With cfg_scale = 0 the
    unconditional pass is skipped (its weight is zero)."""
    codes_kt = np.asarray(codes_kt, dtype=np.int32)
    n_cb, n_frames = codes_kt.shape
    n_text = len(text_ids)
    w0 = n_frames - n_target
    window = codes_kt[:, w0:]
    xc = backbone_full(hybrid_embed(text_ids, text_table, codes_kt, audio_table, cb_vocab), layers, dims)
    _, lc = head_logits(xc[n_text + w0:], final_norm, audio_heads, dims.eps)
    lu = None
    if cfg_scale != 0.0:
        xu = backbone_full(codebook_embed(window.T, audio_table, cb_vocab), layers, dims)
        _, lu = head_logits(xu, final_norm, audio_heads, dims.eps)
        guided = cfg_logits(lc, lu, cfg_scale)
    else:
        guided = lc
    pred, conf, lp = sample_scores(guided, window, n_cb, cb_vocab, mask_id, layer_penalty, class_temp, pos_temp,
                                   top_k_ratio, u_class, u_pos)
    picked = select_top(conf.reshape(-1), n_unmask)
    new_codes = codes_kt.copy()
    new_codes[:, w0:] = apply_picks(window, pred, picked)
    if record is not None:
        record.update(logits_c=lc, logits_u=lu, guided=guided, lp=lp, pred=pred, conf=conf, picked=picked)
    return new_codes, pred, conf, picked


# ---------------------------------------------------------------------------
# Codec RVQ decode (the fourth NEXT row)
# ---------------------------------------------------------------------------

def rvq_decode(codes_qt: np.ndarray, embed: np.ndarray, proj_w: np.ndarray, proj_b: np.ndarray) -> np.ndarray:
    """Residual-VQ decode of the codec's quantizer: for each codebook k, gather the code's
    codebook_dim-wide embedding, project it with project_out[k] (W [out][dim], bias
    [out]) and sum over the codebooks.  [OV-CODEC] (RVQ decode: e_k = embed_k[codes[k]],
    p_k = e_k W_k^T + b_k, out += p_k), [NC-CODEC] (codebook lookup per frame, projected
    and summed before the codec body).

    codes_qt int [Q][T]; embed [Q][codebook_size][dim]; proj_w [Q][out][dim];
    proj_b [Q][out] -> [T][out] (the page then views it as [out][T] for the convolutions)."""
    codes_qt = np.asarray(codes_qt, dtype=np.int64)
    Q, T = codes_qt.shape
    out = None
    for k in range(Q):
        e = as64(embed[k])[codes_qt[k]]              # [T][dim]
        p = e @ as64(proj_w[k]).T + as64(proj_b[k])  # [T][out]
        out = p if out is None else out + p
    return out
