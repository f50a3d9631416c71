"""bf16-storage emulation of the backbone: the oracle's fp64 arithmetic with the values
that the bf16 mode of the HIP path stores in bf16 rounded to bf16 at the same points.

TEST INFRASTRUCTURE (not the oracle).  The oracle (``oracle/backbone.py``) is the exact
definition; this module answers a different question: how far does bf16 storage alone,
with exact arithmetic everywhere else, move the result?  Two uses:

* ``emulated vs oracle`` measures what bf16 storage does to a deep stack (a CPU test pins
  that figure for the batch-1 decode workload), which is why a 28-layer bf16 output
  cannot sit within the single-layer 2e-2 bound of the exact result;
* ``GPU vs emulated`` leaves only fp32-versus-fp64 arithmetic between the two sides (the
  bf16 roundings are the same), so the GPU's stacks are held to a tight bound against it.

Rounding points (bf16 mode of the library, as its header states: weights, tables, heads,
KV cache and every product operand in bf16; residual stream, accumulations, norms and
softmax statistics in fp32):
* the RMSNorm outputs that feed a product (input_layernorm, post_attention_layernorm,
  the final norm before a head);
* the new token's rotated K and its V when they enter the cache (decode), and in the
  MaskGIT pass the rotated q, the rotated K and V that the attention reads;
* the attention output (the o-projection's operand) and the SwiGLU output (the
  down-projection's operand);
* in the MaskGIT attention, each probability weight that multiplies V, taken relative to
  the running reference maximum of the kernel's online softmax (``flash_attention``);
  the normaliser sums the unrounded weights.
The decode attention keeps q and its weights in fp32 (no rounding there).  A prefill of
more than 64 tokens runs on the causal form of the MaskGIT attention kernel: bf16 q and
weights as there (``prefill``).
Values are rounded as the GPU does: the fp64 value to fp32, then to bf16 by round to
nearest even.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from oracle import backbone as O
from workload import gen


def r16(a) -> np.ndarray:
    """fp64 values -> fp32 -> bf16 (round to nearest even) -> fp64 (finite inputs)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32).astype(np.float64)


def decode_layer(x, pos: Sequence[int], cache: O.KVCache, li: int, L: O.Layer, dims: O.Dims,
                 record: Optional[dict] = None) -> np.ndarray:
    """One q_len = 1 decode layer of B streams with the bf16 storage of the decode path."""
    x = np.asarray(x, np.float64)
    B = x.shape[0]
    h = r16(O.rms_norm(x, L.attn_norm, dims.eps))
    q = (h @ L.wq.T).reshape(B, dims.n_heads, dims.head_dim)
    k = (h @ L.wk.T).reshape(B, dims.n_kv_heads, dims.head_dim)
    v = (h @ L.wv.T).reshape(B, dims.n_kv_heads, dims.head_dim)
    p = np.asarray(pos, np.float64).reshape(B, 1)
    q = O.rope(O.rms_norm(q, L.q_norm, dims.eps), p, dims.theta)           # fp32 on the GPU
    k = r16(O.rope(O.rms_norm(k, L.k_norm, dims.eps), p, dims.theta))      # into the bf16 cache
    v = r16(v)
    o = np.empty((B, dims.n_heads, dims.head_dim))
    for b in range(B):
        if cache.length(li, b) != pos[b]:
            raise ValueError("cache length of stream %d is %d, position is %d" % (b, cache.length(li, b), pos[b]))
        kb = k[b][None] if cache.k[li][b] is None else np.concatenate([cache.k[li][b], k[b][None]], axis=0)
        vb = v[b][None] if cache.v[li][b] is None else np.concatenate([cache.v[li][b], v[b][None]], axis=0)
        cache.set(li, b, kb, vb)
        o[b] = O.attend(q[b], kb, vb)
    o = r16(o.reshape(B, -1))
    x1 = x + o @ L.wo.T
    h2 = r16(O.rms_norm(x1, L.ffn_norm, dims.eps))
    m = r16(O.silu(h2 @ L.w_gate.T) * (h2 @ L.w_up.T))
    x2 = x1 + m @ L.w_down.T
    if record is not None:
        record.update(h=h, q=q, k=k, v=v, o=o, x1=x1, h2=h2, m=m, x2=x2)
    return x2


def decode_step(x, pos: Sequence[int], cache: O.KVCache, layers: List[O.Layer], dims: O.Dims) -> np.ndarray:
    for li, L in enumerate(layers):
        x = decode_layer(x, pos, cache, li, L, dims)
    return x


def head_logits(x, final_norm, head, eps: float):
    """Final RMSNorm rounded to bf16 (the head's operand), then the head in fp64."""
    y = r16(O.rms_norm(x, final_norm, eps))
    return y, y @ np.asarray(head, np.float64).T


def flash_attention(Q, K, V, round_p: bool = True, quarters: int = 4, block: int = 32, tile: int = 32,
                    lazy: float = 8.0) -> np.ndarray:
    """Bidirectional attention as the MaskGIT attention kernel accumulates it.

    Q [S][H][d] and K, V [S][Hkv][d] hold bf16 values; query head h reads KV head
    h // (H / Hkv).  Keys come in blocks of ``block``; the blocks are dealt to ``quarters``
    contiguous ranges, each with its own online-softmax state; the queries of one head
    form tiles of ``tile`` that share the decision to raise the reference maximum: a
    tile's references are raised (each query's to its running maximum, in log2 units)
    only when some query of the tile sees a block maximum more than ``lazy`` above its
    reference.  A weight p = 2^(s log2(e)/sqrt(d) - reference of its block) multiplies V
    rounded to bf16 (``round_p``), the normaliser sums the unrounded weights, and every
    partial sum is carried to the final reference by the factor 2^(reference - final)
    (the kernel's rescales, and the merge of the quarters relative to the largest
    reference; fp32 factors there, exact here).  In exact
    arithmetic (round_p False) every choice above cancels: plain softmax attention."""
    Q, K, V = (np.asarray(a, np.float64) for a in (Q, K, V))
    S, H, d = Q.shape
    group = H // K.shape[1]
    c = np.log2(np.e) / np.sqrt(d)
    NB = (S + block - 1) // block
    NBQ = (NB + quarters - 1) // quarters
    nt = (S + tile - 1) // tile
    Sp = nt * tile
    out = np.empty((S, H, d))
    for h in range(H):
        kv = h // group
        qh = np.empty((Sp, d))
        qh[:S] = Q[:, h]
        qh[S:] = Q[S - 1, h]                     # past the sequence: copies of the last query
        s = (qh @ K[:, kv].T) * c                # [Sp][S], log2 units
        ref = np.empty((Sp, S))                  # reference of each weight
        m_fin = np.full((Sp, quarters), -np.inf)
        for qq in range(quarters):
            first = qq * NBQ
            m = np.full((nt, tile), -np.inf)
            for i in range(max(0, min(NBQ, NB - first))):
                k0 = (first + i) * block
                k1 = min(S, k0 + block)
                mx = s[:, k0:k1].max(axis=1).reshape(nt, tile)
                raise_ = np.any(mx > m + lazy, axis=1)   # per tile
                m = np.where(raise_[:, None], np.maximum(m, mx), m)
                ref[:, k0:k1] = m.reshape(Sp, 1)
            m_fin[:, qq] = m.reshape(Sp)
        M = m_fin.max(axis=1, keepdims=True)     # quarter 0 always holds keys: finite
        p = np.exp2(s - ref)
        carry = np.exp2(ref - M)
        l = np.sum(p * carry, axis=1)
        pw = r16(p) if round_p else p
        o = (pw * carry) @ V[:, kv]
        out[:, h] = (o / l[:, None])[:S]
    return out


def flash_attention_causal(Q, K, V, p0: int, round_p: bool = True, quarters: int = 4, block: int = 32,
                           tile: int = 32, lazy: float = 8.0) -> np.ndarray:
    """The causal form of the same kernel (the prefill): query row i is at position p0 + i
    and sees keys [0, p0 + i] of K, V [p0 + S][Hkv][d].  Each tile of ``tile`` queries
    takes the keys below p0 + (first query) + tile in blocks of ``block``, dealt to the
    quarters as above (so the quarters' ranges depend on the tile); keys a query must not
    see get the score -inf before the block maximum.  In exact arithmetic (round_p False)
    this is plain causal softmax attention."""
    Q, K, V = (np.asarray(a, np.float64) for a in (Q, K, V))
    S, H, d = Q.shape
    group = H // K.shape[1]
    c = np.log2(np.e) / np.sqrt(d)
    out = np.empty((S, H, d))
    for t0 in range(0, S, tile):
        rows = np.arange(t0, min(S, t0 + tile))
        qrows = np.minimum(np.arange(t0, t0 + tile), S - 1)   # past the sequence: copies of the last
        ke = min(p0 + S, p0 + t0 + tile)
        NB = (ke + block - 1) // block
        NBQ = (NB + quarters - 1) // quarters
        keys = np.arange(ke)
        visible = keys[None, :] <= (p0 + np.arange(t0, t0 + tile))[:, None]   # [tile][ke]
        for h in range(H):
            kv = h // group
            s = np.where(visible, (Q[qrows, h] @ K[:ke, kv].T) * c, -np.inf)
            ref = np.full((tile, ke), -np.inf)
            m_fin = np.full((tile, quarters), -np.inf)
            for qq in range(quarters):
                first = qq * NBQ
                m = np.full(tile, -np.inf)
                for i in range(max(0, min(NBQ, NB - first))):
                    k0 = (first + i) * block
                    k1 = min(ke, k0 + block)
                    mx = s[:, k0:k1].max(axis=1)
                    if np.any(mx > m + lazy):
                        m = np.maximum(m, mx)
                    ref[:, k0:k1] = m[:, None]
                m_fin[:, qq] = m
            M = m_fin.max(axis=1, keepdims=True)     # quarter 0 holds key 0: finite
            with np.errstate(invalid="ignore"):
                p = np.where(visible, np.exp2(s - ref), 0.0)
                carry = np.where(np.isfinite(ref), np.exp2(ref - M), 0.0)
            l = np.sum(p * carry, axis=1)
            pw = r16(p) if round_p else p
            o = (pw * carry) @ V[:ke, kv]
            out[rows, h] = (o / l[:, None])[:len(rows)]
    return out


def prefill(x, p0: int, cache: O.KVCache, stream: int, layers: List[O.Layer], dims: O.Dims,
            round_p: bool = True) -> np.ndarray:
    """A prefill of more than 64 tokens on the causal flash path: tokens at positions
    p0 .. p0 + S - 1 after the cached prefix of `stream` (bf16 values), with q, the new K
    and V, the attention output, the norms' outputs and the SwiGLU output rounded to
    bf16, and the attention accumulated as flash_attention_causal.  Appends the new K, V
    to the cache."""
    x = np.asarray(x, np.float64)
    S = x.shape[0]
    pos = (p0 + np.arange(S, dtype=np.float64)).reshape(S, 1)
    for li, L in enumerate(layers):
        h = r16(O.rms_norm(x, L.attn_norm, dims.eps))
        q = (h @ L.wq.T).reshape(S, dims.n_heads, dims.head_dim)
        k = (h @ L.wk.T).reshape(S, dims.n_kv_heads, dims.head_dim)
        v = (h @ L.wv.T).reshape(S, dims.n_kv_heads, dims.head_dim)
        q = r16(O.rope(O.rms_norm(q, L.q_norm, dims.eps), pos, dims.theta))
        k = r16(O.rope(O.rms_norm(k, L.k_norm, dims.eps), pos, dims.theta))
        v = r16(v)
        if cache.length(li, stream) != p0:
            raise ValueError("cache length %d, prefill position %d" % (cache.length(li, stream), p0))
        kp, vp = cache.k[li][stream], cache.v[li][stream]
        K = k if kp is None else np.concatenate([kp, k], axis=0)
        Vv = v if vp is None else np.concatenate([vp, v], axis=0)
        cache.set(li, stream, K, Vv)
        o = r16(flash_attention_causal(q, K, Vv, p0, round_p=round_p).reshape(S, -1))
        x1 = x + o @ L.wo.T
        h2 = r16(O.rms_norm(x1, L.ffn_norm, dims.eps))
        m = r16(O.silu(h2 @ L.w_gate.T) * (h2 @ L.w_up.T))
        x = x1 + m @ L.w_down.T
    return x


def backbone_full(x, layers: List[O.Layer], dims: O.Dims, record_layer: Optional[int] = None,
                  record: Optional[dict] = None, round_p: bool = True) -> np.ndarray:
    """All layers of the MaskGIT pass (bidirectional, positions 0..S-1) with the bf16
    storage of that path."""
    x = np.asarray(x, np.float64)
    S = x.shape[0]
    pos = np.arange(S, dtype=np.float64).reshape(S, 1)
    for li, L in enumerate(layers):
        h = r16(O.rms_norm(x, L.attn_norm, dims.eps))
        q = (h @ L.wq.T).reshape(S, dims.n_heads, dims.head_dim)
        k = (h @ L.wk.T).reshape(S, dims.n_kv_heads, dims.head_dim)
        v = (h @ L.wv.T).reshape(S, dims.n_kv_heads, dims.head_dim)
        q = r16(O.rope(O.rms_norm(q, L.q_norm, dims.eps), pos, dims.theta))
        k = r16(O.rope(O.rms_norm(k, L.k_norm, dims.eps), pos, dims.theta))
        v = r16(v)
        o = r16(flash_attention(q, k, v, round_p=round_p).reshape(S, -1))
        x1 = x + o @ L.wo.T
        h2 = r16(O.rms_norm(x1, L.ffn_norm, dims.eps))
        m = r16(O.silu(h2 @ L.w_gate.T) * (h2 @ L.w_up.T))
        x2 = x1 + m @ L.w_down.T
        if record is not None and li == record_layer:
            record.update(h=h, q=q, k=k, v=v, o=o, x1=x1, h2=h2, m=m, x2=x2)
        x = x2
    return x


def maskgit_logits(text_ids, text_table, codes_kt, audio_table, audio_heads, layers, final_norm,
                   dims: O.Dims, cb_vocab: int):
    """Embedding (exact: the GPU sums in double and rounds once), emulated layers, the
    final norm on the audio window and the heads.  Returns (x after the layers, y, logits)."""
    n_text = len(text_ids)
    x = O.hybrid_embed(text_ids, text_table, codes_kt, audio_table, cb_vocab)
    x = np.asarray(x, np.float32).astype(np.float64)   # the residual stream starts in fp32
    x = backbone_full(x, layers, dims)
    y, logits = head_logits(x[n_text:], final_norm, audio_heads, dims.eps)
    return x, y, logits
