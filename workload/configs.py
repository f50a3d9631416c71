"""The five synthetic workloads of the TTS backbone and how their inputs are drawn.

Shapes follow the Qwen3-0.6B-shaped backbone described on the pages (OmniVoice
ARCHITECTURE, "GGUF layout" and "Qwen3 0.6B backbone with custom IO"; the ncnn
Qwen3-TTS port, "模型结构拆解"): 28 layers, hidden 1024, 16 query / 8 KV heads of
128, SwiGLU 3072, RMSNorm eps 1e-6, RoPE theta 1e6.

Every tensor is drawn from the counter-based generator in ``workload.gen`` under a
stream id (kind, index), so the same element can be produced anywhere.  This module
holds no model arithmetic.

Conventions
-----------
* Linear weights are row-major ``[out][in]``; N(0, 0.02^2).
* Norm gains are fp32: all ones (``gains="ones"``, the workloads' setting) or
  1 + N(0, 0.1^2) (``gains="random"``, used by tests so that a dropped gain shows).
* bf16 tensors are handled as uint16 bit patterns on the host.
* A KV-cache prefill is "already normalised and rotated K" and raw V, N(0, 1).
  Element (layer l, stream b, position p, kv head h, dim d) of K is element
  ``((b * KV_POS_STRIDE + p) * n_kv + h) * head_dim + d`` of stream (K_CACHE, l).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from . import gen
from .gen import stream_id

KV_POS_STRIDE = 8192  # logical positions reserved per decode stream (index space only)
PAGE = 16             # tokens per KV page


@dataclass
class Shape:
    n_layers: int = 28
    hidden: int = 1024
    n_heads: int = 16
    n_kv_heads: int = 8
    head_dim: int = 128
    ffn: int = 3072
    eps: float = 1e-6
    theta: float = 1e6


WEIGHT_KINDS = {
    # name: (kind, rows, cols) as functions of the shape
    "wq": (gen.KIND_WQ, lambda s: s.n_heads * s.head_dim, lambda s: s.hidden),
    "wk": (gen.KIND_WK, lambda s: s.n_kv_heads * s.head_dim, lambda s: s.hidden),
    "wv": (gen.KIND_WV, lambda s: s.n_kv_heads * s.head_dim, lambda s: s.hidden),
    "wo": (gen.KIND_WO, lambda s: s.hidden, lambda s: s.n_heads * s.head_dim),
    "w_gate": (gen.KIND_W_GATE, lambda s: s.ffn, lambda s: s.hidden),
    "w_up": (gen.KIND_W_UP, lambda s: s.ffn, lambda s: s.hidden),
    "w_down": (gen.KIND_W_DOWN, lambda s: s.hidden, lambda s: s.ffn),
}
GAIN_KINDS = {
    "attn_norm": (gen.KIND_ATTN_NORM, lambda s: s.hidden),
    "q_norm": (gen.KIND_Q_NORM, lambda s: s.head_dim),
    "k_norm": (gen.KIND_K_NORM, lambda s: s.head_dim),
    "ffn_norm": (gen.KIND_FFN_NORM, lambda s: s.hidden),
}


def layer_weights(seed: int, shape: Shape, layer: int, bf16: bool, gains: str = "ones",
                  std: float = 0.02) -> Dict[str, np.ndarray]:
    """All tensors of one layer: linear weights (fp32, or bf16 bits) and fp32 gains."""
    out = {}
    for name, (kind, rows, cols) in WEIGHT_KINDS.items():
        out[name] = gen.fast_normal(seed, stream_id(kind, layer), (rows(shape), cols(shape)),
                                    std=std, bf16=bf16)
    for name, (kind, n) in GAIN_KINDS.items():
        out[name] = gen.gains(seed, stream_id(kind, layer), n(shape), gains)
    return out


def final_norm(seed: int, shape: Shape, gains: str = "ones") -> np.ndarray:
    return gen.gains(seed, stream_id(gen.KIND_FINAL_NORM, 0), shape.hidden, gains)


def table(seed: int, kind: int, index: int, rows: int, cols: int, bf16: bool,
          std: float = 0.02) -> np.ndarray:
    """An embedding table or head [rows][cols] (fp32 or bf16 bits)."""
    return gen.fast_normal(seed, stream_id(kind, index), (rows, cols), std=std, bf16=bf16)


def table_rows(seed: int, kind: int, index: int, cols: int, row_ids, bf16: bool,
               std: float = 0.02) -> np.ndarray:
    """Selected rows of a table, generated without the rest of it."""
    row_ids = np.asarray(row_ids, dtype=np.int64).reshape(-1)
    out = np.empty((row_ids.size, cols), np.uint16 if bf16 else np.float32)
    for i, r in enumerate(row_ids):
        out[i] = gen.fast_normal(seed, stream_id(kind, index), (cols,), std=std,
                                 start=int(r) * cols, bf16=bf16)
    return out


def kv_prefill(seed: int, shape: Shape, layer: int, b: int, length: int, bf16: bool):
    """(K, V) prefill of one decode stream: arrays [length][n_kv][head_dim]."""
    per_pos = shape.n_kv_heads * shape.head_dim
    start = b * KV_POS_STRIDE * per_pos
    kshape = (length, shape.n_kv_heads, shape.head_dim)
    k = gen.fast_normal(seed, stream_id(gen.KIND_K_CACHE, layer), kshape, 1.0, start, bf16)
    v = gen.fast_normal(seed, stream_id(gen.KIND_V_CACHE, layer), kshape, 1.0, start, bf16)
    return k, v


def page_table(seed: int, lengths_with_room: List[int], extra_pages: int = 0):
    """Scatter each stream's pages over a pool by a seeded permutation.

    Returns (page_table [B][max_pages] int32 with -1 for unused, n_pages)."""
    need = [(n + PAGE - 1) // PAGE for n in lengths_with_room]
    n_pages = int(sum(need)) + int(extra_pages)
    max_pages = max(need) if need else 1
    perm = gen.permutation(seed, stream_id(gen.KIND_PAGE_PERM, 0), n_pages)
    pt = np.full((len(need), max_pages), -1, np.int32)
    c = 0
    for b, n in enumerate(need):
        pt[b, :n] = perm[c:c + n]
        c += n
    return pt, n_pages


@dataclass
class Workload:
    name: str
    seed: int
    shape: Shape
    bf16: bool
    desc: str
    extra: Dict = field(default_factory=dict)


def c1() -> Workload:
    """Single decoder layer, q_len=1 decode, batch 1, fp32, KV prefilled to 64."""
    return Workload("c1_layer_fp32", 0, Shape(n_layers=1), False,
                    "1 layer, fp32, batch 1, KV 64 -> position 64",
                    dict(batch=1, prefill=[64], steps=1))


def c2() -> Workload:
    """28-layer decode, batch 1, bf16, 16 summed codebooks of 2048, KV 1000, 148 steps,
    3072-way head with greedy argmax."""
    return Workload("c2_decode_b1", 0, Shape(), True,
                    "28 layers, bf16, batch 1, KV 1000 -> 1147, 148 steps, 16x2048 tables, 3072 head",
                    dict(batch=1, prefill=[1000], steps=148, n_cb=16, cb_vocab=2048,
                         head_groups=1, head_vocab=3072))


def c3() -> Workload:
    """5-layer code predictor, 256 frames in lockstep, 1-token prefill from a hidden then
    15 q_len=1 steps, own 2048-way table and head per step, argmax fed back."""
    return Workload("c3_predictor", 0, Shape(n_layers=5), True,
                    "5 layers, bf16, 256 frames x (1 prefill + 15 steps), 2048 tables/heads",
                    dict(batch=256, steps=15, cb_vocab=2048))


def c4() -> Workload:
    """MaskGIT pass: 200 text + 750 frames x 8 codebooks of 1025 (id 1024 = mask),
    half the codes masked, 28 bidirectional layers, 8 per-codebook 1025-way heads,
    32 steps on a cosine schedule."""
    return Workload("c4_maskgit", 0, Shape(), True,
                    "28 layers, bf16, S=950 (200 text + 750 frames), 8x1025, 32 steps",
                    dict(n_text=200, n_frames=750, n_cb=8, cb_vocab=1025, mask_id=1024,
                         text_vocab=151676, n_steps=32, layer_penalty=5.0,
                         masked_fraction=0.5))


def c5() -> Workload:
    """Batched paged decode: 64 streams, KV lengths U[200, 4000], 16-token pages,
    8 summed codebooks of 1025, 28 layers, bf16, seed 7."""
    return Workload("c5_paged_decode", 7, Shape(), True,
                    "28 layers, bf16, 64 streams, KV U[200,4000], 16-token pages, 8x1025",
                    dict(batch=64, len_lo=200, len_hi=4000, n_cb=8, cb_vocab=1025,
                         head_groups=8, head_vocab=1025, iters=32))


def c5_lengths(w: Workload) -> np.ndarray:
    e = w.extra
    n = e["len_hi"] - e["len_lo"] + 1
    return (gen.uniform_int(w.seed, stream_id(gen.KIND_LENGTHS, 0), (e["batch"],), n)
            + e["len_lo"]).astype(np.int32)


def maskgit_codes(w: Workload):
    """Initial codes [n_cb][n_frames]: U[0, 1024) with exactly half set to the mask id."""
    e = w.extra
    n_cb, n_frames = e["n_cb"], e["n_frames"]
    codes = gen.uniform_int(w.seed, stream_id(gen.KIND_CODES, 0), (n_cb, n_frames),
                            e["cb_vocab"] - 1)
    n_mask = int(round(e["masked_fraction"] * n_cb * n_frames))
    perm = gen.permutation(w.seed, stream_id(gen.KIND_MASK_PERM, 0), n_cb * n_frames)
    flat = codes.reshape(-1)
    flat[perm[:n_mask]] = e["mask_id"]
    return flat.reshape(n_cb, n_frames).astype(np.int32)


def maskgit_text_ids(w: Workload) -> np.ndarray:
    e = w.extra
    return gen.uniform_int(w.seed, stream_id(gen.KIND_TEXT_IDS, 0), (e["n_text"],),
                           e["text_vocab"]).astype(np.int32)


ALL = {"c1": c1, "c2": c2, "c3": c3, "c4": c4, "c5": c5}


class LazyTable:
    """A [rows][cols] table whose rows are generated on demand (``t[ids]`` -> fp32 values,
    bf16 tables widened).  Lets the oracle read a few rows of a 151676-row table."""

    def __init__(self, seed: int, kind: int, index: int, rows: int, cols: int, bf16: bool,
                 std: float = 0.02):
        self.seed, self.kind, self.index = seed, kind, index
        self.rows, self.cols, self.bf16, self.std = rows, cols, bf16, std
        self.shape = (rows, cols)

    def __getitem__(self, ids):
        ids = np.asarray(ids, dtype=np.int64)
        if ids.ndim == 0:
            return self[ids.reshape(1)][0]
        if np.any(ids < 0) or np.any(ids >= self.rows):
            raise IndexError("row id out of range")
        r = table_rows(self.seed, self.kind, self.index, self.cols, ids.reshape(-1), self.bf16,
                       self.std)
        r = gen.bf16_bits_to_f32(r) if self.bf16 else r
        return r.reshape(ids.shape + (self.cols,))

    def full(self) -> np.ndarray:
        """The whole table as stored (fp32 values or bf16 bits)."""
        return table(self.seed, self.kind, self.index, self.rows, self.cols, self.bf16, self.std)
