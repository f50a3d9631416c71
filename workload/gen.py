"""Seeded synthetic inputs for the TTS backbone, shared by the oracle and the GPU path.

This module holds no model arithmetic: it only turns (seed, stream, element index)
into numbers.  Every value is a pure function of those three integers, so any
element of any tensor can be produced on its own (sampled checks at full size),
and the GPU fill kernel in ``workload/fill.hip`` produces bit-identical tensors on
the device.

Generator
---------
Counter-based Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
as easy as 1, 2, 3", SC'11).  Element ``e`` of stream ``s`` under ``seed`` is word
``e % 4`` of ``philox(counter=(e//4 lo, e//4 hi, s, 0), key=(seed lo, seed hi))``.

Distributions (integer arithmetic only, so host and device agree exactly)
------------------------------------------------------------------------
* ``normal``: an Irwin-Hall approximation of N(0, 1).  From a 32-bit word take
  three 10-bit uniforms b0, b1, b2 and one coin bit c; ``k = b0+b1+b2+c-1535`` lies
  in [-1535, 1535] with mean 0 and variance exactly 2^18 (3 * (1024^2 - 1)/12 + 1/4),
  so ``k/512`` has mean 0 and unit variance.  A tensor of standard deviation ``std``
  is ``fp32(k) * fp32(std/512)`` (one correctly rounded fp32 product).  |k| needs up
  to 11 significant bits, so most unit-variance values are not representable in bf16
  (an fp32-mode input that were rounded to bf16 somewhere would show).
* ``uniform_int(n)``: ``(w * n) >> 32`` for a 32-bit word w.
* bf16 values are produced from fp32 by round-to-nearest-even on the bit pattern.
"""
from __future__ import annotations

import numpy as np

_MASK32 = np.uint64(0xFFFFFFFF)
_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85

# Stream kinds.  A stream id is (kind << 16) | index, index = layer or table number.
KIND_ATTN_NORM = 1
KIND_WQ = 2
KIND_WK = 3
KIND_WV = 4
KIND_Q_NORM = 5
KIND_K_NORM = 6
KIND_WO = 7
KIND_FFN_NORM = 8
KIND_W_GATE = 9
KIND_W_UP = 10
KIND_W_DOWN = 11
KIND_FINAL_NORM = 12
KIND_CB_TABLE = 13
KIND_TEXT_TABLE = 14
KIND_HEAD = 15
KIND_K_CACHE = 16
KIND_V_CACHE = 17
KIND_X_IN = 18
KIND_CODES = 19
KIND_TEXT_IDS = 20
KIND_LENGTHS = 21
KIND_PAGE_PERM = 22
KIND_MASK_PERM = 23
KIND_U_CLASS = 24   # uniforms of the sampler's class noise
KIND_U_POS = 25     # uniforms of the sampler's position noise


def stream_id(kind: int, index: int = 0) -> int:
    return ((int(kind) & 0xFFFF) << 16) | (int(index) & 0xFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds on uint32 values held in uint64 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    for r in range(10):
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
        k0 = (k0 + _W0) & 0xFFFFFFFF
        k1 = (k1 + _W1) & 0xFFFFFFFF
    return c0, c1, c2, c3


def words(seed: int, stream: int, index) -> np.ndarray:
    """32-bit random words for the given element indices (any integer array)."""
    idx = np.asarray(index, dtype=np.uint64)
    blk = idx >> np.uint64(2)
    lane = (idx & np.uint64(3)).astype(np.int64)
    o = philox4x32_10(blk & _MASK32, blk >> np.uint64(32),
                      np.full(idx.shape, stream & 0xFFFFFFFF, np.uint64),
                      np.zeros(idx.shape, np.uint64),
                      seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    out = np.where(lane == 0, o[0], np.where(lane == 1, o[1], np.where(lane == 2, o[2], o[3])))
    return out.astype(np.uint32)


def words_range(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    """Words for the contiguous element range [start, start+n); fast path."""
    if n <= 0:
        return np.zeros(0, np.uint32)
    b0 = start // 4
    b1 = (start + n + 3) // 4
    blk = np.arange(b0, b1, dtype=np.uint64)
    o = philox4x32_10(blk & _MASK32, blk >> np.uint64(32),
                      np.full(blk.shape, stream & 0xFFFFFFFF, np.uint64),
                      np.zeros(blk.shape, np.uint64),
                      seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = np.stack(o, axis=1).reshape(-1).astype(np.uint32)
    off = start - 4 * b0
    return w[off:off + n]


def normal_k(w: np.ndarray) -> np.ndarray:
    """Integer Irwin-Hall variate in [-1535, 1535], mean 0, variance 2^18."""
    w = w.astype(np.int64)
    return (w & 1023) + ((w >> 10) & 1023) + ((w >> 20) & 1023) + ((w >> 30) & 1) - 1535


def normal_scale(std: float) -> np.float32:
    return np.float32(np.float32(std) / np.float32(512.0))


def normal_f32(seed: int, stream: int, shape, std: float = 1.0, start: int = 0) -> np.ndarray:
    n = int(np.prod(shape)) if len(shape) else 1
    k = normal_k(words_range(seed, stream, start, n))
    return (k.astype(np.float32) * normal_scale(std)).reshape(shape)


def normal_f32_at(seed: int, stream: int, index, std: float = 1.0) -> np.ndarray:
    k = normal_k(words(seed, stream, index))
    return k.astype(np.float32) * normal_scale(std)


def uniform_int(seed: int, stream: int, shape, n: int, start: int = 0) -> np.ndarray:
    cnt = int(np.prod(shape)) if len(shape) else 1
    w = words_range(seed, stream, start, cnt).astype(np.uint64)
    return ((w * np.uint64(n)) >> np.uint64(32)).astype(np.int32).reshape(shape)


def open01_of_words(w: np.ndarray) -> np.ndarray:
    """fp32 uniforms strictly inside (0, 1) from 32-bit words: ((w >> 9) + 0.5) * 2^-23.
    (w >> 9) + 0.5 needs 24 significant bits, so the value is exact in fp32; the extremes
    are 2^-24 and 1 - 2^-24."""
    w = np.asarray(w, np.uint64)
    return (((w >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23).astype(np.float32)


def uniform_open01(seed: int, stream: int, shape, start: int = 0) -> np.ndarray:
    """open01_of_words of the stream's words, one word per value."""
    n = int(np.prod(shape))
    return open01_of_words(fast_words(seed, stream, start, n)).reshape(shape)


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    """A seeded permutation of range(n): stable argsort of random 32-bit keys."""
    keys = words_range(seed, stream, 0, n)
    return np.argsort(keys, kind="stable").astype(np.int32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (the bits become the high half of the word)."""
    b = np.asarray(b, dtype=np.uint16)
    out = np.zeros(b.shape + (2,), np.uint16)
    out[..., 1] = b  # little-endian: element 1 is the high half
    return out.view(np.float32).reshape(b.shape)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 value, returned as fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def gains(seed: int, stream: int, n: int, kind: str = "ones") -> np.ndarray:
    """Norm gain vectors (kept in fp32): all ones, or 1 + N(0, 0.1^2) for tests."""
    if kind == "ones":
        return np.ones(n, np.float32)
    return (np.float32(1.0) + normal_f32(seed, stream, (n,), std=0.1)).astype(np.float32)


# ---------------------------------------------------------------------------
# Host fast path (workload/gen_host.c), built with gcc on first use.  The numpy
# functions above are the definition; tests check the two agree.
# ---------------------------------------------------------------------------
import ctypes as _ct
import os as _os
import subprocess as _sp

_HERE = _os.path.dirname(_os.path.abspath(__file__))
_SRC = _os.path.join(_HERE, "gen_host.c")
_LIB_PATH = _os.path.join(_HERE, "_lib", "libwlgen.so")
_lib = None


def build_host_lib(force: bool = False) -> str:
    if force or not _os.path.exists(_LIB_PATH) or \
            _os.path.getmtime(_LIB_PATH) < _os.path.getmtime(_SRC):
        _os.makedirs(_os.path.dirname(_LIB_PATH), exist_ok=True)
        tmp = _LIB_PATH + ".tmp%d" % _os.getpid()
        _sp.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-ffp-contract=off",
                        "-fno-fast-math", "-fopenmp", _SRC, "-o", tmp])
        _os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _host_lib():
    global _lib
    if _lib is None:
        lib = _ct.CDLL(build_host_lib())
        lib.wl_words.argtypes = [_ct.c_uint64, _ct.c_uint32, _ct.c_uint64, _ct.c_int64, _ct.c_void_p]
        lib.wl_words.restype = None
        lib.wl_normal.argtypes = [_ct.c_uint64, _ct.c_uint32, _ct.c_uint64, _ct.c_int64,
                                  _ct.c_float, _ct.c_int, _ct.c_void_p]
        lib.wl_normal.restype = None
        _lib = lib
    return _lib


def fast_words(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint32)
    _host_lib().wl_words(seed, stream, start, n, out.ctypes.data)
    return out


def fast_normal(seed: int, stream: int, shape, std: float = 1.0, start: int = 0,
                bf16: bool = False) -> np.ndarray:
    """normal_f32 (bf16=False) or f32_to_bf16_bits(normal_f32) (bf16=True), fast."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, np.uint16 if bf16 else np.float32)
    _host_lib().wl_normal(seed, stream, start, n, float(normal_scale(std)), 1 if bf16 else 0,
                          out.ctypes.data)
    return out.reshape(shape)
