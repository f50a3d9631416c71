"""Seeded synthetic inputs placed in device memory (torch tensors on the GPU).

Large tensors are generated on the device by workload/fill.hip, which implements the
same generator as workload/gen.py bit for bit; small ones are generated on the host and
copied.  Holds no model arithmetic.  bf16 tensors are int16 tensors holding the bit
patterns (the HIP library takes raw pointers).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

from . import configs as CFG
from . import gen

_HERE = os.path.dirname(os.path.abspath(__file__))
_FILL_SRC = os.path.join(_HERE, "fill.hip")
_FILL_LIB = os.path.join(_HERE, "_lib", "libwlfill.so")
_fill = None


def build_fill_lib(force: bool = True) -> str:
    if force or not os.path.exists(_FILL_LIB) or \
            os.path.getmtime(_FILL_LIB) < os.path.getmtime(_FILL_SRC):
        os.makedirs(os.path.dirname(_FILL_LIB), exist_ok=True)
        tmp = _FILL_LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC",
                               "-shared", "-fvisibility=hidden", "-Xclang", "-target-feature",
                               "-Xclang", "-packed-fp32-ops", _FILL_SRC, "-o", tmp],
                              stderr=subprocess.DEVNULL)
        os.replace(tmp, _FILL_LIB)
    return _FILL_LIB


def _lib():
    global _fill
    if _fill is None:
        if not os.path.exists(_FILL_LIB):
            raise RuntimeError("workload fill library not built: %s" % _FILL_LIB)
        L = C.CDLL(_FILL_LIB)
        L.wl_fill_normal.argtypes = [C.c_void_p, C.c_int64, C.c_uint64, C.c_uint32, C.c_uint64,
                                     C.c_float, C.c_int, C.c_void_p]
        L.wl_fill_normal.restype = C.c_int
        L.wl_fill_kv.argtypes = [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p,
                                 C.c_int, C.c_void_p, C.c_int64, C.c_uint64, C.c_uint32, C.c_uint32,
                                 C.c_float, C.c_int, C.c_void_p]
        L.wl_fill_kv.restype = C.c_int
        L.wl_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]
        L.wl_copy.restype = C.c_int
        _fill = L
    return _fill


def _torch():
    import torch
    return torch


def _stream_ptr():
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def host_to_device(a: np.ndarray):
    """Copy a host array (uint16 bf16 bits -> int16 tensor; others as their dtype)."""
    torch = _torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def normal(shape, seed: int, stream: int, std: float, bf16: bool, start: int = 0):
    """Device tensor equal to gen.fast_normal(seed, stream, shape, std, start, bf16)."""
    torch = _torch()
    t = torch.empty(tuple(shape), dtype=torch.int16 if bf16 else torch.float32, device="cuda")
    n = int(np.prod(shape))
    rc = _lib().wl_fill_normal(t.data_ptr(), n, seed, stream, start, float(gen.normal_scale(std)),
                               1 if bf16 else 0, _stream_ptr())
    if rc != 0:
        raise RuntimeError("wl_fill_normal failed")
    return t


def layer_weights(seed: int, shape: CFG.Shape, layer: int, bf16: bool, gains: str = "ones",
                  std: float = 0.02):
    """Device twin of configs.layer_weights."""
    out = {}
    for name, (kind, rows, cols) in CFG.WEIGHT_KINDS.items():
        out[name] = normal((rows(shape), cols(shape)), seed, gen.stream_id(kind, layer), std, bf16)
    for name, (kind, n) in CFG.GAIN_KINDS.items():
        out[name] = host_to_device(gen.gains(seed, gen.stream_id(kind, layer), n(shape), gains))
    return out


def table(seed: int, kind: int, index: int, rows: int, cols: int, bf16: bool, std: float = 0.02):
    """Device twin of configs.table."""
    return normal((rows, cols), seed, gen.stream_id(kind, index), std, bf16)


def kv_pool(seed: int, shape: CFG.Shape, n_layers: int, lengths, page_table: np.ndarray,
            n_pages: int, bf16: bool):
    """Paged KV pool [n_layers][n_pages][2][Hkv][PAGE][head_dim] holding each stream's
    prefill (configs.kv_prefill) at its pages; every other slot is zero."""
    torch = _torch()
    B, max_pages = page_table.shape
    owner = np.full(n_pages, -1, np.int32)
    for b in range(B):
        for j in range(max_pages):
            if page_table[b, j] >= 0:
                owner[page_table[b, j]] = b * max_pages + j
    owner_d = host_to_device(owner)
    len_d = host_to_device(np.asarray(lengths, np.int32))
    pool = torch.empty((n_layers, n_pages, 2, shape.n_kv_heads, CFG.PAGE, shape.head_dim),
                       dtype=torch.int16 if bf16 else torch.float32, device="cuda")
    for l in range(n_layers):
        rc = _lib().wl_fill_kv(pool[l].data_ptr(), n_pages, shape.n_kv_heads, CFG.PAGE,
                               shape.head_dim, owner_d.data_ptr(), max_pages, len_d.data_ptr(),
                               CFG.KV_POS_STRIDE, seed, gen.stream_id(gen.KIND_K_CACHE, l),
                               gen.stream_id(gen.KIND_V_CACHE, l), float(gen.normal_scale(1.0)),
                               1 if bf16 else 0, _stream_ptr())
        if rc != 0:
            raise RuntimeError("wl_fill_kv failed")
    return pool


def bits_to_f32(t) -> np.ndarray:
    """Device bf16 bits (int16) or fp32 tensor -> host fp32 values."""
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        return gen.bf16_bits_to_f32(a.view(np.uint16))
    return a.astype(np.float32)


def copy(src, dst, nbytes: int) -> None:
    """Plain device copy of nbytes (multiple of 16) through the workload library's copy kernel."""
    assert src.is_cuda and dst.is_cuda
    assert nbytes % 16 == 0 and nbytes <= src.numel() * src.element_size() and \
        nbytes <= dst.numel() * dst.element_size()
    if _lib().wl_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream_ptr()) != 0:
        raise RuntimeError("wl_copy failed")
