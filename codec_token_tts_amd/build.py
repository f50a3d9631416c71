"""Build libttsbb.so (HIP for gfx950) in-tree: codec_token_tts_amd/lib/libttsbb.so.

    python -m codec_token_tts_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(OUT_DIR, "libttsbb.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["k_embed_norm.hip", "k_gemm.hip", "k_rope_decode.hip", "k_flash.hip", "k_head.hip", "k_rvq.hip",
           "ttsbb_api.cpp"]

COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-fvisibility=hidden",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
          # no packed-fp32 instructions in any generated code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, obj: str) -> str:
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), p.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; always rebuilds."""
    obj_dir = os.path.join(OUT_DIR, "_obj")
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), p.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
