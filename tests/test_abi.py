"""The C ABI on the CPU: the library loads and exports exactly what include/ttsbb.h
declares, the header is plain C99, and every entry point rejects bad arguments on the
host before touching a device."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttsbb.h")
LIB_DIR = os.path.join(ROOT, "codec_token_tts_amd", "lib")
LIB = os.path.join(LIB_DIR, "libttsbb.so")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ttsbb_[a-z_]+)\s*\(", src)))


def require_lib():
    if not os.path.exists(LIB):
        pytest.skip("libttsbb.so not built (run __graft_entry__.build())")


def test_library_exports_every_declared_symbol():
    require_lib()
    from codec_token_tts_amd import ttsbb as T
    lib = T.lib()
    decl = declared_functions()
    assert len(decl) == 19
    assert sorted(T.EXPORTS) == decl
    for name in decl:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(ttsbb_\w+)", out))
    assert exported == set(decl)


def test_header_is_c99_and_entry_points_check_arguments(tmp_path):
    require_lib()
    exe = str(tmp_path / "abi_c99")
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic",
                           "-I", os.path.join(ROOT, "include"),
                           os.path.join(ROOT, "tests", "abi_c99.c"), "-o", exe,
                           "-L", LIB_DIR, "-lttsbb", "-Wl,-rpath," + LIB_DIR])
    p = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr
    assert "abi ok" in p.stdout


def test_python_binding_rejects_host_tensors_and_reports_status():
    require_lib()
    import torch

    from codec_token_tts_amd import ttsbb as T
    with pytest.raises(ValueError):
        T.ptr(torch.zeros(3))
    assert T.ttsbb_status_str(T.INVALID_ARG) == "invalid argument"
    st, ctx = T.ttsbb_create(T.ttsbb_default_config(), [], None, raw_status=True)
    assert st == T.INVALID_ARG and not ctx


def test_host_schedule_matches_oracle():
    require_lib()
    from codec_token_tts_amd import ttsbb as T
    from oracle import backbone as O
    for n, s in ((3000, 32), (7, 3), (0, 5), (1, 1), (12345, 17)):
        assert T.ttsbb_unmask_schedule(n, s) == O.unmask_schedule(n, s)
