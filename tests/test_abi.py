"""Host-side checks of libfa.so: exports and argument validation (no GPU needed).

Every call here fails validation before any HIP call, so nothing is launched;
the pointers passed are never dereferenced.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    from exact_io_aware_34_amd import build
    if not os.path.exists(build.LIB):
        build.build()
    L = ctypes.CDLL(build.LIB)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp]
    L.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp,
                              ctypes.c_size_t, vp]
    L.fa_backward_workspace_size.argtypes = [i, i, i, i]
    L.fa_backward_workspace_size.restype = ctypes.c_size_t
    L.fa_status_string.restype = ctypes.c_char_p
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "fa_abi_version", "fa_backward", "fa_backward_workspace_size", "fa_forward",
        "fa_status_string"])


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.fa_abi_version() == 1


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        s = lib.fa_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.fa_status_string(17).decode() == "unknown status"


def test_workspace_size(lib):
    assert lib.fa_backward_workspace_size(4, 12, 8192, 64) == 2 * 4 * 12 * 8192 * 4
    assert lib.fa_backward_workspace_size(1, 1, 3, 64) == 512
    assert lib.fa_backward_workspace_size(0, 1, 3, 64) == 0


FAKE = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced
MISALIGNED = ctypes.c_void_p((1 << 20) + 8)


def fwd(lib, q=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=128, d=64, scale=0.125, dtype=2):
    return lib.fa_forward(q, FAKE, FAKE, o, lse, B, H, N, d, scale, 0, None, dtype, None)


def test_forward_validation(lib):
    assert fwd(lib, q=None) == -1
    assert fwd(lib, lse=None) == -1
    assert fwd(lib, o=MISALIGNED) == -1
    assert fwd(lib, B=0) == -1
    assert fwd(lib, N=0) == -1
    assert fwd(lib, N=-5) == -1
    assert fwd(lib, dtype=3) == -1
    assert fwd(lib, scale=float("nan")) == -1
    assert fwd(lib, scale=float("inf")) == -1
    assert fwd(lib, scale=0.0) == -1
    assert fwd(lib, scale=-0.125) == -1
    assert fwd(lib, d=96) == -2
    assert fwd(lib, d=256) == -2
    assert fwd(lib, N=1 << 30, d=64) == -2


def bwd(lib, dtype=2, ws=FAKE, ws_bytes=1 << 30, d=64, dq=FAKE):
    return lib.fa_backward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE, 2, 3, 100, d,
                           0.125, 1, None, dtype, ws, ws_bytes, None)


def test_backward_validation(lib):
    assert bwd(lib, dq=None) == -1
    assert bwd(lib, dq=MISALIGNED) == -1
    assert bwd(lib, d=80) == -2
    assert bwd(lib, dtype=0) == -2                      # fp32 backward not built
    assert bwd(lib, ws=None) == -3
    assert bwd(lib, ws_bytes=2 * 2 * 3 * 100 * 4 - 1) == -3
