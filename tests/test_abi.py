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
    L.fa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, ctypes.c_size_t, vp]
    L.fa_decode_splits.argtypes = [i] * 6
    L.fa_decode_workspace_size.argtypes = [i] * 6
    L.fa_decode_workspace_size.restype = ctypes.c_size_t
    L.fa_forward_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, vp,
                                 ctypes.c_size_t, vp]
    L.fa_fp8_prepare.argtypes = [vp, vp, vp, i, i, i, i, f, i, vp, vp, ctypes.c_size_t, vp]
    L.fa_forward_fp8_workspace_size.argtypes = [i, i, i, i]
    L.fa_forward_fp8_workspace_size.restype = ctypes.c_size_t
    u64, u32 = ctypes.c_uint64, ctypes.c_uint32
    L.fa_forward_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, f, u64, u32, vp,
                                     vp]
    L.fa_backward_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i,
                                      f, u64, u32, vp, ctypes.c_size_t, vp]
    L.fa_dropout_mask.argtypes = [i, i, i, f, u64, u32, vp, vp]
    L.fa_forward_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, i, vp,
                                   ctypes.c_size_t, vp]
    L.fa_forward_splits.argtypes = [i] * 6
    L.fa_forward_split_workspace_size.argtypes = [i] * 6
    L.fa_forward_split_workspace_size.restype = ctypes.c_size_t
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "fa_abi_version", "fa_backward", "fa_backward_workspace_size", "fa_decode",
        "fa_decode_splits", "fa_decode_workspace_size", "fa_dropout_mask", "fa_forward",
        "fa_forward_dropout", "fa_forward_fp8", "fa_forward_fp8_workspace_size", "fa_fp8_prepare",
        "fa_backward_dropout", "fa_status_string", "fa_forward_split", "fa_forward_splits",
        "fa_forward_split_workspace_size", "fa_decode_noalloc"])


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.fa_abi_version() == 6


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        s = lib.fa_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.fa_status_string(17).decode() == "unknown status"


def test_workspace_size(lib):
    # -D and lse * log2 e (fp32 per row, each padded to 256 bytes), then the
    # block-sparse order (two int32 per 128-row tile, padded to 256 bytes)
    assert lib.fa_backward_workspace_size(4, 12, 8192, 64) == 2 * 4 * 12 * 8192 * 4 + 512
    assert lib.fa_backward_workspace_size(1, 1, 3, 64) == 3 * 256
    assert lib.fa_backward_workspace_size(1, 1, 2048 * 128, 64) == 2 * 2048 * 128 * 4 + 16384
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


def bwd(lib, dtype=2, ws=FAKE, ws_bytes=1 << 30, d=64, dq=FAKE, N=100, mask=None):
    return lib.fa_backward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, dq, FAKE, FAKE, 2, 3, N, d,
                           0.125, 1, mask, dtype, ws, ws_bytes, None)


def test_backward_validation(lib):
    assert bwd(lib, dq=None) == -1
    assert bwd(lib, dq=MISALIGNED) == -1
    assert bwd(lib, d=80) == -2
    assert bwd(lib, dtype=0) == -2                      # fp32 backward not built
    assert bwd(lib, ws=None) == -3
    need = lib.fa_backward_workspace_size(2, 3, 100, 64)
    assert need == 2 * 2560 + 256
    assert bwd(lib, ws_bytes=need - 1) == -3


def test_block_mask_size_limit(lib):
    """A block mask covers at most 2048 x 2048 tiles (N <= 262144): every call
    that takes one rejects a longer sequence before any launch."""
    n_big = 2048 * 128 + 1
    assert bwd(lib, N=n_big, mask=FAKE) == -2
    assert lib.fa_backward_dropout(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 3,
                                   n_big, 64, 0.125, 1, FAKE, 2, 0.1, 1, 0, FAKE, 1 << 40,
                                   None) == -2
    assert lib.fa_forward(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, n_big, 64, 0.125, 0, FAKE, 2,
                          None) == -2
    assert lib.fa_forward_dropout(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, n_big, 64, 0.125, 0, FAKE,
                                  2, 0.1, 1, 0, None, None) == -2


def test_decode_split_choice(lib):
    S = lib.fa_decode_splits

    def expect(Nk, n):
        L = -(-Nk // n)
        L = -(-L // 128) * 128
        return -(-Nk // L)
    # Explicit counts: ranges are a multiple of 128 keys long, so fewer may result.
    for Nk, n in [(1, 1), (1, 8), (1000, 4), (1000, 3), (1000, 7), (129, 2), (65536, 5),
                  (4097, 33)]:
        assert S(1, 1, 1, Nk, 64, n) == expect(Nk, n), (Nk, n)
    assert S(1, 1, 1, 1000, 64, 7) == 4
    # Automatic: about 192 (b*h, range) workgroups, ranges of >= 512 keys.
    assert S(8, 12, 1, 65536, 64, 0) == 2      # 96 heads x 2
    assert S(8, 12, 1, 65536, 128, 0) == 2
    assert S(4, 12, 1, 65536, 64, 0) == 4
    assert S(1, 12, 1, 262144, 64, 0) == 16
    assert S(1, 8, 1, 131072, 128, 0) == 24
    assert S(2, 40, 1, 65536, 64, 0) == 2      # 192 / 80 rounds to 2
    assert S(1, 1, 1, 65536, 64, 0) == 128     # 192 wanted, but ranges >= 512 keys
    assert S(1, 1, 1, 300, 64, 0) == 1
    assert S(64, 16, 1, 8192, 64, 0) == 1
    # Bad input
    assert S(0, 1, 1, 10, 64, 0) == 0
    assert S(1, 1, 5, 4, 64, 0) == 0
    assert S(1, 1, 1, 10, 96, 0) == 0
    assert S(1, 1, 1, 10, 64, -1) == 0


def test_decode_workspace_size(lib):
    W = lib.fa_decode_workspace_size
    assert W(1, 1, 1, 100, 64, 1) == 0
    assert W(1, 1, 1, 100, 64, 0) == 0         # one range
    # 8*12*2 ranges x 1 query: 192 rows of 64 fp32 + 192 fp32, each padded to 256 B
    assert W(8, 12, 1, 65536, 64, 0) == 192 * 64 * 4 + 768
    assert W(2, 3, 4, 1000, 128, 4) == 2 * 3 * 4 * 4 * 128 * 4 + 512


def dec(lib, q=FAKE, lse=FAKE, B=1, H=2, Nq=1, Nk=1000, d=64, scale=0.125, dtype=2, n=4,
        ws=FAKE, ws_bytes=1 << 30):
    return lib.fa_decode(q, FAKE, FAKE, FAKE, lse, B, H, Nq, Nk, d, scale, 1, n, dtype, ws,
                         ws_bytes, None)


def test_decode_validation(lib):
    assert dec(lib, q=None) == -1
    assert dec(lib, q=MISALIGNED) == -1
    assert dec(lib, lse=None) == -1
    assert dec(lib, Nq=0) == -1
    assert dec(lib, Nq=5, Nk=4) == -1           # queries are positions of the sequence
    assert dec(lib, n=-1) == -1
    assert dec(lib, dtype=7) == -1
    assert dec(lib, scale=float("nan")) == -1
    assert dec(lib, d=80) == -2
    assert dec(lib, dtype=0) == -2              # fp32 decode not built
    assert dec(lib, Nq=17, Nk=100) == -2        # more than one MFMA column block of queries
    assert dec(lib, Nk=1 << 26, d=64) == -2
    assert dec(lib, ws=None) == -3
    need = lib.fa_decode_workspace_size(1, 2, 1, 1000, 64, 4)
    assert need > 0 and dec(lib, ws_bytes=need - 1) == -3


def test_fp8_workspace_size(lib):
    W = lib.fa_forward_fp8_workspace_size
    # 3 operand regions of B*H*Npad*d bytes + 3 scale regions of B*H*nt fp32, then the
    # block-sparse work order (two int32 per 128-row tile), each padded to 256
    assert W(4, 12, 8192, 64) == 3 * 48 * 8192 * 64 + 3 * 48 * 128 * 4 + 512
    assert W(1, 1, 65, 128) == 3 * 128 * 128 + 3 * 256 + 256
    assert W(0, 1, 64, 64) == 0


def f8(lib, q=FAKE, o=FAKE, lse=FAKE, N=100, d=64, dtype=2, ws=FAKE, ws_bytes=1 << 30,
       scale=0.125):
    return lib.fa_forward_fp8(q, FAKE, FAKE, o, lse, 2, 3, N, d, scale, 1, None, dtype, None, ws,
                              ws_bytes, None)


def test_fp8_validation(lib):
    assert f8(lib, q=None) == -1
    assert f8(lib, o=MISALIGNED) == -1
    assert f8(lib, lse=None) == -1
    assert f8(lib, N=0) == -1
    assert f8(lib, scale=0.0) == -1
    assert f8(lib, d=96) == -2
    assert f8(lib, dtype=0) == -2                       # fp32 inputs not built
    assert f8(lib, ws=None) == -3
    assert f8(lib, ws=ctypes.c_void_p((1 << 20) + 16)) == -3   # not 256-byte aligned
    need = lib.fa_forward_fp8_workspace_size(2, 3, 100, 64)
    assert f8(lib, ws_bytes=need - 1) == -3
    assert lib.fa_fp8_prepare(FAKE, FAKE, FAKE, 2, 3, 100, 64, 0.125, 2, None, None, 0, None) == -3
    assert lib.fa_fp8_prepare(None, FAKE, FAKE, 2, 3, 100, 64, 0.125, 2, None, FAKE, need,
                              None) == -1
    assert lib.fa_fp8_prepare(FAKE, FAKE, FAKE, 2, 3, 100, 64, 0.0, 2, None, FAKE, need,
                              None) == -1                      # scale must be finite and > 0
    assert lib.fa_fp8_prepare(FAKE, FAKE, FAKE, 2, 3, 100, 64, float("nan"), 2, None, FAKE, need,
                              None) == -1
    # the rotation signs are read as 16-byte vectors
    assert lib.fa_fp8_prepare(FAKE, FAKE, FAKE, 2, 3, 100, 64, 0.125, 2, MISALIGNED, FAKE, need,
                              None) == -1
    assert lib.fa_forward_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 3, 100, 64, 0.125, 1, None, 2,
                              ctypes.c_void_p((1 << 20) + 8), FAKE, need, None) == -1


def test_dropout_validation(lib):
    def fwd_d(p, dtype=2, o_acc=None):
        return lib.fa_forward_dropout(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 100, 64, 0.125, 0, None,
                                      dtype, p, 1, 0, o_acc, None)
    assert fwd_d(-0.1) == -1
    assert fwd_d(1.0) == -1
    assert fwd_d(float("nan")) == -1
    assert fwd_d(0.1, dtype=0) == -2                    # fp32 forward has no dropout
    assert fwd_d(0.0, dtype=0, o_acc=FAKE) == -2        # nor an fp32 o_acc
    assert fwd_d(0.1, o_acc=MISALIGNED) == -1

    def bwd_d(p=0.1, o_acc=FAKE, dtype=2):
        return lib.fa_backward_dropout(FAKE, FAKE, FAKE, o_acc, FAKE, FAKE, FAKE, FAKE, FAKE, 1,
                                       2, 100, 64, 0.125, 0, None, dtype, p, 1, 0, FAKE, 1 << 30,
                                       None)
    assert bwd_d(p=1.5) == -1
    assert bwd_d(o_acc=None) == -1                       # the fp32 O is required
    assert bwd_d(o_acc=MISALIGNED) == -1
    assert bwd_d(dtype=0) == -2
    assert lib.fa_dropout_mask(1, 1, 10, 0.5, 1, 0, None, None) == -1
    assert lib.fa_dropout_mask(1, 1, 10, 1.0, 1, 0, FAKE, None) == -1
    assert lib.fa_dropout_mask(1, 1, 70000, 0.5, 1, 0, FAKE, None) == -2


def test_forward_split_choice(lib):
    def S(B, H, N, d, n, dtype=2):                # default: bf16 inputs
        return lib.fa_forward_splits(B, H, N, d, n, dtype)
    # Automatic: one run once the plain grid fills a round (768 workgroups at
    # d = 64, 512 at d = 128).
    assert S(4, 12, 8192, 64, 0) == 1          # 3072 query tiles
    assert S(1, 6, 16384, 64, 0) == 1          # 768
    assert S(1, 4, 16384, 128, 0) == 1         # 512
    # Smaller grids: one round of (query tile, run) workgroups, >= 10 key tiles per run.
    assert S(1, 4, 16384, 64, 0) == 2          # 512 tiles -> ceil(768 / 512)
    assert S(1, 1, 4096, 64, 0) == 6           # 32 tiles -> 24 wanted, 64 key tiles / 10
    assert S(1, 1, 16384, 64, 0) == 6          # 128 tiles -> ceil(768 / 128)
    assert S(1, 2, 8192, 128, 0) == 4          # 128 tiles -> ceil(512 / 128)
    assert S(1, 2, 4096, 128, 0) == 6          # 64 tiles -> 8 wanted, 64 key tiles / 10
    assert S(1, 1, 256, 64, 0) == 1            # 4 key tiles
    assert S(1, 1, 1000, 64, 0) == 1           # 16 key tiles: one run of >= 10
    assert S(1, 1, 1000, 64, 0, 1) == 1        # fp16: the same rule
    # fp32 inputs: 256 workgroups wanted, runs of >= 1 key tile
    assert S(1, 1, 256, 64, 0, 0) == 4         # 4 key tiles, one per run
    assert S(1, 1, 1000, 64, 0, 0) == 16       # 16 key tiles, 8 query tiles -> 32 wanted
    assert S(1, 1, 4096, 64, 0, 0) == 8        # 32 query tiles -> 8 wanted
    assert S(1, 4, 8192, 64, 0, 0) == 1        # 256 query tiles
    assert S(4, 12, 8192, 64, 0, 0) == 1       # full grid
    assert S(1, 1, 100, 64, 0, 0) == 2         # 2 key tiles, one per run
    # Explicit counts are capped at the key tiles and at 64.
    assert S(1, 1, 300, 64, 9) == 5
    assert S(1, 1, 1 << 16, 64, 100) == 64
    assert S(1, 1, 4096, 64, 3) == 3
    # Bad input
    assert S(0, 1, 10, 64, 0) == 0
    assert S(1, 1, 10, 96, 0) == 0
    assert S(1, 1, 10, 64, -1) == 0
    assert S(1, 1, 10, 64, 0, 7) == 0          # unknown dtype


def test_forward_split_workspace_size(lib):
    def W(B, H, N, d, n, dtype=2):
        return lib.fa_forward_split_workspace_size(B, H, N, d, n, dtype)
    def order(N):  # block-sparse work order: two int32 per 128-row tile, padded to 256 bytes
        return -(-(2 * -(-N // 128) * 4) // 256) * 256
    assert W(4, 12, 8192, 64, 0) == order(8192) == 512     # one run: the order only
    assert W(1, 1, 300, 64, 1) == order(300) == 256
    # 6 runs of 4096 rows x 64 fp32, then 6 x 4096 fp32, then the order
    assert W(1, 1, 4096, 64, 0) == 6 * 4096 * 64 * 4 + 6 * 4096 * 4 + 256
    assert W(1, 2, 300, 128, 3) == (2 * 3 * 300 * 128 * 4 + (-(-2 * 3 * 300 * 4 // 256)) * 256
                                    + 256)
    assert W(1, 1, 256, 64, 0, 0) == 4 * 256 * 64 * 4 + 4 * 256 * 4 + 256  # fp32: 4 runs
    assert W(1, 1, 2048 * 128, 64, 1) == 2 * 2048 * 4
    assert W(1, 1, 256, 64, 0, 9) == 0


def fsplit(lib, q=FAKE, lse=FAKE, B=1, H=1, N=4096, d=64, scale=0.125, dtype=2, n=4, ws=FAKE,
           ws_bytes=1 << 30):
    return lib.fa_forward_split(q, FAKE, FAKE, FAKE, lse, B, H, N, d, scale, 0, None, dtype, n,
                                ws, ws_bytes, None)


def test_forward_split_validation(lib):
    assert fsplit(lib, n=-1) == -1
    assert fsplit(lib, q=None) == -1
    assert fsplit(lib, q=MISALIGNED) == -1
    assert fsplit(lib, lse=None) == -1
    assert fsplit(lib, B=0) == -1
    assert fsplit(lib, dtype=9) == -1
    assert fsplit(lib, scale=float("inf")) == -1
    assert fsplit(lib, d=80) == -2
    assert fsplit(lib, ws=None) == -3
    assert fsplit(lib, ws=MISALIGNED) == -3
    need = lib.fa_forward_split_workspace_size(1, 1, 4096, 64, 4, 2)
    assert need > 0 and fsplit(lib, ws_bytes=need - 1) == -3


def test_binding_rejects_host_or_mistyped_buffers():
    """The Python binding checks every caller-supplied buffer before a call
    reaches libfa: a host tensor, a wrong dtype or shape, or a non-contiguous
    one raises ValueError (a host pointer handed to a kernel would fault)."""
    import torch

    from exact_io_aware_34_amd import fa
    ok = torch.empty((2, 3, 4), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU"):
        fa._check_f32(ok, (2, 3, 4), "lse")                      # on the host
    with pytest.raises(ValueError):
        fa._check_workspace(torch.empty(16, dtype=torch.uint8))  # on the host
    with pytest.raises(ValueError):
        fa._check_f32(object(), (2, 3, 4), "grads")
    assert fa._check_workspace(None) == 0
    q = torch.empty((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        fa.forward(q, q, q)
    with pytest.raises(ValueError, match="GPU"):
        fa.backward(q, q, q, q, torch.empty((1, 1, 8)), q)


def test_decode_noalloc_validation(lib):
    """fa_decode_noalloc rejects what fa_decode rejects, and partials larger
    than its 16 MiB device array with FA_ERR_WORKSPACE, before touching the
    GPU (these calls run without one)."""
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]

    def dn(B=1, H=32, Nq=16, Nk=64 * 128, d=128, n=64, dtype=2, q=FAKE):
        return lib.fa_decode_noalloc(q, FAKE, FAKE, FAKE, FAKE, B, H, Nq, Nk, d, 0.088, 0, n,
                                     dtype, None)
    assert lib.fa_decode_workspace_size(1, 32, 16, 64 * 128, 128, 64) > (16 << 20)
    assert dn() == -3
    assert dn(q=None, n=1) == -1
    assert dn(Nq=5, Nk=4, n=1) == -1
    assert dn(d=96, n=1) == -2
    assert dn(dtype=0, n=1) == -2
