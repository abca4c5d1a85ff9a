"""Thin Python binding of libfa.so, the gfx950 attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/fa.h``.  torch provides device memory and
the current stream.  Importing this module raises ImportError when the
library has not been built (there is no other code path).

    from exact_io_aware_34_amd import fa
    o, lse = fa.forward(q, k, v, causal=True)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=True)
    o, lse = fa.forward(q, k, v, n_splits=0)          # split key runs for small grids
    o, lse = fa.decode(q_new, k_cache, v_cache)        # Nq <= 16 queries, Nk keys
    o, lse = fa.forward_fp8(q, k, v, signs=signs, causal=True)   # E4M3 operands
"""

import ctypes
import functools
import os

import torch  # loads torch's HIP runtime first, so libfa.so binds to the same one

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libfa.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing; build it with `python -m exact_io_aware_34_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
_lib.fa_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _i, _vp]
_lib.fa_forward.restype = _i
_lib.fa_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _i, _i, _i, _i, _f, _i, _vp, _i, _vp, ctypes.c_size_t, _vp]
_lib.fa_backward.restype = _i
_lib.fa_backward_workspace_size.argtypes = [_i, _i, _i, _i]
_lib.fa_backward_workspace_size.restype = ctypes.c_size_t
_lib.fa_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _i, _vp,
                           ctypes.c_size_t, _vp]
_lib.fa_decode.restype = _i
_lib.fa_decode_splits.argtypes = [_i, _i, _i, _i, _i, _i]
_lib.fa_decode_splits.restype = _i
_lib.fa_decode_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i]
_lib.fa_decode_workspace_size.restype = ctypes.c_size_t
_lib.fa_forward_fp8.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _i, _vp, _vp,
                                ctypes.c_size_t, _vp]
_lib.fa_forward_fp8.restype = _i
_lib.fa_fp8_prepare.argtypes = [_vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp, ctypes.c_size_t,
                                _vp]
_lib.fa_fp8_prepare.restype = _i
_lib.fa_forward_fp8_workspace_size.argtypes = [_i, _i, _i, _i]
_lib.fa_forward_fp8_workspace_size.restype = ctypes.c_size_t
_u64, _u32 = ctypes.c_uint64, ctypes.c_uint32
_lib.fa_forward_dropout.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _i, _f,
                                    _u64, _u32, _vp, _vp]
_lib.fa_forward_dropout.restype = _i
_lib.fa_backward_dropout.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                                     _f, _i, _vp, _i, _f, _u64, _u32, _vp, ctypes.c_size_t, _vp]
_lib.fa_backward_dropout.restype = _i
_lib.fa_dropout_mask.argtypes = [_i, _i, _i, _f, _u64, _u32, _vp, _vp]
_lib.fa_dropout_mask.restype = _i
_lib.fa_forward_split.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _i, _i, _vp,
                                  ctypes.c_size_t, _vp]
_lib.fa_forward_split.restype = _i
_lib.fa_forward_splits.argtypes = [_i, _i, _i, _i, _i, _i]
_lib.fa_forward_splits.restype = _i
_lib.fa_forward_split_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i]
_lib.fa_forward_split_workspace_size.restype = ctypes.c_size_t
_lib.fa_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _i,
                                   _vp]
_lib.fa_decode_noalloc.restype = _i
_lib.fa_status_string.argtypes = [_i]
_lib.fa_status_string.restype = ctypes.c_char_p
_lib.fa_abi_version.restype = _i

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
DTYPE_CODES = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
MASK_BLOCK = 128


class FAError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"libfa status {status}: {status_string(status)}")


def status_string(status: int) -> str:
    return _lib.fa_status_string(status).decode()


def abi_version() -> int:
    return _lib.fa_abi_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_inputs(*ts):
    ref = ts[0]
    if ref.dim() != 4:
        raise ValueError("tensors must be (batch, heads, seq, head_dim)")
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU")
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError("q, k, v (and o, dO) must share shape and dtype")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if ref.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {ref.dtype}")


def _check_f32(t, shape, name):
    """A caller-supplied fp32 GPU tensor the kernels write or read in full."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous float32 of shape {tuple(shape)}")


def _check_workspace(workspace):
    if workspace is None:
        return 0
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise ValueError("workspace must be a GPU tensor")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace.numel() * workspace.element_size()


def _mask_arg(block_mask, n):
    if block_mask is None:
        return None
    t = -(-n // MASK_BLOCK)
    if block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != (t, t):
        raise ValueError(f"block_mask must be uint8 of shape ({t}, {t})")
    if not block_mask.is_cuda or not block_mask.is_contiguous():
        raise ValueError("block_mask must be a contiguous GPU tensor")
    return block_mask


@functools.lru_cache(maxsize=256)
def default_scale(d: int) -> float:
    return float(torch.tensor(d ** -0.5, dtype=torch.float32))


def _dtype_code(dtype):
    if dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {dtype}")
    return DTYPE_CODES[dtype]


@functools.lru_cache(maxsize=256)
def forward_splits(B, H, N, d, n_splits=0, dtype=torch.bfloat16) -> int:
    """Number of key runs fa_forward_split uses for this shape and input dtype
    (0 on bad input)."""
    return int(_lib.fa_forward_splits(B, H, N, d, n_splits, _dtype_code(dtype)))


def fa_forward_splits_used(B, H, N, d, n_splits, dtype=torch.bfloat16) -> int:
    """Key runs fa_forward_split would use (1 when the plain forward runs)."""
    return forward_splits(B, H, N, d, n_splits, dtype) if n_splits != 1 else 1


@functools.lru_cache(maxsize=256)
def forward_split_workspace_size(B, H, N, d, n_splits=0, dtype=torch.bfloat16) -> int:
    return int(_lib.fa_forward_split_workspace_size(B, H, N, d, n_splits, _dtype_code(dtype)))


def forward(q, k, v, causal=False, scale=None, block_mask=None, out=None, lse=None,
            stream=None, dropout_p=0.0, seed=0, offset=0, n_splits=0, workspace=None,
            o_acc=None):
    """Exact attention forward: returns (o, lse) with o in q's dtype, lse fp32.
    dropout_p > 0 drops probabilities with the mask fa_dropout_mask describes;
    `o_acc` (fp32, q's shape) then receives O before its rounding to q's
    dtype, which the dropout backward needs.  Without dropout the call is
    fa_forward_split: n_splits = 0 (default) lets the library split the key
    range of grids too small to fill the GPU (one run, i.e. fa_forward, for
    every other grid), 1 never splits, > 1 asks for that many runs; a
    block-sparse call without the causal flag also takes fa_forward_split,
    whose workspace holds its query-tile work order.  `workspace` is
    allocated here when None and needed."""
    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    mask = _mask_arg(block_mask, N)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_inputs(q, o)
    _check_f32(lse, (B, H, N), "lse")
    if o_acc is not None:
        _check_f32(o_acc, (B, H, N, d), "o_acc")
    drop = bool(dropout_p) or o_acc is not None
    if drop and n_splits not in (0, 1):
        raise ValueError("split key runs are not offered with dropout")
    # fa_forward_split also takes the block-sparse (not causal) forward, whose
    # workspace holds the query-tile work order.
    ordered = mask is not None and not causal and q.dtype != torch.float32
    if not drop and (ordered or fa_forward_splits_used(B, H, N, d, n_splits, q.dtype) > 1):
        ws_bytes = forward_split_workspace_size(B, H, N, d, n_splits, q.dtype)
        if workspace is None and ws_bytes > 0:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        nbytes = _check_workspace(workspace)
        rc = _lib.fa_forward_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                   scale, int(bool(causal)), _ptr(mask), DTYPE_CODES[q.dtype],
                                   int(n_splits), _ptr(workspace), nbytes, _stream(stream))
    elif drop:
        rc = _lib.fa_forward_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                     scale, int(bool(causal)), _ptr(mask), DTYPE_CODES[q.dtype],
                                     float(dropout_p), int(seed), int(offset), _ptr(o_acc),
                                     _stream(stream))
    else:
        rc = _lib.fa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                             scale, int(bool(causal)), _ptr(mask), DTYPE_CODES[q.dtype],
                             _stream(stream))
    if rc != 0:
        raise FAError(rc)
    return o, lse


@functools.lru_cache(maxsize=256)
def workspace_size(B, H, N, d) -> int:
    return int(_lib.fa_backward_workspace_size(B, H, N, d))


def backward(q, k, v, o, lse, do, causal=False, scale=None, block_mask=None,
             workspace=None, grads=None, stream=None, dropout_p=0.0, seed=0, offset=0,
             o_acc=None):
    """Exact attention backward: returns fp32 (dq, dk, dv).  With dropout,
    pass the forward's (dropout_p, seed, offset) so the same mask applies, and
    its fp32 output `o_acc` (required then; `o` is not read)."""
    _check_inputs(q, k, v, o, do)
    B, H, N, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    mask = _mask_arg(block_mask, N)
    _check_f32(lse, (B, H, N), "lse")
    drop = bool(dropout_p) or o_acc is not None
    if drop:
        if o_acc is None:
            raise ValueError("the dropout backward needs the forward's fp32 output o_acc")
        _check_f32(o_acc, (B, H, N, d), "o_acc")
    if grads is None:
        grads = tuple(torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
                      for _ in range(3))
    if len(grads) != 3:
        raise ValueError("grads must be a (dq, dk, dv) tuple")
    for name, g in zip(("dq", "dk", "dv"), grads):
        _check_f32(g, (B, H, N, d), name)
    ws_bytes = workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    dq, dk, dv = grads
    ws_n = _check_workspace(workspace)
    if drop:
        rc = _lib.fa_backward_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o_acc), _ptr(do),
                                      _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, scale,
                                      int(bool(causal)), _ptr(mask), DTYPE_CODES[q.dtype],
                                      float(dropout_p), int(seed), int(offset), _ptr(workspace),
                                      ws_n, _stream(stream))
    else:
        rc = _lib.fa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                              _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, scale,
                              int(bool(causal)), _ptr(mask), DTYPE_CODES[q.dtype],
                              _ptr(workspace), ws_n, _stream(stream))
    if rc != 0:
        raise FAError(rc)
    return dq, dk, dv


@functools.lru_cache(maxsize=256)
def decode_splits(B, H, Nq, Nk, d, n_splits=0) -> int:
    """Number of key ranges fa_decode uses for this shape (0 on bad input)."""
    return int(_lib.fa_decode_splits(B, H, Nq, Nk, d, n_splits))


@functools.lru_cache(maxsize=256)
def decode_workspace_size(B, H, Nq, Nk, d, n_splits=0) -> int:
    return int(_lib.fa_decode_workspace_size(B, H, Nq, Nk, d, n_splits))


def decode(q, k, v, causal=False, scale=None, n_splits=0, out=None, lse=None, workspace=None,
           stream=None):
    """Decode attention: q (B, H, Nq, d) are the last Nq positions of the
    (B, H, Nk, d) cached keys and values.  Returns (o, lse) like forward()."""
    for t in (q, k, v):
        if t.dim() != 4 or not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous 4-d GPU tensors of one dtype")
    B, H, Nq, d = q.shape
    if tuple(k.shape[:2]) != (B, H) or k.shape[3] != d or k.shape != v.shape:
        raise ValueError("k and v must be (B, H, Nk, d) matching q")
    if q.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    Nk = k.shape[2]
    scale = default_scale(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous():
        raise ValueError("out must be contiguous, shaped and typed like q")
    _check_f32(lse, (B, H, Nq), "lse")
    ws_bytes = decode_workspace_size(B, H, Nq, Nk, d, n_splits)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    nbytes = _check_workspace(workspace)
    rc = _lib.fa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d, scale,
                        int(bool(causal)), int(n_splits), DTYPE_CODES[q.dtype], _ptr(workspace),
                        nbytes, _stream(stream))
    if rc != 0:
        raise FAError(rc)
    return o, lse


NOALLOC_SCRATCH_BYTES = 16 << 20   # FA_NOALLOC_SCRATCH_BYTES of fa.h


def decode_noalloc(q, k, v, causal=False, scale=None, n_splits=0, out=None, lse=None,
                   stream=None):
    """decode() through fa_decode_noalloc: the key-range partials live in the
    library's own device array, so the call allocates nothing on the device
    (pass `out` and `lse` to allocate nothing here either).  Calls that
    overlap on one GPU share that array and race."""
    for t in (q, k, v):
        if t.dim() != 4 or not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous 4-d GPU tensors of one dtype")
    B, H, Nq, d = q.shape
    if tuple(k.shape[:2]) != (B, H) or k.shape[3] != d or k.shape != v.shape:
        raise ValueError("k and v must be (B, H, Nk, d) matching q")
    if q.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    Nk = k.shape[2]
    scale = default_scale(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    if o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() or not o.is_cuda:
        raise ValueError("out must be a contiguous GPU tensor shaped and typed like q")
    _check_f32(lse, (B, H, Nq), "lse")
    rc = _lib.fa_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nk, d,
                                scale, int(bool(causal)), int(n_splits), DTYPE_CODES[q.dtype],
                                _stream(stream))
    if rc != 0:
        raise FAError(rc)
    return o, lse


@functools.lru_cache(maxsize=256)
def fp8_workspace_size(B, H, N, d) -> int:
    return int(_lib.fa_forward_fp8_workspace_size(B, H, N, d))


def _fp8_args(q, k, v, signs, workspace):
    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    if signs is not None:
        if signs.dtype != torch.int8 or tuple(signs.shape) != (d,) or not signs.is_cuda:
            raise ValueError(f"signs must be an int8 GPU tensor of shape ({d},)")
        if not signs.is_contiguous() or signs.data_ptr() % 16:
            raise ValueError("signs must be contiguous and 16-byte aligned")
    ws_bytes = fp8_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    _check_workspace(workspace)
    return workspace


def fp8_prepare(q, k, v, signs=None, scale=None, workspace=None, stream=None):
    """Rotation + block quantisation only, for softmax scale `scale` (default
    1/sqrt(d)); returns the filled workspace."""
    workspace = _fp8_args(q, k, v, signs, workspace)
    B, H, N, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    rc = _lib.fa_fp8_prepare(_ptr(q), _ptr(k), _ptr(v), B, H, N, d, scale, DTYPE_CODES[q.dtype],
                             _ptr(signs), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != 0:
        raise FAError(rc)
    return workspace


def fp8_views(workspace, B, H, N, d):
    """Views of the workspace regions in the layout fa.h documents:
    (q8, k8, v8t) as uint8 and (s_q, s_k, s_v) as float32."""
    nt = -(-N // 64)
    pad = lambda b: -(-b // 256) * 256  # noqa: E731
    op, sc = pad(B * H * nt * 64 * d), pad(B * H * nt * 4)
    ws = workspace.view(torch.uint8)
    q8 = ws[0:B * H * nt * 64 * d].view(B, H, nt * 64, d)
    k8 = ws[op:op + B * H * nt * 64 * d].view(B, H, nt * 64, d)
    v8t = ws[2 * op:2 * op + B * H * nt * 64 * d].view(B, H, nt, d, 64)
    scales = [ws[3 * op + i * sc:3 * op + i * sc + B * H * nt * 4].view(torch.float32).view(B, H, nt)
              for i in range(3)]
    return (q8, k8, v8t), tuple(scales)


def forward_fp8(q, k, v, signs=None, causal=False, scale=None, block_mask=None, out=None,
                lse=None, workspace=None, stream=None):
    """FP8 forward with incoherent processing: returns (o, lse) like forward()."""
    workspace = _fp8_args(q, k, v, signs, workspace)
    B, H, N, d = q.shape
    scale = default_scale(d) if scale is None else float(scale)
    mask = _mask_arg(block_mask, N)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_inputs(q, o)
    _check_f32(lse, (B, H, N), "lse")
    rc = _lib.fa_forward_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, scale,
                             int(bool(causal)), _ptr(mask), DTYPE_CODES[q.dtype], _ptr(signs),
                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream))
    if rc != 0:
        raise FAError(rc)
    return o, lse


def dropout_mask(B, H, N, dropout_p, seed=0, offset=0, device="cuda", stream=None):
    """The keep mask (B, H, N, N) uint8 that forward/backward apply."""
    keep = torch.empty((B, H, N, N), dtype=torch.uint8, device=device)
    rc = _lib.fa_dropout_mask(B, H, N, float(dropout_p), int(seed), int(offset), _ptr(keep),
                              _stream(stream))
    if rc != 0:
        raise FAError(rc)
    return keep
