"""GPU parity at the edges of the tiling (through the C ABI), forward and backward.

Shapes that end exactly on, or one past, the 64-row units and 128-row tiles;
a head count that is not a multiple of the eight XCDs (the causal grids map
workgroups to heads round robin); block masks with an empty row (queries that
see no key: O = 0, lse = -inf, dQ = 0) and an empty column (keys no query
sees: dK = dV = 0), alone and combined with causal masking; a scale other
than 1/sqrt(d).  Each case is compared element by element with the fp64
oracle on the same rounded inputs.
"""

import numpy as np
import pytest
import torch

from exact_io_aware_34_amd import workloads as W
from tests.parity import (DT, LSE_TOL, TOL, assert_close, f64, oracle_backward_heads,
                          oracle_forward_heads)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    from exact_io_aware_34_amd import fa as _fa
    return _fa


def holed_mask(N, seed):
    """Dense 128x128 tile mask with one empty row and one empty column."""
    t = -(-N // 128)
    g = torch.Generator().manual_seed(seed)
    m = (torch.rand((t, t), generator=g) < 0.7).to(torch.uint8)
    m[0, :] = 0                    # query tile 0 sees nothing
    m[:, t - 1] = 0                # nobody sees the last key tile
    if t > 2:
        m[1, 1] = 1                # keep some work on the diagonal
    return m


CASES = [
    # B, H, N, d, dtype, causal, mask, scale (None = 1/sqrt(d))
    (1, 1, 64, 64, "bf16", True, None, None),
    (1, 1, 65, 64, "bf16", False, None, None),
    (1, 2, 192, 64, "bf16", True, None, None),
    (1, 1, 256, 64, "f16", False, None, 0.3),
    (2, 5, 320, 64, "f16", True, None, None),
    (1, 2, 384, 64, "bf16", False, "holed", None),
    (1, 2, 384, 64, "bf16", True, "holed", None),
    (1, 1, 449, 64, "f16", True, "holed", None),
    (1, 2, 300, 128, "bf16", True, "holed", None),
    (1, 1, 256, 128, "f16", False, None, 0.3),
]


def _inputs(B, H, N, d, dtype, mask_kind, scale):
    q, k, v, do = W.draw_qkvdo(B, H, N, d, dtype, seed=7 * N + d + B * H)
    mask = holed_mask(N, seed=N) if mask_kind == "holed" else None
    return q, k, v, do, mask, (W.scale_for(d) if scale is None else scale)


@pytest.mark.parametrize("B,H,N,d,dtype,causal,mask_kind,scale", CASES)
def test_edges_forward(fa, B, H, N, d, dtype, causal, mask_kind, scale):
    q, k, v, do, mask, sc = _inputs(B, H, N, d, dtype, mask_kind, scale)
    md = None if mask is None else mask.cuda()
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=sc, block_mask=md)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    heads = [(b, h) for b in range(B) for h in range(H)]
    for (b, h), (ro, rl) in zip(heads, oracle_forward_heads(q, k, v, sc, causal, mask, heads)):
        assert_close(f"o[{b},{h}]", f64(o[b, h]), ro, TOL[DT[dtype]])
        assert_close(f"lse[{b},{h}]", f64(lse[b, h]), rl, LSE_TOL)
    if mask_kind == "holed":
        # Query tile 0 sees no key: exact zeros and -inf, not merely small values.
        assert torch.all(o[:, :, :128] == 0)
        assert torch.all(torch.isneginf(lse[:, :, :128]))


@pytest.mark.parametrize("B,H,N,d,dtype,causal,mask_kind,scale", CASES)
def test_edges_backward(fa, B, H, N, d, dtype, causal, mask_kind, scale):
    q, k, v, do, mask, sc = _inputs(B, H, N, d, dtype, mask_kind, scale)
    md = None if mask is None else mask.cuda()
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=sc, block_mask=md)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=sc, block_mask=md)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    heads = [(b, h) for b in range(B) for h in range(H)]
    tol = TOL[DT[dtype]]
    for (b, h), (rq, rk, rv) in zip(heads, oracle_backward_heads(q, k, v, do, sc, causal, mask,
                                                                 heads)):
        assert_close(f"dq[{b},{h}]", f64(dq[b, h]), rq, tol)
        assert_close(f"dk[{b},{h}]", f64(dk[b, h]), rk, tol)
        assert_close(f"dv[{b},{h}]", f64(dv[b, h]), rv, tol)
    if mask_kind == "holed":
        t = -(-N // 128)
        assert torch.all(dq[:, :, :128] == 0)
        assert torch.all(dk[:, :, (t - 1) * 128:] == 0)
        assert torch.all(dv[:, :, (t - 1) * 128:] == 0)
    assert np.isfinite(dq.numpy()).all() and np.isfinite(dk.numpy()).all()
