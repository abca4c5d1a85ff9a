"""GPU parity at the edges of the tiling (through the C ABI), forward and backward.

Shapes that end exactly on, or one past, the 64-row units and 128-row tiles;
a head count that is not a multiple of the eight XCDs (the causal grids map
workgroups to heads round robin); block masks with an empty row (queries that
see no key: O = 0, lse = -inf, dQ = 0) and an empty column (keys no query
sees: dK = dV = 0), alone and combined with causal masking; a scale other
than 1/sqrt(d); the largest block-mask grid (2048 x 2048 tiles) at a ragged
N.  Each case is compared element by element with the fp64 oracle on the
same rounded inputs.
"""

import numpy as np
import pytest
import torch

import oracle
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
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=sc, block_mask=md,
                        n_splits=1)
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
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=sc, block_mask=md, n_splits=1)
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


@pytest.mark.parametrize("causal", [False, True])
def test_largest_mask_grid_block_diagonal(fa, causal):
    """The largest block mask the kernels accept (2048 x 2048 tiles) at a
    ragged N = 262100 (last tile 84 rows), with only the diagonal tiles set.
    Query tile t then sees exactly key tile t, and key tile t receives
    gradient only from query tile t, so every tile is an independent
    attention problem of at most 128 rows: sampled tiles (first, second,
    middle, last two) are compared element by element with the oracle run
    on that tile alone, forward and backward."""
    B, H, N, d, dtype = 1, 2, 262100, 64, "bf16"
    t = -(-N // 128)
    assert t == 2048
    q, k, v, do = W.draw_qkvdo(B, H, N, d, dtype, seed=101)
    sc = W.scale_for(d)
    mask = torch.eye(t, dtype=torch.uint8)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=sc, block_mask=mask.cuda(),
                        n_splits=1)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=sc,
                             block_mask=mask.cuda())
    torch.cuda.synchronize()
    tol = TOL[DT[dtype]]
    for tile in (0, 1, 1023, t - 2, t - 1):
        r = slice(128 * tile, min(N, 128 * (tile + 1)))
        for h in range(H):
            a = [f64(x[0, h, r]) for x in (q, k, v, do)]
            ro, rl = oracle.forward_head(a[0], a[1], a[2], sc, causal=causal)
            rq, rk, rv = oracle.backward_head(*a, sc, causal=causal)
            tag = f"tile {tile} head {h}"
            assert_close(f"o {tag}", f64(o[0, h, r].cpu()), ro, tol)
            assert_close(f"lse {tag}", f64(lse[0, h, r].cpu()), rl, LSE_TOL)
            assert_close(f"dq {tag}", f64(dq[0, h, r].cpu()), rq, tol)
            assert_close(f"dk {tag}", f64(dk[0, h, r].cpu()), rk, tol)
            assert_close(f"dv {tag}", f64(dv[0, h, r].cpu()), rv, tol)
    for x in (o, lse, dq, dk, dv):
        assert torch.isfinite(x).all()
