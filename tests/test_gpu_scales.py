"""GPU parity at softmax scales away from 1/sqrt(d) (through the C ABI).

The flat bars of the other parity tests are sized for the workloads' scale
1/sqrt(d).  A larger scale concentrates each softmax row on few keys, and
the outputs and gradients grow with it (|dq| reaches ~25 at scale 1), so
the inputs' 16-bit rounding alone passes the flat bar there.  These cases
compare every element with the fp64 oracle against per-element bounds
derived from the kernels' arithmetic (tests.parity.forward_bound and
backward_bound: P and dS rounded to the input type, everything else in
fp32).  The backward is handed the oracle's O rounded to the input type
and its lse rounded to fp32, so its inputs come from the oracle alone; the
forward is run plain and with split key runs.
"""

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_34_amd import workloads as W
from tests.parity import (DT, LSE_TOL, assert_within, backward_bound, f64, forward_bound,
                          max_abs, random_block_mask)

pytestmark = pytest.mark.gpu

CASES = [
    # N, d, dtype, causal, sparse, scale
    (700, 128, "bf16", False, False, 0.3),
    (513, 64, "f16", True, False, 0.5),
    (300, 64, "bf16", True, False, 1.0),
    (450, 128, "f16", True, True, 0.05),
    (333, 128, "bf16", True, True, 0.6),
    (257, 64, "f32", True, False, 0.3),
    (129, 128, "f32", False, False, 0.02),
]


@pytest.fixture(scope="module")
def fa():
    from exact_io_aware_34_amd import fa as _fa
    return _fa


@pytest.mark.parametrize("N,d,dtype,causal,sparse,scale", CASES)
def test_scale(fa, N, d, dtype, causal, sparse, scale):
    dt = DT[dtype]
    q, k, v, do = W.draw_qkvdo(1, 1, N, d, dtype, seed=N + d)
    mask = random_block_mask(N, 0.4, seed=N) if sparse else None
    mnp = None if mask is None else mask.numpy()
    a = [f64(t[0, 0]) for t in (q, k, v, do)]
    t = oracle.backward_head_terms(*a, scale, causal, mnp)
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    md = None if mask is None else mask.cuda()
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale, block_mask=md, n_splits=1)
    so, slse = fa.forward(qd, kd, vd, causal=causal, scale=scale, block_mask=md, n_splits=3)
    o_in = torch.from_numpy(t["o"]).to(dt)[None, None]
    lse_in = torch.from_numpy(t["lse"]).float()[None, None]
    grads = None
    if dtype != "f32":
        grads = fa.backward(qd, kd, vd, o_in.cuda(), lse_in.cuda(), dod, causal=causal,
                            scale=scale, block_mask=md)
    torch.cuda.synchronize()
    fb = forward_bound(t, *a[:3], scale, dt)
    r = [assert_within("o", f64(o[0, 0]), t["o"], fb),
         assert_within("split o", f64(so[0, 0]), t["o"], fb)]
    assert max_abs(f64(lse[0, 0]), t["lse"]) <= LSE_TOL
    assert max_abs(f64(slse[0, 0]), t["lse"]) <= LSE_TOL
    if grads is not None:
        g = oracle.backward_head(*a, scale, causal, mnp)
        bounds = backward_bound(t, *a, f64(o_in[0, 0]), scale, dt)
        for name, got, ref, bnd in zip(("dq", "dk", "dv"), grads, g, bounds):
            r.append(assert_within(name, f64(got[0, 0]), ref, bnd))
    print("worst |err| / bound:", [f"{x:.2f}" for x in r], flush=True)


DROP_CASES = [
    # N, d, dtype, causal, sparse, scale, p
    (400, 128, "bf16", False, False, 0.3, 0.2),
    (333, 64, "f16", True, True, 0.6, 0.1),
    (257, 64, "bf16", True, False, 1.0, 0.3),
]


@pytest.mark.parametrize("N,d,dtype,causal,sparse,scale,p", DROP_CASES)
def test_scale_dropout(fa, N, d, dtype, causal, sparse, scale, p):
    """Fused dropout at the same large scales, against the same per-element
    bounds with the keep mask times 1 / (1 - p) where the kernels apply it;
    the backward is handed the oracle's O (as the fp32 output it takes) and
    lse."""
    dt = DT[dtype]
    seed, offset = 90210 + N, 4
    q, k, v, do = W.draw_qkvdo(1, 1, N, d, dtype, seed=N + d + 1)
    mask = random_block_mask(N, 0.4, seed=N + 1) if sparse else None
    mnp = None if mask is None else mask.numpy()
    a = [f64(t[0, 0]) for t in (q, k, v, do)]
    t = oracle.backward_head_dropout_terms(*a, scale, p, seed, offset, 0, causal, mnp)
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    md = None if mask is None else mask.cuda()
    o_acc = torch.empty(qd.shape, dtype=torch.float32, device="cuda")
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale, block_mask=md, dropout_p=p,
                        seed=seed, offset=offset, o_acc=o_acc)
    o_in = torch.from_numpy(t["o"]).float()[None, None].cuda()
    lse_in = torch.from_numpy(t["lse"]).float()[None, None].cuda()
    grads = fa.backward(qd, kd, vd, o, lse_in, dod, causal=causal, scale=scale, block_mask=md,
                        dropout_p=p, seed=seed, offset=offset, o_acc=o_in)
    torch.cuda.synchronize()
    r = [assert_within("o", f64(o[0, 0]), t["o"], forward_bound(t, *a[:3], scale, dt)),
         assert_within("o_acc", f64(o_acc[0, 0]), t["o"],
                       forward_bound(t, *a[:3], scale, dt, out_rounded=False))]
    assert max_abs(f64(lse[0, 0]), t["lse"]) <= LSE_TOL
    g = oracle.backward_head_dropout(*a, scale, p, seed, offset, 0, causal, mnp)
    bounds = backward_bound(t, *a, f64(o_in[0, 0]), scale, dt)
    for name, got, ref, bnd in zip(("dq", "dk", "dv"), grads, g, bounds):
        r.append(assert_within(name, f64(got[0, 0]), ref, bnd))
    print("worst |err| / bound:", [f"{x:.2f}" for x in r], flush=True)
