"""GPU parity of the split-key-range forward (fa_forward_split) against the
fp64 oracle, through the C ABI.

The split forward must give what fa_forward gives: the same attention, here
reached by per-run online softmax plus the logsumexp merge.  Cases cover
automatic and explicit run counts, runs left empty (more runs than a short
causal row has key tiles), ragged N, block-sparse masks whose runs hold no
kept tile, both head dimensions and all three input types.
"""

import pytest
import torch

from exact_io_aware_34_amd import workloads as W
from tests.parity import (DT, LSE_TOL, TOL, assert_close, f64, oracle_forward_heads,
                          random_block_mask)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    from exact_io_aware_34_amd import fa as _fa
    return _fa


def run_split(fa, q, k, v, scale, causal, mask, n_splits):
    dev = "cuda"
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    md = None if mask is None else mask.to(dev)
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale, block_mask=md,
                        n_splits=n_splits)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


CASES = [
    # B, H, N, d, dtype, causal, sparse, n_splits (0 = library's choice)
    (1, 1, 4096, 64, "bf16", False, False, 0),
    (1, 1, 4096, 64, "bf16", True, False, 0),
    (1, 2, 1000, 64, "f16", True, False, 5),
    (1, 1, 300, 64, "bf16", True, False, 64),    # capped at 5 key tiles; short rows get empty runs
    (2, 1, 130, 64, "bf16", False, False, 3),
    (1, 2, 1000, 64, "bf16", False, True, 7),    # runs with no kept tile
    (1, 1, 1500, 64, "f16", True, True, 0),
    (1, 2, 777, 128, "bf16", False, False, 0),
    (1, 1, 900, 128, "f16", True, False, 4),
    (1, 1, 1000, 128, "bf16", True, True, 6),
    (1, 1, 64, 64, "bf16", True, False, 2),      # one key tile: one run
    (1, 1, 4096, 64, "f32", False, False, 0),
    (1, 2, 700, 64, "f32", True, False, 4),
    (1, 1, 1000, 128, "f32", True, True, 5),
    (1, 1, 333, 128, "f32", False, False, 3),
]


@pytest.mark.parametrize("B,H,N,d,dtype,causal,sparse,n_splits", CASES)
def test_split_forward(fa, B, H, N, d, dtype, causal, sparse, n_splits):
    q, k, v, _ = W.draw_qkvdo(B, H, N, d, dtype, seed=N * 7 + d + n_splits)
    mask = random_block_mask(N, 0.3, seed=N + 3) if sparse else None
    scale = W.scale_for(d)
    o, lse = run_split(fa, q, k, v, scale, causal, mask, n_splits)
    heads = [(b, h) for b in range(B) for h in range(H)]
    tol = TOL[DT[dtype]]
    for (b, h), (ro, rl) in zip(heads, oracle_forward_heads(q, k, v, scale, causal, mask, heads)):
        assert_close(f"o[{b},{h}]", f64(o[b, h]), ro, tol)
        assert_close(f"lse[{b},{h}]", f64(lse[b, h]), rl, LSE_TOL)


def test_split_counts_agree(fa):
    """Every run count gives the plain forward's result within rounding."""
    B, H, N, d = 1, 2, 2000, 64
    q, k, v, _ = W.draw_qkvdo(B, H, N, d, "bf16", seed=99)
    scale = W.scale_for(d)
    dev = "cuda"
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o1, l1 = fa.forward(qd, kd, vd, causal=True, scale=scale, n_splits=1)
    for n in (2, 3, 8, 31):
        on, ln = fa.forward(qd, kd, vd, causal=True, scale=scale, n_splits=n)
        torch.cuda.synchronize()
        assert fa.forward_splits(B, H, N, d, n) == n
        assert_close(f"o n={n}", f64(on), f64(o1), 2 * TOL[torch.bfloat16])
        assert_close(f"lse n={n}", f64(ln), f64(l1), LSE_TOL)


@pytest.mark.parametrize("name", ["dense_n4096_d64_bf16", "dense_n4096_d64_f32",
                                  "dense_n256_d64_f32"])
def test_split_named_small_workload(fa, name):
    """The single-head workloads (32 query tiles at N = 4096, two at N = 256
    in fp32) in the configuration the benchmark times for them
    (library-chosen run count)."""
    w = W.make(name)
    wl = w["workload"]
    assert fa.forward_splits(wl.B, wl.H, wl.N, wl.d, 0, w["q"].dtype) > 1
    o, lse = run_split(fa, w["q"], w["k"], w["v"], w["scale"], w["causal"], w["mask"], 0)
    (ro, rl), = oracle_forward_heads(w["q"], w["k"], w["v"], w["scale"], w["causal"],
                                     w["mask"], [(0, 0)])
    assert_close("o", f64(o[0, 0]), ro, TOL[w["q"].dtype])
    assert_close("lse", f64(lse[0, 0]), rl, LSE_TOL)


def test_split_rejects_dropout(fa):
    q = torch.zeros((1, 1, 256, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fa.forward(q, q, q, dropout_p=0.1, n_splits=2)


def test_default_forward_splits_small_grids(fa):
    """fa.forward's default (n_splits = 0) is the library's choice: a single
    head of N = 4096 (32 workgroups) runs split key ranges, bit for bit the
    explicit n_splits = 0 call, and a full grid runs the plain forward."""
    q, k, v, _ = W.draw_qkvdo(1, 1, 4096, 64, "bf16", seed=5)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    assert fa.forward_splits(1, 1, 4096, 64, 0) > 1
    o0, l0 = fa.forward(qd, kd, vd)
    o1, l1 = fa.forward(qd, kd, vd, n_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert fa.forward_splits(4, 12, 8192, 64, 0) == 1
