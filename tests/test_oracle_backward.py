"""Pins for the oracle's backward pass (oracle/attention.py).

The pages only say that the backward pass recomputes S and P from Q, K and
the saved statistics; the gradient formulas are the softmax chain rule.  They
are pinned here by central finite differences of L = sum(dO * O) in float64,
by torch autograd through torch's own attention routine, by closed-form
special cases and by invariants that hold at any size.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import backward_head, forward_head

RNG = np.random.default_rng(4321)


def randn(*shape):
    return RNG.standard_normal(shape)


def loss(q, k, v, do, scale, causal, bm, mb):
    o, _ = forward_head(q, k, v, scale, causal=causal, block_mask=bm, mask_block=mb)
    return float(np.sum(do * o))


def finite_difference_grads(q, k, v, do, scale, causal, bm, mb, h=1e-5):
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(g.shape):
            x0 = args[which][idx]
            args[which][idx] = x0 + h
            lp = loss(*args, do, scale, causal, bm, mb)
            args[which][idx] = x0 - h
            lm = loss(*args, do, scale, causal, bm, mb)
            args[which][idx] = x0
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


CASES = [
    # n, d, causal, masked
    (16, 8, False, False),
    (16, 8, True, False),
    (16, 8, False, True),
    (13, 8, True, True),
    (16, 64, True, False),
]


@pytest.mark.parametrize("n,d,causal,masked", CASES)
def test_gradients_match_finite_differences(n, d, causal, masked):
    q, k, v, do = randn(n, d), randn(n, d), randn(n, d), randn(n, d)
    mb, bm = 4, None
    if masked:
        t = -(-n // mb)
        bm = (np.random.default_rng(n).random((t, t)) < 0.5).astype(np.uint8)
        np.fill_diagonal(bm, 1)
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv = backward_head(q, k, v, do, scale, causal, bm, mb, chunk=5)
    fq, fk, fv = finite_difference_grads(q, k, v, do, scale, causal, bm, mb)
    for got, ref in ((dq, fq), (dk, fk), (dv, fv)):
        err = np.max(np.abs(got - ref)) / max(1e-12, np.max(np.abs(ref)))
        assert err <= 1e-6, err


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_gradients_match_torch_autograd_fp64(causal, masked):
    n, d, mb = 160, 16, 32
    q, k, v, do = randn(n, d), randn(n, d), randn(n, d), randn(n, d)
    bm = None
    if masked:
        bm = (np.random.default_rng(8).random((5, 5)) < 0.4).astype(np.uint8)
        np.fill_diagonal(bm, 1)
    dq, dk, dv = backward_head(q, k, v, do, 0.3, causal, bm, mb, chunk=37)
    ok = torch.from_numpy(oracle.allowed(np.arange(n), n, causal, bm, mb))
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq[None], tk[None], tv[None], attn_mask=ok[None], scale=0.3)[0]
    o.backward(torch.from_numpy(do))
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def test_gradient_invariants():
    """sum_j dK_j = 0, sum_j dV_j = sum_i dO_i, D_i = sum_j P_ij dP_ij."""
    n, d = 300, 32
    q, k, v, do = randn(n, d), randn(n, d), randn(n, d), randn(n, d)
    for causal in (False, True):
        dq, dk, dv = backward_head(q, k, v, do, 0.2, causal, chunk=64)
        np.testing.assert_allclose(dk.sum(axis=0), 0.0, rtol=0, atol=1e-11)
        np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), rtol=0, atol=1e-11)
        o, lse = forward_head(q, k, v, 0.2, causal=causal)
        s = 0.2 * (q @ k.T)
        ok = oracle.allowed(np.arange(n), n, causal)
        p = np.where(ok, np.exp(s - lse[:, None]), 0.0)
        dp = do @ v.T
        np.testing.assert_allclose(oracle.rowsum_do_o(do, o), (p * dp).sum(axis=1),
                                   rtol=0, atol=1e-12)


def test_single_token_gradients():
    q, k, v, do = randn(1, 64), randn(1, 64), randn(1, 64), randn(1, 64)
    dq, dk, dv = backward_head(q, k, v, do, 0.125)
    assert np.max(np.abs(dq)) <= 1e-13 and np.max(np.abs(dk)) <= 1e-13
    np.testing.assert_allclose(dv, do, rtol=0, atol=1e-15)


def test_identical_keys_and_constant_values():
    n, d = 100, 16
    q, v, do = randn(n, d), randn(n, d), randn(n, d)
    k = np.tile(randn(1, d), (n, 1))
    for causal in (False, True):
        dq, _, _ = backward_head(q, k, v, do, 0.25, causal)
        assert np.max(np.abs(dq)) <= 1e-13       # scores don't depend on which key
    k = randn(n, d)
    vc = np.tile(randn(1, d), (n, 1))
    for causal in (False, True):
        dq, dk, _ = backward_head(q, k, vc, do, 0.25, causal)
        assert np.max(np.abs(dq)) <= 1e-13 and np.max(np.abs(dk)) <= 1e-13


def test_fully_masked_rows_contribute_nothing():
    n, d, mb = 8, 4, 4
    mask = np.array([[0, 0], [1, 1]], np.uint8)
    q, k, v, do = randn(n, d), randn(n, d), randn(n, d), randn(n, d)
    dq, dk, dv = backward_head(q, k, v, do, 0.5, False, mask, mb)
    assert np.all(dq[:4] == 0)
    do2 = do.copy()
    do2[:4] = 1e3 * randn(4, d)                  # upstream grads of empty rows are ignored
    _, dk2, dv2 = backward_head(q, k, v, do2, 0.5, False, mask, mb)
    np.testing.assert_allclose(dk, dk2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, dv2, rtol=0, atol=1e-13)


def test_batched_wrapper_matches_heads():
    shp = (2, 2, 30, 8)
    q, k, v, do = randn(*shp), randn(*shp), randn(*shp), randn(*shp)
    g = oracle.backward(q, k, v, do, 0.3, causal=True)
    for b in range(2):
        for h in range(2):
            gh = backward_head(q[b, h], k[b, h], v[b, h], do[b, h], 0.3, True)
            for x, y in zip(g, gh):
                np.testing.assert_array_equal(x[b, h], y)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("chunk", [7, 64, 500])
def test_sampled_gradients_match_torch_autograd_fp64(causal, masked, chunk):
    """backward_head_sampled at sampled query rows and key columns against
    torch autograd through its attention routine (an independent route),
    including chunks that hold no sampled row and see no sampled key."""
    n, d, mb = 200, 16, 32
    q, k, v, do = randn(n, d), randn(n, d), randn(n, d), randn(n, d)
    bm = None
    if masked:
        bm = (np.random.default_rng(9).random((7, 7)) < 0.3).astype(np.uint8)
        np.fill_diagonal(bm, 1)
    rows = np.array([0, 1, 63, 64, 150, 199])
    cols = np.array([0, 5, 31, 32, 130, 199])
    dq, dk, dv = oracle.backward_head_sampled(q, k, v, do, 0.3, causal, bm, rows, cols, mb,
                                              chunk=chunk)
    ok = torch.from_numpy(oracle.allowed(np.arange(n), n, causal, bm, mb))
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq[None], tk[None], tv[None], attn_mask=ok[None], scale=0.3)[0]
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy()[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy()[cols], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy()[cols], rtol=0, atol=1e-12)


def test_sampled_gradients_finite_differences():
    n, d = 12, 8
    q, k, v, do = randn(n, d), randn(n, d), randn(n, d), randn(n, d)
    rows, cols = np.array([0, 7, 11]), np.array([2, 11])
    dq, dk, dv = oracle.backward_head_sampled(q, k, v, do, 0.35, True, None, rows, cols, 4,
                                              chunk=5)
    fq, fk, fv = finite_difference_grads(q, k, v, do, 0.35, True, None, 4)
    for got, ref in ((dq, fq[rows]), (dk, fk[cols]), (dv, fv[cols])):
        assert np.max(np.abs(got - ref)) <= 1e-6 * max(1e-12, np.max(np.abs(ref)))


@pytest.mark.parametrize("causal,masked", [(False, False), (True, True)])
def test_backward_terms(causal, masked):
    """backward_head_terms: P's rows sum to 1 (0 on a row with no allowed
    key), dS's rows sum to 0 (sum_j P_ij (dP_ij - D_i) = D_i - D_i), and
    scale dS K, scale dS^T Q, P^T dO, P V give backward_head's gradients and
    forward_head's output."""
    n, d, scale = 300, 16, 0.4
    q, k, v, do = (randn(n, d) for _ in range(4))
    bm = None
    if masked:
        bm = np.ones((3, 3), dtype=np.uint8)
        bm[1, :] = 0
    t = oracle.backward_head_terms(q, k, v, do, scale, causal, bm, mask_block=128)
    live = np.ones(n, dtype=bool) if bm is None else (np.arange(n) // 128) != 1
    np.testing.assert_allclose(t["p"].sum(axis=1), live.astype(float), atol=1e-12)
    np.testing.assert_allclose(t["ds"].sum(axis=1), 0.0, atol=1e-12)
    assert np.all(np.isneginf(t["lse"][~live]))
    o, lse = forward_head(q, k, v, scale, causal, bm)
    np.testing.assert_allclose(t["o"], o, atol=1e-12)
    np.testing.assert_allclose(t["lse"], lse, atol=1e-12)
    dq, dk, dv = backward_head(q, k, v, do, scale, causal, bm)
    np.testing.assert_allclose(scale * t["ds"] @ k, dq, atol=1e-12)
    np.testing.assert_allclose(scale * t["ds"].T @ q, dk, atol=1e-12)
    np.testing.assert_allclose(t["p"].T @ do, dv, atol=1e-12)
