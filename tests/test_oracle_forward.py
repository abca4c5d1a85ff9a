"""Pins for the oracle's forward pass (oracle/attention.py).

Each test checks the oracle against something other than its own formula:
closed forms, invariants of softmax attention, a pure-Python brute force,
and torch's independent attention routine.  A dropped term, a wrong sign or
index, or a transposed operand in the oracle fails at least one of them.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import forward_head

RNG = np.random.default_rng(1234)


def randn(*shape, rng=RNG):
    return rng.standard_normal(shape)


def brute_force_row(q, k, v, scale, i, ok):
    """Row i of attention with Python floats: math.exp and math.fsum only."""
    scores = [scale * math.fsum(q[i][c] * k[j][c] for c in range(len(q[i])))
              for j in range(len(k)) if ok(i, j)]
    keys = [j for j in range(len(k)) if ok(i, j)]
    if not keys:
        return [0.0] * len(v[0]), -math.inf
    weights = [math.exp(s) for s in scores]          # tiny N, no overflow
    z = math.fsum(weights)
    out = [math.fsum(w * v[j][c] for w, j in zip(weights, keys)) / z
           for c in range(len(v[0]))]
    return out, math.log(z)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(1, 4), (5, 3), (8, 8)])
def test_brute_force_tiny(n, d, causal):
    q, k, v = randn(n, d), randn(n, d), randn(n, d)
    scale = 0.37
    o, lse = forward_head(q, k, v, scale, causal=causal, chunk=3)
    for i in range(n):
        ref_o, ref_lse = brute_force_row(q.tolist(), k.tolist(), v.tolist(), scale, i,
                                         lambda a, b: (not causal) or b <= a)
        assert np.max(np.abs(o[i] - ref_o)) <= 1e-13
        assert abs(lse[i] - ref_lse) <= 1e-13


def test_brute_force_tiny_block_mask():
    n, d, mb = 8, 4, 2
    mask = np.array([[1, 0, 1, 0], [0, 1, 0, 0], [1, 1, 1, 0], [0, 0, 1, 1]], np.uint8)
    q, k, v = randn(n, d), randn(n, d), randn(n, d)
    for causal in (False, True):
        o, lse = forward_head(q, k, v, 0.5, causal=causal, block_mask=mask, mask_block=mb)
        for i in range(n):
            ok = lambda a, b: mask[a // mb][b // mb] == 1 and ((not causal) or b <= a)  # noqa: E731
            ref_o, ref_lse = brute_force_row(q.tolist(), k.tolist(), v.tolist(), 0.5, i, ok)
            assert np.max(np.abs(o[i] - ref_o)) <= 1e-13
            assert lse[i] == ref_lse or abs(lse[i] - ref_lse) <= 1e-13


def test_rows_sum_to_one_via_ones_column():
    n, d = 300, 16
    q, k = randn(n, d) * 3, randn(n, d) * 3
    v = np.ones((n, 1))
    for causal in (False, True):
        o, _ = forward_head(q, k, v, 0.25, causal=causal, chunk=64)
        assert np.max(np.abs(o - 1.0)) <= 1e-15 * 4


def test_single_token():
    q, k, v = randn(1, 64), randn(1, 64), randn(1, 64)
    o, lse = forward_head(q, k, v, 0.125)
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    assert abs(lse[0] - 0.125 * float(q[0] @ k[0])) <= 1e-14


def test_identical_keys_give_mean_of_allowed_values():
    n, d = 200, 32
    q, v = randn(n, d), randn(n, d)
    k = np.tile(randn(1, d), (n, 1))
    mask = (np.random.default_rng(5).random((4, 4)) < 0.6).astype(np.uint8)
    np.fill_diagonal(mask, 1)
    for causal in (False, True):
        for bm in (None, mask):
            o, lse = forward_head(q, k, v, 0.2, causal=causal, block_mask=bm, mask_block=64)
            ok = oracle.allowed(np.arange(n), n, causal, bm, 64)
            cnt = ok.sum(axis=1)
            mean_v = (ok.astype(float) @ v) / cnt[:, None]
            np.testing.assert_allclose(o, mean_v, rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse, 0.2 * (q @ k[0]) + np.log(cnt), rtol=0, atol=1e-12)


def test_constant_value_rows():
    n, d = 130, 8
    q, k = randn(n, d), randn(n, d)
    c = randn(1, d)
    v = np.tile(c, (n, 1))
    for causal in (False, True):
        o, _ = forward_head(q, k, v, 0.3, causal=causal)
        np.testing.assert_allclose(o, v, rtol=0, atol=1e-14)


def test_causal_row_zero_attends_only_itself():
    n, d = 500, 64
    q, k, v = randn(n, d), randn(n, d), randn(n, d)
    o, lse = forward_head(q, k, v, 0.125, causal=True, rows=np.array([0]))
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=1e-15)
    assert abs(lse[0] - 0.125 * float(q[0] @ k[0])) <= 1e-13


def test_causal_row_equals_attention_over_prefix():
    n, d = 77, 16
    q, k, v = randn(n, d), randn(n, d), randn(n, d)
    o, lse = forward_head(q, k, v, 0.25, causal=True, chunk=10)
    for i in (0, 1, 9, 10, 40, 76):
        oi, li = forward_head(q[i:i + 1], k[:i + 1], v[:i + 1], 0.25, causal=False)
        np.testing.assert_allclose(o[i], oi[0], rtol=0, atol=1e-14)
        assert abs(lse[i] - li[0]) <= 1e-13


def test_key_value_permutation_invariance():
    n, d = 96, 16
    q, k, v = randn(n, d), randn(n, d), randn(n, d)
    perm = np.random.default_rng(9).permutation(n)
    o1, l1 = forward_head(q, k, v, 0.25)
    o2, l2 = forward_head(q, k[perm], v[perm], 0.25)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)
    # pairing keys with the wrong values must change the result
    o3, _ = forward_head(q, k, v[perm], 0.25)
    assert np.max(np.abs(o3 - o1)) > 1e-3


def test_common_key_shift_moves_only_lse():
    """k_j -> k_j + w adds scale<q_i,w> to every score of row i."""
    n, d = 120, 16
    q, k, v = randn(n, d), randn(n, d), randn(n, d)
    w = randn(d)
    for causal in (False, True):
        o1, l1 = forward_head(q, k, v, 0.3, causal=causal)
        o2, l2 = forward_head(q, k + w, v, 0.3, causal=causal)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2 - l1, 0.3 * (q @ w), rtol=0, atol=1e-12)


def test_affine_values():
    n, d = 64, 8
    q, k, v = randn(n, d), randn(n, d), randn(n, d)
    o1, _ = forward_head(q, k, v, 0.3, causal=True)
    o2, _ = forward_head(q, k, 2.5 * v - 1.75, 0.3, causal=True)
    np.testing.assert_allclose(o2, 2.5 * o1 - 1.75, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_matches_torch_attention_fp64(causal, masked):
    """Independent route: torch's scaled_dot_product_attention in float64."""
    n, d, mb = 192, 32, 64
    q, k, v = randn(n, d), randn(n, d), randn(n, d)
    bm = None
    if masked:
        bm = (np.random.default_rng(3).random((3, 3)) < 0.5).astype(np.uint8)
        np.fill_diagonal(bm, 1)
    o, lse = forward_head(q, k, v, 0.2, causal=causal, block_mask=bm, mask_block=mb, chunk=50)
    ok = torch.from_numpy(oracle.allowed(np.arange(n), n, causal, bm, mb))
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq[None], tk[None], tv[None], attn_mask=ok[None], scale=0.2)[0]
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-13)
    s = (tq @ tk.T) * 0.2
    ref_lse = torch.logsumexp(s.masked_fill(~ok, -float("inf")), dim=-1)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=0, atol=1e-12)


def test_sparse_semantics():
    n, d, mb = 256, 16, 64
    q, k, v = randn(n, d), randn(n, d), randn(n, d)
    t = n // mb
    ones = np.ones((t, t), np.uint8)
    for causal in (False, True):
        a = forward_head(q, k, v, 0.25, causal=causal)
        b = forward_head(q, k, v, 0.25, causal=causal, block_mask=ones, mask_block=mb)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
    # diagonal-only mask == attention inside each 64-row block separately
    o, lse = forward_head(q, k, v, 0.25, block_mask=np.eye(t, dtype=np.uint8), mask_block=mb)
    for blk in range(t):
        s_ = slice(blk * mb, (blk + 1) * mb)
        ob, lb = forward_head(q[s_], k[s_], v[s_], 0.25)
        np.testing.assert_allclose(o[s_], ob, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[s_], lb, rtol=0, atol=1e-13)


def test_fully_masked_row_gives_zero_and_neg_inf():
    n, d, mb = 8, 4, 4
    mask = np.array([[0, 0], [1, 1]], np.uint8)      # rows 0..3 see nothing
    q, k, v = randn(n, d), randn(n, d), randn(n, d)
    o, lse = forward_head(q, k, v, 0.5, block_mask=mask, mask_block=mb)
    assert np.all(o[:4] == 0) and np.all(np.isneginf(lse[:4]))
    assert np.all(np.isfinite(lse[4:]))


def test_chunking_and_row_sampling_do_not_change_results():
    n, d = 300, 16
    q, k, v = randn(n, d), randn(n, d), randn(n, d)
    o1, l1 = forward_head(q, k, v, 0.25, causal=True, chunk=512)
    o2, l2 = forward_head(q, k, v, 0.25, causal=True, chunk=7)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    rows = np.array([299, 3, 150])
    o3, l3 = forward_head(q, k, v, 0.25, causal=True, rows=rows)
    np.testing.assert_allclose(o3, o1[rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(l3, l1[rows], rtol=0, atol=1e-14)


def test_batched_wrapper_matches_heads():
    q, k, v = randn(2, 3, 40, 8), randn(2, 3, 40, 8), randn(2, 3, 40, 8)
    o, lse = oracle.forward(q, k, v, 0.3, causal=True)
    for b in range(2):
        for h in range(3):
            oh, lh = forward_head(q[b, h], k[b, h], v[b, h], 0.3, causal=True)
            np.testing.assert_array_equal(o[b, h], oh)
            np.testing.assert_array_equal(lse[b, h], lh)
