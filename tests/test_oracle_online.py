"""Pins for the online-softmax recurrence (oracle/online.py).

The recurrence must reach the plain two-pass softmax exactly up to rounding:
checked against the direct (max, sum of exponentials) of whole rows, against
the two-pass forward of oracle/attention.py, and against the worked example
that the ultralytics glossary page prints (tests/golden/).
"""

import json
import os

import numpy as np
import pytest
import torch

from exact_io_aware_34_amd.workloads import draw_page_qkv
from oracle import forward_head, merge_stats, online_softmax_deferred
from oracle import online_softmax_normalised_each_step

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(77)


def direct_stats(x):
    m = np.max(x)
    return m, np.sum(np.exp(x - m))


def test_merge_identity_over_random_splits():
    for trial in range(200):
        n = int(RNG.integers(1, 300))
        x = RNG.standard_normal(n) * RNG.uniform(0.1, 20)
        cuts = np.sort(RNG.choice(np.arange(1, n), size=min(n - 1, int(RNG.integers(0, 8))),
                                  replace=False)) if n > 1 else []
        parts = np.split(x, cuts)
        m, ell = -np.inf, 0.0
        for p in parts:
            m, ell = merge_stats(m, ell, *direct_stats(p))
        m_ref, l_ref = direct_stats(x)
        assert m == m_ref
        assert abs(ell - l_ref) <= 1e-14 * l_ref


def test_merge_with_empty_part_is_identity():
    m, ell = merge_stats(-np.inf, 0.0, 1.5, 2.0)
    assert (m, ell) == (1.5, 2.0)
    m, ell = merge_stats(-np.inf, 0.0, -np.inf, 0.0)
    assert np.isneginf(m) and ell == 0.0


def test_merge_is_symmetric_and_rescales_smaller_part():
    m, ell = merge_stats(3.0, 2.0, 1.0, 5.0)
    assert m == 3.0
    assert abs(ell - (2.0 + np.exp(-2.0) * 5.0)) <= 1e-15
    assert merge_stats(1.0, 5.0, 3.0, 2.0) == (m, ell)


@pytest.mark.parametrize("form", [online_softmax_normalised_each_step, online_softmax_deferred])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 7, 64, 200])
def test_online_forms_equal_two_pass(form, causal, block):
    n, d = 200, 16
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    s = 0.25 * (q @ k.T)
    if causal:
        s = np.where(np.tril(np.ones((n, n), bool)), s, -np.inf)
    o, m, ell = form(s, v, block)
    o_ref, lse_ref = forward_head(q, k, v, 0.25, causal=causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(m + np.log(ell), lse_ref, rtol=0, atol=1e-13)
    assert np.all(m == np.max(s, axis=1))


@pytest.mark.parametrize("form", [online_softmax_normalised_each_step, online_softmax_deferred])
def test_online_forms_row_with_no_key(form):
    s = np.array([[-np.inf] * 5, [0.1, -np.inf, 0.3, -np.inf, 2.0]])
    v = RNG.standard_normal((5, 3))
    o, m, ell = form(s, v, 2)
    assert np.all(o[0] == 0) and np.isneginf(m[0]) and ell[0] == 0
    w = np.exp(s[1] - 2.0)
    np.testing.assert_allclose(o[1], (w @ v) / w.sum(), rtol=0, atol=1e-14)


def test_online_forms_large_score_range():
    """Scores spanning thousands of units: rescaling must keep everything finite."""
    s = np.array([np.linspace(-4000, 4000, 97), np.linspace(4000, -4000, 97)])
    v = RNG.standard_normal((97, 4))
    for form in (online_softmax_normalised_each_step, online_softmax_deferred):
        o, _, _ = form(s, v, 10)
        np.testing.assert_allclose(o[0], v[-1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(o[1], v[0], rtol=0, atol=1e-12)


def test_glossary_worked_example_fp32():
    """The page's fp32 loop differs from fp32 standard attention by ~4.3e-7."""
    g = json.load(open(os.path.join(GOLDEN, "glossary_loop_n4096.json")))
    n, d, block = g["n"], g["d"], g["block"]
    q, k, v = draw_page_qkv(n, d, g["seed"])
    assert block * n / (n * n) == g["tile_fraction_of_matrix"]
    assert [n, block] == g["largest_score_tile"]
    # standard attention in fp32, the page's reference line (library route)
    reference = (torch.softmax(q @ k.T / d ** 0.5, dim=-1) @ v).numpy()
    s32 = (q @ k.T / d ** 0.5).numpy()                        # fp32 scores
    out, _, _ = online_softmax_deferred(s32, v.numpy(), block, dtype=np.float32)
    assert out.dtype == np.float32
    diff = float(np.max(np.abs(out - reference)))
    printed = g["printed_max_abs_diff_fp32"]
    assert printed / 10 <= diff <= printed * 10, diff         # same order: fp32 rounding
    # and the fp64 definition sits within fp32 rounding of both
    o64, _ = forward_head(q.numpy(), k.numpy(), v.numpy(), 1.0 / d ** 0.5)
    assert np.max(np.abs(o64 - reference)) <= printed * 10
    assert np.max(np.abs(o64 - out)) <= printed * 10
    out_n, _, _ = online_softmax_normalised_each_step(s32, v.numpy(), block, dtype=np.float32)
    assert np.max(np.abs(out_n - reference)) <= printed * 10
