"""Pins for the decode oracle (oracle/decode.py).

Decode is the forward definition with Nq <= Nk queries placed at the end of
the sequence.  It is pinned against: the square causal forward (Nq = Nk), the
rectangular non-causal forward, pure-Python brute force with math.fsum,
closed forms (one key, identical keys, one visible key), explicit visibility
tables, and -- for the split/combine pair -- the direct result over the whole
key range, the (m, l) merge of oracle/online.py, order invariance and
single-part identity.  The last test plants plausible slips in copies of the
functions and checks that the pins catch them.
"""

import math

import numpy as np
import pytest

from oracle import (combine, decode, decode_allowed, decode_head, forward_head, merge_stats,
                    split_partials)

RNG = np.random.default_rng(2024)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def brute(q, k, v, scale, causal):
    nq, nk = q.shape[0], k.shape[0]
    o = np.zeros((nq, v.shape[1]))
    lse = np.zeros(nq)
    for i in range(nq):
        keys = [j for j in range(nk) if (not causal) or j <= nk - nq + i]
        s = [scale * math.fsum(q[i, c] * k[j, c] for c in range(q.shape[1])) for j in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = math.fsum(e)
        lse[i] = m + math.log(tot)
        for c in range(v.shape[1]):
            o[i, c] = math.fsum(e[t] * v[keys[t], c] for t in range(len(keys))) / tot
    return o, lse


@pytest.mark.parametrize("nq,nk,causal", [(1, 1, False), (1, 7, True), (3, 5, True),
                                         (4, 9, False), (2, 2, True), (5, 11, True)])
def test_brute_force(nq, nk, causal):
    q, k, v = rand(nq, 6), rand(nk, 6), rand(nk, 5)
    o, lse = decode_head(q, k, v, 0.37, causal)
    ro, rl = brute(q, k, v, 0.37, causal)
    np.testing.assert_allclose(o, ro, atol=1e-13)
    np.testing.assert_allclose(lse, rl, atol=1e-13)


def test_square_causal_is_the_forward_rule():
    n, d = 40, 16
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    o, lse = decode_head(q, k, v, 0.25, causal=True)
    ro, rl = forward_head(q, k, v, 0.25, causal=True)
    np.testing.assert_allclose(o, ro, atol=1e-13)
    np.testing.assert_allclose(lse, rl, atol=1e-13)


def test_rectangular_noncausal_is_the_forward_definition():
    q, k, v = rand(3, 8), rand(50, 8), rand(50, 8)
    o, lse = decode_head(q, k, v, 0.5)
    ro, rl = forward_head(q, k, v, 0.5, causal=False)
    np.testing.assert_allclose(o, ro, atol=1e-13)
    np.testing.assert_allclose(lse, rl, atol=1e-13)


def test_visibility_table():
    ok = decode_allowed(2, 5, causal=True)
    assert ok.tolist() == [[True, True, True, True, False], [True, True, True, True, True]]
    assert decode_allowed(2, 5, causal=False).all()


def test_closed_forms():
    d = 4
    q = rand(1, d)
    kk = rand(1, d)
    k = np.repeat(kk, 9, axis=0)
    v = rand(9, d)
    o, lse = decode_head(q, k, v, 0.7)
    np.testing.assert_allclose(o[0], v.mean(axis=0), atol=1e-14)
    np.testing.assert_allclose(lse[0], 0.7 * float(q[0] @ kk[0]) + math.log(9), atol=1e-13)
    # causal, first of three queries over three keys: sees only key 0
    q3, k3, v3 = rand(3, d), rand(3, d), rand(3, d)
    o3, l3 = decode_head(q3, k3, v3, 0.3, causal=True)
    np.testing.assert_allclose(o3[0], v3[0], atol=1e-15)
    np.testing.assert_allclose(l3[0], 0.3 * float(q3[0] @ k3[0]), atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_split_then_combine_is_direct(causal):
    for trial in range(30):
        nq = int(RNG.integers(1, 6))
        nk = int(RNG.integers(nq, 200))
        q, k, v = rand(nq, 8, scale=2.0), rand(nk, 8, scale=2.0), rand(nk, 8)
        cuts = sorted(set(RNG.integers(0, nk + 1, size=int(RNG.integers(0, 6))).tolist()))
        bounds = [0] + [c for c in cuts if 0 < c < nk] + [nk]
        o_p, l_p = split_partials(q, k, v, 0.6, causal, bounds)
        o, lse = combine(o_p, l_p)
        ro, rl = decode_head(q, k, v, 0.6, causal)
        np.testing.assert_allclose(o, ro, atol=1e-12)
        np.testing.assert_allclose(lse, rl, atol=1e-12)


def test_split_with_invisible_parts():
    # causal, Nq = 1 at position Nk-1 sees everything; Nq = 4 at the end: the
    # last part is invisible to the first query.
    q, k, v = rand(4, 8), rand(12, 8), rand(12, 8)
    o_p, l_p = split_partials(q, k, v, 0.4, True, [0, 5, 10, 11, 12])
    assert l_p[3][0] == -np.inf and l_p[2][0] == -np.inf and np.all(o_p[3][0] == 0)
    o, lse = combine(o_p, l_p)
    ro, rl = decode_head(q, k, v, 0.4, True)
    np.testing.assert_allclose(o, ro, atol=1e-13)
    np.testing.assert_allclose(lse, rl, atol=1e-13)


def test_combine_matches_the_m_l_merge_and_is_order_free():
    q, k, v = rand(3, 8, scale=3.0), rand(90, 8, scale=3.0), rand(90, 8)
    bounds = [0, 7, 31, 32, 90]
    o_p, l_p = split_partials(q, k, v, 0.9, False, bounds)
    # (m, l) merge from oracle/online.py applied to the per-part statistics:
    # with o_s normalised, l_s = exp(lse_s - m_s) for any m_s; take m_s = lse_s.
    for i in range(3):
        m, ell = -np.inf, 0.0
        for s in range(len(l_p)):
            m, ell = merge_stats(m, ell, l_p[s][i], 1.0)
        _, lse = combine(o_p, l_p)
        np.testing.assert_allclose(m + math.log(ell), lse[i], atol=1e-13)
    perm = [2, 0, 3, 1]
    o1, l1 = combine(o_p, l_p)
    o2, l2 = combine([o_p[j] for j in perm], [l_p[j] for j in perm])
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    o3, l3 = combine([o_p[0]], [l_p[0]])
    np.testing.assert_allclose(o3, o_p[0], atol=0)
    np.testing.assert_allclose(l3, l_p[0], atol=0)


def test_combine_all_empty():
    o, lse = combine([np.ones((2, 3)), np.ones((2, 3))], [np.full(2, -np.inf), np.full(2, -np.inf)])
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_large_scores_do_not_overflow():
    q = np.full((2, 4), 30.0)
    k = rand(64, 4, scale=30.0)
    v = rand(64, 4)
    o_p, l_p = split_partials(q, k, v, 1.0, False, [0, 16, 64])
    o, lse = combine(o_p, l_p)
    ro, rl = decode_head(q, k, v, 1.0, False)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-15, atol=1e-9)


def test_batched_wrapper():
    q, k, v = rand(2, 3, 2, 8), rand(2, 3, 20, 8), rand(2, 3, 20, 8)
    o, lse = decode(q, k, v, 0.3, causal=True)
    for b in range(2):
        for h in range(3):
            ro, rl = decode_head(q[b, h], k[b, h], v[b, h], 0.3, True)
            np.testing.assert_allclose(o[b, h], ro, atol=0)
            np.testing.assert_allclose(lse[b, h], rl, atol=0)


# ---- planted mistakes: each must fail at least one pin above ----

def _top_left_causal(q, k, v, scale, causal=False, keys=None):
    nq, nk = q.shape[0], k.shape[0]
    sel = np.arange(nk) if keys is None else np.asarray(keys)
    s = scale * (q @ k[sel].T)
    ok = np.ones((nq, sel.size), bool)
    if causal:
        ok &= sel[None, :] <= np.arange(nq)[:, None]          # aligned to the start: wrong
    from oracle.attention import _row_softmax
    p, lse = _row_softmax(s, ok)
    return p @ v[sel], lse


def _combine_unweighted(o_parts, lse_parts):
    lse = np.log(np.sum(np.exp(np.stack(lse_parts)), axis=0))
    return np.mean(np.stack(o_parts), axis=0), lse               # weights dropped: wrong


def _combine_no_shift(o_parts, lse_parts):
    l_s = np.stack(lse_parts)
    w = np.exp(l_s)                                              # no max shift: overflows
    return (w[:, :, None] * np.stack(o_parts)).sum(0) / w.sum(0)[:, None], np.log(w.sum(0))


def test_pins_catch_planted_mistakes():
    q, k, v = rand(3, 8), rand(9, 8), rand(9, 8)
    wrong_o, _ = _top_left_causal(q, k, v, 0.4, causal=True)
    ro, _ = brute(q, k, v, 0.4, True)
    assert not np.allclose(wrong_o, ro, atol=1e-6)

    qq, kk, vv = rand(3, 8, scale=2.0), rand(60, 8, scale=2.0), rand(60, 8)
    o_p, l_p = split_partials(qq, kk, vv, 0.6, False, [0, 10, 60])
    ro, rl = decode_head(qq, kk, vv, 0.6, False)
    wo, _ = _combine_unweighted(o_p, l_p)
    assert not np.allclose(wo, ro, atol=1e-6)

    q2 = np.full((2, 4), 30.0)
    k2 = rand(64, 4, scale=30.0)
    v2 = rand(64, 4)
    o_p, l_p = split_partials(q2, k2, v2, 1.0, False, [0, 16, 64])
    with np.errstate(over="ignore", invalid="ignore"):
        wo, wl = _combine_no_shift(o_p, l_p)
    assert not (np.isfinite(wo).all() and np.isfinite(wl).all())
