"""Pins for the FP8 emulation (oracle/fp8.py).

* e4m3 against torch's float8_e4m3fn conversion (an independent library
  route) on every representable value, every midpoint (ties), values just
  either side of them and a log-uniform sweep; closed-form ties; saturation;
  the count of distinct outputs.
* hadamard against scipy.linalg.hadamard; H H^T = d I.
* rotate: the d = 2 closed form, norms and dot products preserved.
* pow2_scale: closed forms at and around 448 * 2^k, and brute force over k
  (the smallest power of two whose 448 multiple reaches amax).
* block_quantize: every scale is that power of two, each block's largest
  magnitude maps into (224, 448], the relative error of every normal-range
  entry is at most 2^-4, zero blocks.
* fp8_forward_head: with the identity in place of e4m3 it is exact attention
  (with or without the rotation, causal, masked) -- the rotation cancels and
  every scale, the base-2 factor included, folds back; with e4m3 its error
  against exact attention is that
  of 3-bit mantissas; with outliers in Q and K the rotation lowers the error
  on every seed, by about 2.3x on lse on average (the marketmaker.cc page
  reports 2.6x for the method on its own inputs).
* Planted slips in copies of the functions fail these pins.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as F

RNG = np.random.default_rng(88)


def torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).float().double().numpy()


def all_finite_e4m3():
    v = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().double().numpy()
    return np.unique(v[np.isfinite(v)])


def test_e4m3_matches_library_conversion():
    fin = all_finite_e4m3()
    pos = fin[fin > 0]
    mids = (pos[1:] + pos[:-1]) / 2
    x = np.concatenate([fin, mids, -mids, pos[:-1] * (1 + 2 ** -20), pos[1:] * (1 - 2 ** -20),
                        np.sign(RNG.standard_normal(20000)) * 2.0 ** RNG.uniform(-14, 8.8, 20000)])
    x = x[np.abs(x) <= 448].astype(np.float32).astype(np.float64)   # exactly representable inputs
    np.testing.assert_array_equal(F.e4m3(x), torch_e4m3(x))


def test_e4m3_closed_forms():
    assert F.e4m3(1 + 2 ** -4) == 1.0              # tie between 1 and 1.125 -> even mantissa
    assert F.e4m3(1 + 3 * 2 ** -4) == 1.25         # tie between 1.125 and 1.25 -> 1.25
    assert F.e4m3(2 ** -10) == 0.0                 # tie between 0 and 2^-9 -> 0
    assert F.e4m3(3 * 2 ** -10) == 2 ** -8         # tie between 2^-9 and 2^-8 -> 2^-8
    assert F.e4m3(448) == 448 and F.e4m3(1e6) == 448 and F.e4m3(-500) == -448
    assert F.e4m3(2 ** -6) == 2 ** -6 and F.e4m3(240.0) == 240.0
    x = np.concatenate([np.linspace(0, 448, 200001), np.geomspace(2.0 ** -12, 448, 200001)])
    assert np.unique(F.e4m3(x)).size == 127        # 0x00 .. 0x7E


def test_hadamard():
    from scipy.linalg import hadamard as sp_h
    for d in (1, 2, 4, 8, 64, 128):
        h = F.hadamard(d)
        np.testing.assert_array_equal(h, sp_h(d))
        np.testing.assert_array_equal(h @ h.T, d * np.eye(d))


def test_rotate():
    a, b = 0.7, -1.9
    np.testing.assert_allclose(F.rotate(np.array([[a, b]]), [1, -1]),
                               [[(a - b) / math.sqrt(2), (a + b) / math.sqrt(2)]], atol=1e-15)
    x, y = RNG.standard_normal((5, 64)), RNG.standard_normal((7, 64))
    s = RNG.choice([-1.0, 1.0], 64)
    rx, ry = F.rotate(x, s), F.rotate(y, s)
    np.testing.assert_allclose(np.linalg.norm(rx, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(rx @ ry.T, x @ y.T, atol=1e-12)
    assert not np.allclose(rx, x)


def test_pow2_scale():
    assert F.pow2_scale(0.0) == 1.0
    assert F.pow2_scale(448.0) == 1.0 and F.pow2_scale(448.0 * (1 + 2 ** -40)) == 2.0
    assert F.pow2_scale(224.0) == 0.5 and F.pow2_scale(224.0 * (1 + 2 ** -40)) == 1.0
    assert F.pow2_scale(1.0) == 2.0 ** -8 and F.pow2_scale(1.75) == 2.0 ** -8
    assert F.pow2_scale(1.76) == 2.0 ** -7
    assert F.pow2_scale(1e-300) == 2.0 ** -126                 # clamped
    for a in np.concatenate([2.0 ** RNG.uniform(-100, 100, 2000), 448.0 * 2.0 ** np.arange(-20, 21)]):
        k = next(k for k in range(-200, 200) if 448.0 * 2.0 ** k >= a)    # brute force
        assert F.pow2_scale(a) == 2.0 ** max(k, -126), a


def test_block_quantize():
    x = RNG.standard_normal((150, 64)) * np.repeat([1.0, 30.0, 0.01], 50)[:, None]
    x[100:150] = 0.0
    x8, sc = F.block_quantize(x, 64)
    assert sc.shape == (3,) and sc[2] == 1.0 and np.all(x8[128:] == 0)
    for b in range(2):
        blk = x8[64 * b: 64 * (b + 1)]
        amax = np.abs(x[64 * b: 64 * (b + 1)]).max()
        assert sc[b] == F.pow2_scale(amax) and sc[b] >= amax / 448 > sc[b] / 2
        assert 224.0 < np.max(np.abs(blk)) <= 448.0
    deq = x8 * np.repeat(sc, 64)[:150, None]
    normal = np.abs(x8) >= 2 ** -6
    rel = np.abs(deq - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 2 ** -4 + 1e-12
    assert set(np.unique(F.e4m3(x8))) == set(np.unique(x8))     # already on the grid


def _ident(x):
    return np.asarray(x, dtype=np.float64)


@pytest.mark.parametrize("causal,masked,rotated", [(False, False, True), (True, False, True),
                                                   (True, True, True), (False, True, False)])
def test_exact_without_rounding(causal, masked, rotated):
    n, d = 200, 64
    q, k, v = (RNG.standard_normal((n, d)) * 2 for _ in range(3))
    mask = None
    if masked:
        mask = (RNG.random((2, 2)) < 0.7).astype(np.uint8)
        mask[0, 0] = 1
    s = RNG.choice([-1.0, 1.0], d) if rotated else None
    o, lse = F.fp8_forward_head(q, k, v, 0.125, causal, mask, s, quantize=_ident)
    ro, rl = oracle.forward_head(q, k, v, 0.125, causal, mask)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


def _rms(a):
    a = np.asarray(a)
    return float(np.sqrt(np.mean(a[np.isfinite(a)] ** 2)))


def test_error_is_that_of_three_bit_mantissas():
    """N(0,1) inputs: the FP8 result is off by a few percent (not by 1e-3 as a
    16-bit path, and not by O(1) as a broken one)."""
    n, d = 512, 64
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    s = RNG.choice([-1.0, 1.0], d)
    o, lse = F.fp8_forward_head(q, k, v, 0.125, True, None, s)
    ro, rl = oracle.forward_head(q, k, v, 0.125, True)
    rel = _rms(o - ro) / _rms(ro)
    assert 0.01 < rel < 0.1, rel
    assert _rms(lse - rl) < 0.05


def outlier_qkv(n, d, rng, frac=1e-3, sd=10.0):
    """N(0,1) Q, K, V; a fraction `frac` of the Q and K entries redrawn from N(0, sd^2)."""
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    for x in (q, k):
        m = rng.random(x.shape) < frac
        x[m] = rng.standard_normal(m.sum()) * sd
    return q, k, v


def test_rotation_reduces_error_with_outliers():
    # Ten seeds of this recipe gave lse-error ratios 1.87..6.42 (mean 3.14)
    # and O-error ratios 1.30..1.72 (mean 1.44); the first six (lse mean
    # 2.33, O mean 1.41) are checked here.
    ratios_lse, ratios_o = [], []
    for seed in range(6):
        rng = np.random.default_rng(100 + seed)
        q, k, v = outlier_qkv(1024, 64, rng)
        s = rng.choice([-1.0, 1.0], 64)
        ro, rl = oracle.forward_head(q, k, v, 0.125, True)
        on, ln = F.fp8_forward_head(q, k, v, 0.125, True, None, None)
        orr, lr = F.fp8_forward_head(q, k, v, 0.125, True, None, s)
        ratios_lse.append(_rms(ln - rl) / _rms(lr - rl))
        ratios_o.append(_rms(on - ro) / _rms(orr - ro))
    assert min(ratios_lse) > 1.5 and np.mean(ratios_lse) > 2.0, ratios_lse
    assert min(ratios_o) > 1.15 and np.mean(ratios_o) > 1.25, ratios_o


def test_terms_recompose_the_output():
    """The step-4 quantities returned with terms=True give back o and lse:
    o = (e4m3(p) sv) @ v8 / l, lse = (max_j x_ij + log2 l) ln 2 (2^(x - m)
    sums to l, and p is 1 at each row's max)."""
    n, d = 150, 64
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    v[64:128] *= 20.0                                            # a value block of its own scale
    s = RNG.choice([-1.0, 1.0], d)
    o, l, t = F.fp8_forward_head(q, k, v, 0.125, True, None, s, terms=True)
    o2 = (F.e4m3(t["p"]) * t["sv"][None, :]) @ t["v8"] / t["l"][:, None]
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    assert np.allclose(t["p"].max(axis=1), 1.0) and np.allclose(t["p"].sum(axis=1), t["l"])
    assert np.all(np.triu(t["p"], 1) == 0)                      # causal: nothing above
    _, sv = F.block_quantize(v, 64)
    np.testing.assert_array_equal(t["sv"], np.repeat(sv, 64)[:n])
    assert sv[1] >= 8 * max(sv[0], sv[2])
    # s_abs bounds |x| and equals it where every product has one sign
    o3, l3, t3 = F.fp8_forward_head(np.abs(q), np.abs(k), v, 0.125, False, None, None,
                                    terms=True)
    np.testing.assert_allclose((t3["s_abs"].max(axis=1) + np.log2(t3["l"])) * math.log(2), l3,
                               atol=1e-12)


def test_rows_selects_query_rows():
    n, d = 150, 64
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    s = RNG.choice([-1.0, 1.0], d)
    o, l = F.fp8_forward_head(q, k, v, 0.125, True, None, s)
    rows = [0, 63, 64, 149]
    o2, l2 = F.fp8_forward_head(q, k, v, 0.125, True, None, s, rows=rows)
    np.testing.assert_allclose(o2, o[rows], atol=1e-14)
    np.testing.assert_allclose(l2, l[rows], atol=1e-14)


# ---- planted slips ----

def _e4m3_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    step = np.where(ax >= 2.0 ** -6, 2.0 ** (np.maximum(e, -6) - 3), 2.0 ** -9)
    return np.copysign(np.minimum(np.floor(ax / step + 0.5) * step, 448.0), x)


def _forward_q_only_rotated(q, k, v, scale, causal, signs):
    return F.fp8_forward_head(F.rotate(q, signs), k, v, scale, causal, None, None, quantize=_ident)


def _forward_one_v_scale(q, k, v, scale, causal):
    """Slip: every value block multiplied by the largest value-block scale."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    n = q.shape[0]
    c = scale * math.log2(math.e)
    q8, sq = F.block_quantize(q * c, 64, _ident)
    k8, sk = F.block_quantize(k, 64, _ident)
    v8, sv = F.block_quantize(v, 64, _ident)
    x = (q8 * np.repeat(sq, 64)[:n, None]) @ (k8 * np.repeat(sk, 64)[:n, None]).T
    x = np.where(oracle.allowed(np.arange(n), n, causal), x, -np.inf)
    p = np.exp2(x - x.max(axis=1, keepdims=True))
    return sv.max() * (p @ v8) / p.sum(axis=1, keepdims=True)


def _forward_natural_exp(q, k, v, scale, causal):
    """Slip: base-2 scores fed to a natural exponential."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    n = q.shape[0]
    x = (q * scale * math.log2(math.e)) @ k.T
    x = np.where(oracle.allowed(np.arange(n), n, causal), x, -np.inf)
    p = np.exp(x - x.max(axis=1, keepdims=True))
    return (p @ v) / p.sum(axis=1, keepdims=True)


def test_pins_catch_planted_slips():
    fin = all_finite_e4m3()
    pos = fin[fin > 0]
    mids = (pos[1:] + pos[:-1]) / 2
    assert not np.array_equal(_e4m3_half_up(mids), torch_e4m3(mids))

    n, d = 130, 64
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    v[64:] *= 10.0                                     # value blocks with different scales
    s = RNG.choice([-1.0, 1.0], d)
    ro, _ = oracle.forward_head(q, k, v, 0.125, True)
    wo, _ = _forward_q_only_rotated(q, k, v, 0.125, True, s)
    assert np.abs(wo - ro).max() > 1e-3
    wo = _forward_one_v_scale(q, k, v, 0.125, True)
    assert np.abs(wo - ro).max() > 1e-3
    wo = _forward_natural_exp(q, k, v, 0.125, True)
    assert np.abs(wo - ro).max() > 1e-3
