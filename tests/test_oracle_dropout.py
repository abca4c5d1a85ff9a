"""Pins for the dropout oracle (oracle/dropout.py).

* philox(width=64) equals numpy's Philox bit generator (Philox-4x64-10, an
  independent library implementation) on several keys and counters, which
  pins the round function, word order and key schedule shared with the
  4x32 variant the method uses; the 4x32 Weyl constants are the upper halves
  of the 4x64 ones; the vectorised and scalar evaluations agree; the 4x32
  output is statistically uniform, bit-balanced and avalanches.
* keep_threshold / keep_scale closed forms; keep fractions within binomial
  bounds; p = 0 keeps everything; the mask depends on head, seed, offset.
* forward_head_dropout: p = 0 is exact attention; pure-Python brute force
  with the mask; unbiased over many seeds.
* philox(width=32) equals rocRAND's Philox-4x32-10 (its header compiled for the
  CPU) on 406 counter/key tuples.
* backward_head_dropout: central finite differences of sum(dO o O) with the
  mask fixed (dense and causal, p = 0.35 and 0.7); p = 0 is the plain
  backward.
* Planted slips fail these pins.
"""

import math
import os

import numpy as np
import pytest

import oracle
from oracle import dropout as DR

RNG = np.random.default_rng(1234)


def numpy_philox_blocks(key, counter, n_blocks):
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(counter, dtype=np.uint64))
    raw = bg.random_raw(4 * n_blocks)
    return [tuple(int(x) for x in raw[4 * b:4 * b + 4]) for b in range(n_blocks)]


def add_counter(c, inc):
    v = sum(int(w) << (64 * i) for i, w in enumerate(c)) + inc
    v %= 1 << 256
    return tuple((v >> (64 * i)) & ((1 << 64) - 1) for i in range(4))


@pytest.mark.parametrize("key,counter", [
    ((0x0123456789ABCDEF, 0xFEDCBA9876543210), (0, 0, 0, 0)),
    ((0, 0), (5, 0, 0, 0)),
    ((0xFFFFFFFFFFFFFFFF, 1), ((1 << 64) - 1, 7, 0, 0)),          # carry into word 1
    ((0x9E3779B97F4A7C15, 0x42), (3, 1 << 63, 12345, 1 << 60)),
])
def test_philox_4x64_matches_library(key, counter):
    # numpy advances its 256-bit counter by one before each block of 4 words.
    got = numpy_philox_blocks(key, counter, 3)
    for b in range(3):
        assert DR.philox(add_counter(counter, b + 1), key, width=64) == got[b]


def test_philox_variants_share_constants():
    (m32, w32), (m64, w64) = DR.PHILOX_CONSTANTS[32], DR.PHILOX_CONSTANTS[64]
    assert all(a == b >> 32 for a, b in zip(w32, w64))
    # Weyl constants: the golden ratio's fraction and sqrt(3) - 1, in units of 2^-64
    assert abs(w64[0] / 2 ** 64 - (math.sqrt(5) - 1) / 2) < 1e-15
    assert abs(w64[1] / 2 ** 64 - (math.sqrt(3) - 1)) < 1e-15


def test_philox_vector_equals_scalar():
    c = RNG.integers(0, 2 ** 32, size=(4, 50), dtype=np.uint64)
    key = (0xDEADBEEF, 0x12345678)
    vec = DR.philox(tuple(c), key)
    for n in range(50):
        sc = DR.philox(tuple(int(c[w, n]) for w in range(4)), key)
        assert tuple(int(vec[w][n]) for w in range(4)) == sc


def test_philox_4x32_statistics():
    n = 1 << 16
    ctr = (np.arange(n, dtype=np.uint64), np.zeros(n, np.uint64) + 3, np.zeros(n, np.uint64),
           np.zeros(n, np.uint64))
    out = np.stack(DR.philox(ctr, (0x1234, 0x5678))).astype(np.uint32)   # (4, n)
    by = out.view(np.uint8).ravel()
    hist = np.bincount(by, minlength=256)
    e = by.size / 256
    chi2 = float(np.sum((hist - e) ** 2 / e))
    assert 150 < chi2 < 380                    # df = 255: mean 255, sd 22.6
    bits = np.unpackbits(out.view(np.uint8), bitorder="little").reshape(4, n, 32)
    frac = bits.mean(axis=1)
    assert np.all(np.abs(frac - 0.5) < 5 * 0.5 / math.sqrt(n))
    # avalanche: neighbouring counters differ in about half of the 128 bits
    x = out[:, :-1] ^ out[:, 1:]
    flips = np.unpackbits(x.T.copy().view(np.uint8), axis=1).sum(axis=1)
    assert abs(flips.mean() - 64) < 0.5
    assert len({tuple(col) for col in out.T[:4096]}) == 4096


def test_thresholds():
    assert DR.keep_threshold(0.0) == 0 and DR.keep_scale(0.0) == 1.0
    assert DR.keep_threshold(0.1) == 26
    assert DR.keep_threshold(0.5) == 128 and DR.keep_scale(0.5) == 2.0
    assert DR.keep_threshold(0.999) == 255
    assert DR.keep_scale(0.25) == 256 / 192


def test_keep_mask():
    n = 512
    r = np.arange(n)
    for p in (0.1, 0.5):
        z = DR.keep_mask(3, r, r, seed=77, offset=5, p=p)
        keep = 1 - DR.keep_threshold(p) / 256
        sd = math.sqrt(keep * (1 - keep) / z.size)
        assert abs(z.mean() - keep) < 5 * sd
    assert DR.keep_mask(0, r[:64], r, 1, 0, 0.0).all()
    base = DR.keep_mask(1, r[:64], r[:64], 9, 0, 0.5)
    for other in (DR.keep_mask(2, r[:64], r[:64], 9, 0, 0.5), DR.keep_mask(1, r[:64], r[:64], 10, 0, 0.5),
                  DR.keep_mask(1, r[:64], r[:64], 9, 1, 0.5),
                  DR.keep_mask(1, r[:64], r[:64], 9 + (1 << 32), 0, 0.5)):
        assert 0.3 < np.mean(base != other) < 0.7
    # sub-blocks of rows/cols agree with the whole
    np.testing.assert_array_equal(DR.keep_mask(1, [5, 70], [3, 200, 511], 9, 0, 0.5),
                                  DR.keep_mask(1, r, r, 9, 0, 0.5)[np.ix_([5, 70], [3, 200, 511])])


def test_forward_p0_is_exact_attention():
    q, k, v = (RNG.standard_normal((40, 16)) for _ in range(3))
    o, l = DR.forward_head_dropout(q, k, v, 0.25, 0.0, 5, 0, 0, causal=True)
    ro, rl = oracle.forward_head(q, k, v, 0.25, causal=True)
    np.testing.assert_allclose(o, ro, atol=1e-14)
    np.testing.assert_allclose(l, rl, atol=1e-14)


def test_forward_brute_force():
    n, d, p = 9, 5, 0.3
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    z = DR.keep_mask(2, range(n), range(n), 11, 3, p)
    c = DR.keep_scale(p)
    o, _ = DR.forward_head_dropout(q, k, v, 0.4, p, 11, 3, 2, causal=True)
    for i in range(n):
        s = [0.4 * math.fsum(q[i] * k[j]) for j in range(i + 1)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        tot = math.fsum(e)
        for col in range(d):
            want = math.fsum(e[j] / tot * z[i, j] * c * v[j, col] for j in range(i + 1))
            assert abs(o[i, col] - want) < 1e-13


def test_forward_unbiased():
    n, d, p = 8, 4, 0.5
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    ro, _ = oracle.forward_head(q, k, v, 0.5)
    acc = np.zeros((n, d))
    reps = 400
    for seed in range(reps):
        acc += DR.forward_head_dropout(q, k, v, 0.5, p, seed, 0, 0)[0]
    mean = acc / reps
    # per element the sample mean has sd <= |v|max / sqrt(reps) (p = 1/2, scale 2)
    assert np.abs(mean - ro).max() < 5 * np.abs(v).max() / math.sqrt(reps)


def _loss_grads(q, k, v, do, scale, p, seed, causal, mask, eps=1e-6):
    def loss(q_, k_, v_):
        o, _ = DR.forward_head_dropout(q_, k_, v_, scale, p, seed, 2, 1, causal, mask)
        return float(np.sum(do * o))
    grads = []
    for x, idx in ((q, 0), (k, 1), (v, 2)):
        g = np.zeros_like(x)
        for ind in np.ndindex(*x.shape):
            args = [q.copy(), k.copy(), v.copy()]
            args[idx][ind] += eps
            lp = loss(*args)
            args[idx][ind] -= 2 * eps
            lm = loss(*args)
            g[ind] = (lp - lm) / (2 * eps)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal,p", [(False, 0.35), (True, 0.35), (True, 0.7)])
def test_backward_finite_differences(causal, p):
    n, d = 12, 6
    q, k, v, do = (RNG.standard_normal((n, d)) for _ in range(4))
    ana = DR.backward_head_dropout(q, k, v, do, 0.3, p, 21, 2, 1, causal, None)
    num = _loss_grads(q, k, v, do, 0.3, p, 21, causal, None)
    for a, b in zip(ana, num):
        np.testing.assert_allclose(a, b, atol=2e-7, rtol=1e-6)


def test_backward_p0_is_plain_backward():
    q, k, v, do = (RNG.standard_normal((30, 8)) for _ in range(4))
    for a, b in zip(DR.backward_head_dropout(q, k, v, do, 0.3, 0.0, 1, 0, 0, True),
                    oracle.backward_head(q, k, v, do, 0.3, causal=True)):
        np.testing.assert_allclose(a, b, atol=1e-13)


def test_backward_single_key_row_has_no_query_gradient():
    """Causal row 0 sees one key: dS_00 = P_00 (c Z_00 dP_00 - D_0) with
    D_0 = c Z_00 dP_00 exactly, so dQ_0 = 0 whatever the mask decided."""
    n, d, p = 20, 8, 0.3
    q, k, v, do = (RNG.standard_normal((n, d)) for _ in range(4))
    for seed in range(6):
        dq, _, _ = DR.backward_head_dropout(q, k, v, do, 0.3, p, seed, 0, 2, True)
        assert np.abs(dq[0]).max() < 1e-14


def _rocrand_philox(tuples):
    """rocRAND's Philox-4x32-10 round function (its header, built here with g++)."""
    import shutil
    import subprocess
    import tempfile
    src = os.path.join(os.path.dirname(__file__), "rocrand_philox_ref.cpp")
    inc = "/opt/rocm/include"
    if shutil.which("g++") is None or not os.path.exists(
            os.path.join(inc, "rocrand", "rocrand_philox4x32_10.h")):
        pytest.skip("g++ or the rocRAND headers are not installed")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "philox_ref")
        subprocess.run(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", inc, src, "-o", exe],
                       check=True, capture_output=True)
        text = "".join(" ".join(str(int(x)) for x in t) + "\n" for t in tuples)
        out = subprocess.run([exe], input=text, check=True, capture_output=True, text=True)
    return [tuple(int(w) for w in line.split()) for line in out.stdout.splitlines()]


def test_philox_4x32_matches_rocrand():
    """philox(width=32) against rocRAND's Philox-4x32-10 (a library route):
    its multipliers, Weyl constants, round function and word order."""
    m = 0xFFFFFFFF
    tuples = [(0, 0, 0, 0, 0, 0), (m, m, m, m, m, m), (1, 0, 0, 0, 0, 0), (0, 0, 0, 1, 0, 0),
              (0, 0, 0, 0, 1, 0), (0, 0, 0, 0, 0, 1)]
    tuples += [tuple(int(x) for x in RNG.integers(0, 2 ** 32, size=6, dtype=np.uint64))
               for _ in range(400)]
    ref = _rocrand_philox(tuples)
    assert len(ref) == len(tuples)
    for t, r in zip(tuples, ref):
        assert DR.philox(t[:4], t[4:], width=32) == r
    c = np.array([t[:4] for t in tuples], dtype=np.uint64).T
    vec = DR.philox(tuple(c), (tuples[-1][4], tuples[-1][5]))
    last = _rocrand_philox([tuple(int(c[w, i]) for w in range(4)) + tuples[-1][4:]
                            for i in range(c.shape[1])])
    assert [tuple(int(vec[w][i]) for w in range(4)) for i in range(c.shape[1])] == last


# ---- planted slips ----

def _bwd_mask_missing_in_dp(q, k, v, do, scale, p, seed, offset, bh, causal, mask):
    n = q.shape[0]
    rows = np.arange(n)
    pm, _ = oracle.attention._row_softmax(scale * q @ k.T, oracle.allowed(rows, n, causal, mask))
    zc = DR.keep_mask(bh, rows, rows, seed, offset, p) * DR.keep_scale(p)
    o = (pm * zc) @ v
    ds = pm * (do @ v.T - np.sum(do * o, 1)[:, None])          # mask and scale dropped
    return scale * ds @ k, scale * ds.T @ q, (pm * zc).T @ do


def _keep_strict(bh, rows, cols, seed, offset, p):
    """keep iff byte > t (instead of >=)."""
    i, j = np.meshgrid(np.asarray(rows), np.asarray(cols), indexing="ij")
    words = DR.philox(tuple(np.asarray(c, dtype=np.uint64) for c in
                            (j // 4, i // 4, np.full(i.shape, bh), np.full(i.shape, offset))),
                      (seed & 0xFFFFFFFF, seed >> 32))
    w = np.choose(i % 4, [x.astype(np.uint64) for x in words])
    byte = (w >> (np.uint64(8) * (j % 4).astype(np.uint64))) & np.uint64(0xFF)
    return byte > np.uint64(DR.keep_threshold(p))


def test_pins_catch_planted_slips():
    n, d, p = 12, 6, 0.35
    q, k, v, do = (RNG.standard_normal((n, d)) for _ in range(4))
    num = _loss_grads(q, k, v, do, 0.3, p, 21, False, None)
    wrong = _bwd_mask_missing_in_dp(q, k, v, do, 0.3, p, 21, 2, 1, False, None)
    assert np.abs(wrong[0] - num[0]).max() > 1e-3
    # "keep iff byte > t" would drop bytes equal to 0 at p = 0
    r = np.arange(256)
    assert not _keep_strict(0, r, r, 1, 0, 0.0).all()
    # a 4x64 Philox with the word order of its outputs swapped is caught
    key, c = (1, 2), (0, 0, 0, 0)
    x = DR.philox(add_counter(c, 1), key, width=64)
    assert (x[1], x[0], x[3], x[2]) != numpy_philox_blocks(key, c, 1)[0]


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_match_the_whole_head(causal):
    """forward_head_dropout(rows=...) and dq_rows_dropout give the whole-head
    functions' values at those rows (each row needs only its own scores and
    keep bytes), at rows on both sides of 4-row Philox blocks."""
    n, d, p, seed, bh = 70, 8, 0.3, 987654321, 5
    q, k, v, do = (RNG.standard_normal((n, d)) for _ in range(4))
    rows = np.array([0, 3, 4, 33, 68, 69])
    o, lse = DR.forward_head_dropout(q, k, v, 0.4, p, seed, 2, bh, causal)
    o_r, lse_r = DR.forward_head_dropout(q, k, v, 0.4, p, seed, 2, bh, causal, rows=rows)
    np.testing.assert_allclose(o_r, o[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_r, lse[rows], rtol=0, atol=1e-13)
    dq, _, _ = DR.backward_head_dropout(q, k, v, do, 0.4, p, seed, 2, bh, causal)
    dq_r = DR.dq_rows_dropout(q, k, v, do, 0.4, p, seed, 2, bh, rows, causal)
    np.testing.assert_allclose(dq_r, dq[rows], rtol=0, atol=1e-12)


def test_backward_terms_reproduce_the_whole_head():
    """backward_head_dropout_terms: its P rows sum to 1, its O is
    forward_head_dropout's, and scale dS K, scale dS^T Q, (P Z / (1 - p))^T dO
    are backward_head_dropout's gradients."""
    n, d, p, seed, scale = 50, 8, 0.25, 4242, 0.6
    q, k, v, do = (RNG.standard_normal((n, d)) for _ in range(4))
    t = DR.backward_head_dropout_terms(q, k, v, do, scale, p, seed, 3, 2, True)
    np.testing.assert_allclose(t["p"].sum(axis=1), 1.0, atol=1e-12)
    o, lse = DR.forward_head_dropout(q, k, v, scale, p, seed, 3, 2, True)
    np.testing.assert_allclose(t["o"], o, atol=1e-13)
    np.testing.assert_allclose(t["lse"], lse, atol=1e-13)
    dq, dk, dv = DR.backward_head_dropout(q, k, v, do, scale, p, seed, 3, 2, True)
    np.testing.assert_allclose(scale * t["ds"] @ k, dq, atol=1e-12)
    np.testing.assert_allclose(scale * t["ds"].T @ q, dk, atol=1e-12)
    np.testing.assert_allclose((t["p"] * t["zc"]).T @ do, dv, atol=1e-12)
