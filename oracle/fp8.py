"""FP8 attention with incoherent processing, emulated in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

The marketmaker.cc page (section "FA3 : Mécanique de la trémie", point 3)
describes the method in one sentence: naive FP8 attention is wrecked by outliers, so the vectors are
rotated randomly before a per-block quantisation, which spreads an outlier's
magnitude over all coordinates; it reports 2.6 times less numerical error
than naive FP8.  The steps below are the plain reading of that sentence,
in its order:

1. Rotation.  R = diag(sigma) H_d / sqrt(d), with H_d the Sylvester-Hadamard
   matrix (entries +-1, H_d H_d^T = d I) and sigma a vector of random signs
   (drawn by the caller and passed in).  R is orthogonal, so
   (q R)(k R)^T = q k^T: the scores are unchanged in exact arithmetic.
   Q and K rows are rotated; V is not (its rotation would not cancel).  The
   rotated Q is also multiplied by c = scale * log2(e), so that the scores
   below come out in base-2 units (the page leaves open where the softmax
   scale enters; here it is quantised with Q).
2. Per-block quantisation.  Each block of `block` consecutive rows of c Q R,
   of K R and of V gets one scale s, the smallest power of two with
   448 s >= amax (448 is the largest finite E4M3 value; s = 1 for an
   all-zero block, and s >= 2^-126): a shared power-of-two scale as in the
   OCP microscaling formats.  Its entries become e4m3(x / s); |x / s| <= 448.
3. Scores from the quantised operands in base 2, x_ij = s_q s_k <q8_i, k8_j>
   (exact: every FP8 product is exact in float64, and so are the
   power-of-two scales), softmax statistics m = max_j x_ij,
   l = sum_j 2^(x_ij - m) and lse = (m + log2 l) ln 2 in float64.
4. Probabilities in FP8 for the P V product: P_ij = 2^(x_ij - m_i), rounded
   to E4M3, each multiplied by its value block's scale s_v[t(j)]:
   o_i = sum_j e4m3(P_ij) s_v[t(j)] v8_j / l_i, with l_i the sum of the
   unrounded P_ij.

E4M3 is the OCP 8-bit format: 1 sign, 4 exponent (bias 7) and 3 mantissa
bits, no infinities, largest finite value 448, smallest normal 2^-6,
subnormal spacing 2^-9.  Rounding is to nearest, ties to even; values past
448 saturate to +-448 (every quantisation step above keeps |x| <= 448).
"""

import math

import numpy as np

from .attention import allowed

E4M3_MAX = 448.0


def e4m3(x):
    """Round to the nearest E4M3 value (ties to even), saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    # Spacing of the grid at |x|: 2^(e - 3) for normal values (3 fraction
    # bits), 2^-9 in the subnormal range |x| < 2^-6.
    step = np.where(ax >= 2.0 ** -6, 2.0 ** (np.maximum(e, -6) - 3), 2.0 ** -9)
    r = np.round(ax / step) * step          # numpy rounds halves to even
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, x)


def hadamard(d):
    """Sylvester-Hadamard matrix H_d (d a power of two): entries +-1."""
    assert d >= 1 and d & (d - 1) == 0
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate(x, signs):
    """Rows of x times R = diag(signs) H_d / sqrt(d)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    return (x * np.asarray(signs, dtype=np.float64)) @ hadamard(d) / math.sqrt(d)


def pow2_scale(amax):
    """The smallest power of two s with 448 s >= amax, at least 2^-126; 1 for
    amax = 0.  The comparisons 448 * 2^k >= amax are exact in float64."""
    amax = float(amax)
    if amax == 0.0:
        return 1.0
    k = math.ceil(math.log2(amax / E4M3_MAX))
    while E4M3_MAX * 2.0 ** k < amax:
        k += 1
    while E4M3_MAX * 2.0 ** (k - 1) >= amax:
        k -= 1
    return 2.0 ** max(k, -126)


def block_quantize(x, block, quantize=e4m3):
    """Per-block E4M3 quantisation of the rows of x with power-of-two scales.

    Returns (x8, scales): x8 holds the E4M3 values (as float64), scales one
    float64 per block of `block` rows, so that x ~= x8 * scale of its block.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    nb = -(-n // block)
    x8 = np.zeros_like(x)
    scales = np.ones(nb)
    for b in range(nb):
        rows = slice(b * block, min(n, (b + 1) * block))
        amax = float(np.max(np.abs(x[rows]))) if x[rows].size else 0.0
        if amax > 0:
            scales[b] = pow2_scale(amax)
            x8[rows] = quantize(x[rows] / scales[b])
    return x8, scales


def fp8_forward_head(q, k, v, scale, causal=False, block_mask=None, signs=None, block=64,
                     quantize=e4m3, rows=None, terms=False):
    """(o, lse) of one head by the FP8 method above (float64 emulation).

    signs=None skips the rotation (naive block-quantised FP8).  `quantize`
    is the rounding applied to every quantised operand; passing the identity
    turns the method into exact attention (a pin of the composition).
    `rows` restricts the output to those query rows (the operands are still
    quantised whole).  terms=True also returns the step-4 quantities as a
    dict: p (the unrounded P_ij = 2^(x_ij - m_i), 0 off the visible keys),
    sv (the value-block scale of each key), v8 and l, with
    o = (e4m3(p) * sv) @ v8 / l, and s_abs = s_q s_k <|q8_i|, |k8_j|> (the
    base-2 scores' sum of absolute products).
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    n, d = q.shape
    if signs is not None:
        q, k = rotate(q, signs), rotate(k, signs)
    c = scale * math.log2(math.e)

    q8, sq = block_quantize(q * c, block, quantize)
    k8, sk = block_quantize(k, block, quantize)
    v8, sv = block_quantize(v, block, quantize)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    rq = np.repeat(sq, block)[:n][rows]
    rk = np.repeat(sk, block)[:n]
    x = (q8[rows] * rq[:, None]) @ (k8 * rk[:, None]).T      # base-2 scores
    ok = allowed(rows, n, causal, block_mask)
    x = np.where(ok, x, -np.inf)
    m = x.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp2(x - m_safe[:, None])                  # 0 where not allowed
    ell = p.sum(axis=1)
    svk = np.repeat(sv, block)[:n]
    p8 = quantize(p)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = (p8 * svk[None, :]) @ v8 / ell[:, None]
        lse = (m_safe + np.log2(ell)) * math.log(2.0)
    o[empty] = 0.0
    lse[empty] = -np.inf
    if terms:
        s_abs = (np.abs(q8[rows]) * rq[:, None]) @ (np.abs(k8) * rk[:, None]).T
        return o, lse, {"p": p, "sv": svk, "v8": v8, "l": ell, "s_abs": s_abs}
    return o, lse


def fp8_forward(q, k, v, scale, causal=False, block_mask=None, signs=None, block=64):
    """Batched (B, H, N, d) version of fp8_forward_head."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, H, n, d = q.shape
    o = np.zeros_like(q)
    lse = np.zeros((B, H, n))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = fp8_forward_head(q[b, h], k[b, h], v[b, h], scale, causal,
                                                  block_mask, signs, block)
    return o, lse
