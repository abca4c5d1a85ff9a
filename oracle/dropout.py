"""Attention with dropout on the probabilities, float64, CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Dropout belongs to the fused operation: the reading guide lists it with the
matrix products, masking and softmax that one kernel fuses so that nothing
N x N goes back to HBM ("Ideias centrais", "Fusão de Kernels", xyznot.com),
and the marketmaker.cc page's integration passes `dropout_p` to PyTorch's
fused attention ("L'intégration est de huit lignes").  Plain reading, as in
that call: each probability P_ij is kept with probability 1 - p and scaled by
1 / (1 - p), or zeroed, independently; the output is O = (P o Z) V / (1 - p)
with Z the keep mask; the softmax statistic lse is that of P (before
dropout).  Differentiating with the mask fixed: dV = (P o Z)^T dO / (1 - p),
dP = (dO V^T) o Z / (1 - p), dS = P o (dP - D) with D_i = sum_c dO_ic O_ic
(O the output with dropout), dQ = scale dS K, dK = scale dS^T Q.

The mask is not stored: a counter-based generator recomputes it wherever it
is needed.  The generator is Philox-4xW-R of Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC 2011): four W-bit counter
words, two key words, R rounds of
    (x0, x1, x2, x3) <- (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0))
with the key advanced by the Weyl constants (W0, W1) between rounds.  The
method uses Philox-4x32-10.

Mapping of elements to random bits (a choice of this implementation; the
pages say nothing about it): element (query i, key j) of head bh uses byte
j mod 4 of word i mod 4 of Philox-4x32-10 at counter (j div 4, i div 4, bh,
offset) with key (seed mod 2^32, seed div 2^32); one call covers a 4 x 4
block of (query, key) pairs.  The element is kept iff that byte is >= t,
t = floor(256 p + 1/2) (clamped to 255): dropout probabilities act in steps
of 1/256, and the kept values are scaled by 1 / (1 - t / 256).
"""

import numpy as np

from .attention import _row_softmax, allowed

# Multipliers and Weyl constants of the Philox variants (Salmon et al.).
PHILOX_CONSTANTS = {
    32: ((0xD2511F53, 0xCD9E8D57), (0x9E3779B9, 0xBB67AE85)),
    64: ((0xD2E7470EE14C6C93, 0xCA5A826395121157), (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)),
}


def philox(ctr, key, width=32, rounds=10):
    """Philox-4x`width`-`rounds` of four counter words and two key words.

    Words are Python ints (any width) or, for width 32, numpy uint64 arrays
    holding 32-bit values (evaluated elementwise).
    """
    (m0, m1), (w0, w1) = PHILOX_CONSTANTS[width]
    mask = (1 << width) - 1
    x0, x1, x2, x3 = ctr
    k0, k1 = key
    vec = isinstance(x0, np.ndarray)
    if vec:
        assert width == 32
        x0, x1, x2, x3 = (np.asarray(x, dtype=np.uint64) for x in (x0, x1, x2, x3))
        k0, k1 = np.uint64(k0), np.uint64(k1)
        mask, m0, m1, w0, w1 = (np.uint64(v) for v in (mask, m0, m1, w0, w1))
        sh = np.uint64(32)
    else:
        sh = width
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + w0) & mask
            k1 = (k1 + w1) & mask
        p0 = m0 * x0           # < 2^(2 width): exact in Python ints and, for width 32, in uint64
        p1 = m1 * x2
        x0, x1, x2, x3 = (p1 >> sh) ^ x1 ^ k0, p1 & mask, (p0 >> sh) ^ x3 ^ k1, p0 & mask
    return x0, x1, x2, x3


def keep_threshold(p):
    """Byte threshold t of dropout probability p (a float32 value, 0 <= p < 1)."""
    p = float(np.float32(p))
    assert 0.0 <= p < 1.0
    return min(255, int(np.floor(p * 256.0 + 0.5)))


def keep_scale(p):
    return 256.0 / (256.0 - keep_threshold(p))


def keep_mask(bh, rows, cols, seed, offset, p):
    """Boolean keep mask of head bh for query rows x key cols."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    i = np.broadcast_to(rows[:, None], (rows.size, cols.size))
    j = np.broadcast_to(cols[None, :], (rows.size, cols.size))
    ctr = (j // 4, i // 4, np.full(i.shape, bh), np.full(i.shape, offset))
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    words = philox(tuple(np.asarray(c, dtype=np.uint64) for c in ctr), key, 32, 10)
    w = np.select([i % 4 == 0, i % 4 == 1, i % 4 == 2], list(words[:3]), words[3])
    byte = (w >> (np.uint64(8) * (j % 4).astype(np.uint64))) & np.uint64(0xFF)
    return byte >= np.uint64(keep_threshold(p))


def forward_head_dropout(q, k, v, scale, p, seed, offset, bh, causal=False, block_mask=None,
                         rows=None):
    """(o, lse) of one head with dropout on the probabilities, at query rows
    `rows` (default all): each row needs only its own scores and keep bytes."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    n = k.shape[0]
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    s = scale * (q[rows] @ k.T)
    pm, lse = _row_softmax(s, allowed(rows, n, causal, block_mask))
    z = keep_mask(bh, rows, np.arange(n), seed, offset, p)
    return (pm * z) @ v * keep_scale(p), lse


def backward_head_dropout(q, k, v, do, scale, p, seed, offset, bh, causal=False,
                          block_mask=None):
    """(dq, dk, dv) of one head with dropout, the mask held fixed.

    Everything comes from q, k, v and dO: P from the scores, the output
    O = (P o Z) V / (1 - p) that D_i = sum_c dO_ic O_ic needs is recomputed
    here, exactly.
    """
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    n = q.shape[0]
    rows = np.arange(n)
    s = scale * (q @ k.T)
    pm, _ = _row_softmax(s, allowed(rows, n, causal, block_mask))
    zc = keep_mask(bh, rows, rows, seed, offset, p) * keep_scale(p)
    pd = pm * zc
    o = pd @ v
    d = np.sum(do * o, axis=1)
    dp = (do @ v.T) * zc
    ds = pm * (dp - d[:, None])
    return scale * ds @ k, scale * ds.T @ q, pd.T @ do


def dq_rows_dropout(q, k, v, do, scale, p, seed, offset, bh, rows, causal=False,
                    block_mask=None):
    """dq of one head with dropout at query rows `rows` only, by the same
    definitions as backward_head_dropout: dq_i = scale sum_j dS_ij k_j needs
    row i's P, keep bytes, dP and D_i = sum_c dO_ic O_ic alone."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    n = k.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    s = scale * (q[rows] @ k.T)
    pm, _ = _row_softmax(s, allowed(rows, n, causal, block_mask))
    zc = keep_mask(bh, rows, np.arange(n), seed, offset, p) * keep_scale(p)
    o = (pm * zc) @ v
    d = np.sum(do[rows] * o, axis=1)
    ds = pm * ((do[rows] @ v.T) * zc - d[:, None])
    return scale * ds @ k


def backward_head_dropout_terms(q, k, v, do, scale, p, seed, offset, bh, causal=False,
                                block_mask=None):
    """One head's intermediate quantities of backward_head_dropout, whole
    (N x N): {"p": P, "zc": Z / (1 - p), "ds": dS, "lse": lse, "o": O} with
    O = (P o Z) V / (1 - p), by the same definitions.  Tests bound a kernel's
    rounding error with them; small N only."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    n = q.shape[0]
    rows = np.arange(n)
    s = scale * (q @ k.T)
    pm, lse = _row_softmax(s, allowed(rows, n, causal, block_mask))
    zc = keep_mask(bh, rows, rows, seed, offset, p) * keep_scale(p)
    o = (pm * zc) @ v
    d = np.sum(do * o, axis=1)
    ds = pm * ((do @ v.T) * zc - d[:, None])
    return {"p": pm, "zc": zc, "ds": ds, "lse": lse, "o": o}
