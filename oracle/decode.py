"""Decode-time attention (few queries, long key/value history), float64, CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

The sloger.press page ("Что это изменило на практике") describes decoding as
one (or a few) new queries against a long history of keys and values, with
no square score matrix, and says kernels for it parallelise the scan over the
keys and values.  The plain reading implemented here:

* queries q (Nq x d) are the last Nq positions of a sequence whose keys and
  values k, v (Nk x d, Nk >= Nq) are all cached;
* scores s_ij = scale * <q_i, k_j>; without the causal flag every query sees
  every key; with it, query i (absolute position Nk - Nq + i) sees the keys
  j <= Nk - Nq + i -- the causal rule of "Le masquage causal" (marketmaker.cc
  page) aligned to the end of the sequence, which for Nq = Nk is the square
  rule of the forward pass;
* o_i and lse_i = m_i + ln l_i as in the forward pass.

Splitting the key range into parts and combining the per-part results is the
merge of the reading guide's "Rastreamento Incremental do Softmax" (xyznot.com,
"Método"): for a row split into parts with statistics (m_s, l_s), the whole
row has m = max_s m_s and l = sum_s exp(m_s - m) l_s.  Written with one
statistic per part, lse_s = m_s + ln l_s and o_s normalised within the part,
this is lse = ln sum_s exp(lse_s) and o = sum_s exp(lse_s - lse) o_s.
"""

import numpy as np

from .attention import _row_softmax


def decode_allowed(nq, nk, causal, keys=None):
    """Boolean (nq, len(keys)): may query i attend to key j (absolute index)?"""
    keys = np.arange(nk, dtype=np.int64) if keys is None else np.asarray(keys, dtype=np.int64)
    ok = np.ones((nq, keys.size), dtype=bool)
    if causal:
        pos = nk - nq + np.arange(nq, dtype=np.int64)
        ok &= keys[None, :] <= pos[:, None]
    return ok


def decode_head(q, k, v, scale, causal=False, keys=None):
    """(o, lse) of the queries against the keys `keys` (default all of them).

    `keys` selects a contiguous or arbitrary subset of the Nk cached keys by
    absolute index; the causal rule always uses absolute positions.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    nq, nk = q.shape[0], k.shape[0]
    assert nk >= nq, "the queries are the last Nq of the Nk positions"
    sel = np.arange(nk) if keys is None else np.asarray(keys, dtype=np.int64)
    s = scale * (q @ k[sel].T)
    p, lse = _row_softmax(s, decode_allowed(nq, nk, causal, sel))
    return p @ v[sel], lse


def split_partials(q, k, v, scale, causal, bounds):
    """Per-part (o_s, lse_s) for the key ranges [bounds[s], bounds[s+1])."""
    nk = np.asarray(k).shape[0]
    assert bounds[0] == 0 and bounds[-1] == nk and all(a <= b for a, b in zip(bounds, bounds[1:]))
    parts = [decode_head(q, k, v, scale, causal, keys=np.arange(a, b))
             for a, b in zip(bounds, bounds[1:])]
    return [p[0] for p in parts], [p[1] for p in parts]


def combine(o_parts, lse_parts):
    """Merge per-part results: lse = ln sum exp(lse_s), o = sum exp(lse_s - lse) o_s.

    Parts with lse_s = -inf (no visible key) weigh nothing; a row with no
    visible key in any part gets o = 0, lse = -inf.
    """
    lse_s = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])   # (S, nq)
    o_s = np.stack([np.asarray(x, dtype=np.float64) for x in o_parts])       # (S, nq, d)
    m = lse_s.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_s - m_safe[None, :])                                      # exp(-inf) = 0
    tot = w.sum(axis=0)
    tot_safe = np.where(empty, 1.0, tot)
    lse = np.where(empty, -np.inf, m_safe + np.log(tot_safe))
    o = (w[:, :, None] * o_s).sum(axis=0) / tot_safe[:, None]
    return o, lse


def decode(q, k, v, scale, causal=False):
    """Batched (B, H, Nq, d) x (B, H, Nk, d): returns (o, lse) as float64 arrays."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, nq, d = q.shape
    o = np.zeros((B, H, nq, d))
    lse = np.zeros((B, H, nq))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = decode_head(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse
