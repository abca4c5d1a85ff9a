"""The online-softmax recurrence, step by step, on given score blocks.

TEST INFRASTRUCTURE ONLY (see the package docstring).

These functions take the method's steps in the pages' order and notation so
the oracle's tests can show that the blockwise recurrence reaches the plain
two-pass softmax of ``attention.py`` (the pages say it is a reassociation,
exact in exact arithmetic: "La récurrence softmax en ligne", marketmaker.cc;
"Online softmax", sloger.press).  They operate on a precomputed row block of
scores so that the recurrence is tested in isolation from the products.

* ``merge_stats``: the (m, l) combination of two sub-vectors, "Rastreamento
  Incremental do Softmax" (xyznot.com, section "Método").
* ``online_softmax_normalised_each_step``: the four per-block steps of the
  same section (block max, block exponentials and sum, new global
  normalisers, output rescaled and renormalised by l_new at every block),
  which is also the order of the marketmaker.cc page's loop.
* ``online_softmax_deferred``: the variant where O stays unnormalised: each
  key block's own (max, sum, unnormalised output) is merged into the running
  triple with the merge weights, and O is divided by l once at the end (the
  deferred normalisation of the "FA2" section of marketmaker.cc; the
  ultralytics.com glossary's loop computes the same quantity).

When the running max is still -inf (no allowed key seen yet), the rescale
factor exp(m_old - m_new) is taken as 1 instead of exp(-inf + inf) = NaN; a
block whose entries are all -inf contributes nothing.
"""

import numpy as np


def _exp_diff(a, b):
    """exp(a - b) with exp(-inf - (-inf)) read as 1 (the empty-prefix case)."""
    a = np.asarray(a)
    b = np.asarray(b)
    both_empty = np.isneginf(a) & np.isneginf(b)
    with np.errstate(invalid="ignore"):
        d = np.where(both_empty, 0.0, a - b)
    return np.exp(d)


def merge_stats(m1, l1, m2, l2):
    """Combine (max, sum-of-exp) statistics of two parts of a row."""
    m = np.maximum(m1, m2)
    ell = _exp_diff(m1, m) * l1 + _exp_diff(m2, m) * l2
    return m, ell


def _blocks(n, block):
    return [(j, min(n, j + block)) for j in range(0, n, block)]


def online_softmax_normalised_each_step(s, v, block, dtype=np.float64):
    """Rows of softmax(s) @ v, visiting key blocks of width `block` in order.

    s: (R, N) scores (entries of -inf are excluded keys); v: (N, d).
    Returns (o, m, l).  Rows with no allowed key return o = 0, l = 0.
    """
    s = np.asarray(s, dtype=dtype)
    v = np.asarray(v, dtype=dtype)
    r, n = s.shape
    o = np.zeros((r, v.shape[1]), dtype=dtype)
    m = np.full(r, -np.inf, dtype=dtype)
    ell = np.zeros(r, dtype=dtype)
    for j0, j1 in _blocks(n, block):
        s_ij = s[:, j0:j1]
        m_ij = s_ij.max(axis=1)                              # block row max
        p_ij = _exp_diff(s_ij, m_ij[:, None]).astype(dtype)
        p_ij = np.where(np.isneginf(s_ij), 0.0, p_ij).astype(dtype)
        l_ij = p_ij.sum(axis=1)                               # block row sum
        m_new, l_new = merge_stats(m, ell, m_ij, l_ij)        # new normalisers
        keep = _exp_diff(m, m_new)
        take = _exp_diff(m_ij, m_new)
        safe = np.where(l_new > 0, l_new, 1.0)
        o = ((ell * keep / safe)[:, None] * o
             + (take / safe)[:, None] * (p_ij @ v[j0:j1])).astype(dtype)
        m, ell = m_new.astype(dtype), l_new.astype(dtype)
    return o, m, ell


def online_softmax_deferred(s, v, block, dtype=np.float64):
    """Same result, keeping O unnormalised until the last block.

    Each key block b contributes its own statistics (m_b, l_b) and its own
    unnormalised output u_b = sum_j exp(s_j - m_b) v_j; the running triple
    (m, l, u) absorbs them with the two weights of the incremental-softmax
    merge, exp(m - m_new) for what was there and exp(m_b - m_new) for the new
    block ("Rastreamento Incremental do Softmax", xyznot.com, section
    "Método").  Division by l happens once, after the last block (the
    deferred normalisation of the "FA2" section of marketmaker.cc).

    Returns (o, m, l).  Rows with no allowed key return o = 0, l = 0.
    """
    s = np.asarray(s, dtype=dtype)
    v = np.asarray(v, dtype=dtype)
    r, n = s.shape
    m = np.full(r, -np.inf, dtype=dtype)
    ell = np.zeros(r, dtype=dtype)
    u = np.zeros((r, v.shape[1]), dtype=dtype)
    for j0, j1 in _blocks(n, block):
        blk = s[:, j0:j1]
        m_b = blk.max(axis=1)
        e_b = np.where(np.isneginf(blk), 0.0, _exp_diff(blk, m_b[:, None])).astype(dtype)
        l_b = e_b.sum(axis=1)
        u_b = e_b @ v[j0:j1]
        m_new, ell = merge_stats(m, ell, m_b, l_b)
        w_old = _exp_diff(m, m_new).astype(dtype)[:, None]
        w_new = _exp_diff(m_b, m_new).astype(dtype)[:, None]
        u = (w_old * u + w_new * u_b).astype(dtype)
        m, ell = m_new.astype(dtype), ell.astype(dtype)
    o = u / np.where(ell > 0, ell, 1.0).astype(dtype)[:, None]
    return o.astype(dtype), m, ell
