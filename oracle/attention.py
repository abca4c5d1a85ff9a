"""Exact attention by its plain definition, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed (per batch b, head h; Q, K, V, dO are N x d):

* scores  s_ij = scale * <q_i, k_j>           -- the scaled product of the
  "Pourquoi l'attention est liée à la mémoire" section (marketmaker.cc page)
  and of the ultralytics page's PyTorch loop.  The reading guide (xyznot.com,
  "Problema e motivação") prints S = QK^T without the scale; the scale is read
  as applied, with the value passed in by the caller.
* allowed(i, j) = (not causal or j <= i) and (mask is None or
  mask[i // 128][j // 128] != 0) -- causal rule of "Le masquage causal"
  (marketmaker.cc): keys in the future of the query are excluded, the
  diagonal kept; block mask of "Extensão: Block-Sparse FlashAttention"
  (xyznot.com), one {0,1} entry per tile pair, here fixed 128 x 128 tiles
  shared by every (b, h); the two combine with AND.
* o_i = sum_j softmax_j(s_i.) v_j over allowed j, and the per-row softmax
  statistic saved for the backward pass -- the pages keep (m, l) (section
  "Passe arrière", marketmaker.cc; "Recomputação no Backward Pass",
  xyznot.com); it is stored here as one number, lse_i = m_i + ln l_i, which
  carries the same information (P_ij = exp(s_ij - lse_i)).
* backward: P is recomputed from the scores and the row statistic (same
  sections), then the softmax chain rule, which the pages do not print:
      dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
      dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
  These are pinned by central finite differences and by torch autograd
  in tests/test_oracle_backward.py.

A row with no allowed key (only reachable with a caller's custom mask) gets
o_i = 0, lse_i = -inf and zero gradient contributions.

Rows are processed in chunks so that no N x N array is ever held; the chunk
only changes the order of summation into dK and dV.
"""

import numpy as np

MASK_BLOCK = 128


def allowed(rows, n_keys, causal, block_mask=None, mask_block=MASK_BLOCK):
    """Boolean (len(rows), n_keys): may query row i attend to key j?"""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(n_keys, dtype=np.int64)
    ok = np.ones((rows.size, n_keys), dtype=bool)
    if causal:
        ok &= cols[None, :] <= rows[:, None]
    if block_mask is not None:
        bm = np.asarray(block_mask)
        ok &= bm[rows[:, None] // mask_block, cols[None, :] // mask_block] != 0
    return ok


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _row_softmax(s, ok):
    """Two-pass softmax of each row of s over the entries where ok holds.

    Returns (P, lse); rows with no allowed entry give P = 0, lse = -inf.
    """
    s = np.where(ok, s, -np.inf)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])          # exp(-inf) = 0 on disallowed keys
    ell = e.sum(axis=1)
    ell_safe = np.where(empty, 1.0, ell)
    p = e / ell_safe[:, None]
    lse = np.where(empty, -np.inf, m_safe + np.log(ell_safe))
    return p, lse


def forward_head(q, k, v, scale, causal=False, block_mask=None,
                 mask_block=MASK_BLOCK, chunk=512, rows=None):
    """One head: returns (o, lse) for the query rows `rows` (default all).

    q: (N, d), k, v: (N, d).  `rows` lets a caller evaluate sampled rows one by
    one at sizes where the full head would be too slow.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = k.shape[0]
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    o = np.zeros((rows.size, v.shape[1]))
    lse = np.zeros(rows.size)
    for c0 in range(0, rows.size, chunk):
        r = rows[c0:c0 + chunk]
        s = scale * (q[r] @ k.T)
        p, lse[c0:c0 + r.size] = _row_softmax(s, allowed(r, n, causal, block_mask, mask_block))
        o[c0:c0 + r.size] = p @ v
    return o, lse


def rowsum_do_o(do, o):
    """D_i = sum_c dO_ic * O_ic (the backward pass's per-row term)."""
    return np.einsum("...c,...c->...", _f64(do), _f64(o))


def backward_head(q, k, v, do, scale, causal=False, block_mask=None,
                  mask_block=MASK_BLOCK, chunk=512):
    """One head: returns (dq, dk, dv), each (N, d), from its own recomputed P."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for c0 in range(0, n, chunk):
        r = np.arange(c0, min(n, c0 + chunk))
        s = scale * (q[r] @ k.T)
        p, _ = _row_softmax(s, allowed(r, n, causal, block_mask, mask_block))
        o = p @ v
        d_row = rowsum_do_o(do[r], o)
        dp = do[r] @ v.T
        ds = p * (dp - d_row[:, None])
        dv += p.T @ do[r]
        dq[r] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r])
    return dq, dk, dv


def backward_head_terms(q, k, v, do, scale, causal=False, block_mask=None,
                        mask_block=MASK_BLOCK):
    """One head's intermediate quantities of backward_head, whole (N x N):
    {"p": P, "ds": dS, "lse": lse, "o": o}, by the same definitions.  Tests
    bound a kernel's rounding error with them; small N only."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = k.shape[0]
    s = scale * (q @ k.T)
    p, lse = _row_softmax(s, allowed(np.arange(q.shape[0]), n, causal, block_mask, mask_block))
    o = p @ v
    ds = p * (do @ v.T - rowsum_do_o(do, o)[:, None])
    return {"p": p, "ds": ds, "lse": lse, "o": o}


def backward_head_sampled(q, k, v, do, scale, causal=False, block_mask=None, q_rows=(),
                          k_cols=(), mask_block=MASK_BLOCK, chunk=512):
    """One head's dq at query rows `q_rows` and dk, dv at key rows `k_cols`.

    The same definitions as backward_head, evaluated only where asked:
    dq_i = scale sum_j dS_ij k_j needs row i alone; dk_j = scale sum_i dS_ij q_i
    and dv_j = sum_i P_ij dO_i need P_ij and D_i = sum_c dO_ic o_ic of every
    row i that sees key j, so every such row is evaluated whole (its softmax
    and its output o_i), in chunks of rows; chunks that hold no sampled row
    and see none of the sampled keys are passed over.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = k.shape[0]
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_cols = np.asarray(k_cols, dtype=np.int64)
    dq = np.zeros((q_rows.size, q.shape[1]))
    dk = np.zeros((k_cols.size, k.shape[1]))
    dv = np.zeros((k_cols.size, v.shape[1]))
    for c0 in range(0, n, chunk):
        r = np.arange(c0, min(n, c0 + chunk))
        ok = allowed(r, n, causal, block_mask, mask_block)
        in_chunk = (q_rows >= c0) & (q_rows < c0 + r.size)
        sees = ok[:, k_cols]
        if not in_chunk.any() and not sees.any():
            continue
        s = scale * (q[r] @ k.T)
        p, _ = _row_softmax(s, ok)
        d_row = rowsum_do_o(do[r], p @ v)
        if in_chunk.any():
            li = q_rows[in_chunk] - c0
            ds = p[li] * (do[r][li] @ v.T - d_row[li, None])
            dq[in_chunk] = scale * (ds @ k)
        pc = p[:, k_cols]
        ds_c = pc * (do[r] @ v[k_cols].T - d_row[:, None])
        dv += pc.T @ do[r]
        dk += scale * (ds_c.T @ q[r])
    return dq, dk, dv


def _heads(x):
    x = np.asarray(x)
    return x.shape[0], x.shape[1]


def forward(q, k, v, scale, causal=False, block_mask=None, mask_block=MASK_BLOCK):
    """(B, H, N, d) inputs -> o (B, H, N, d) float64, lse (B, H, N) float64."""
    b_, h_ = _heads(q)
    o = np.zeros(np.shape(q), dtype=np.float64)
    lse = np.zeros(np.shape(q)[:3], dtype=np.float64)
    for b in range(b_):
        for h in range(h_):
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h], v[b, h], scale,
                                              causal, block_mask, mask_block)
    return o, lse


def backward(q, k, v, do, scale, causal=False, block_mask=None, mask_block=MASK_BLOCK):
    """(B, H, N, d) inputs -> dq, dk, dv (B, H, N, d) float64."""
    b_, h_ = _heads(q)
    out = [np.zeros(np.shape(q), dtype=np.float64) for _ in range(3)]
    for b in range(b_):
        for h in range(h_):
            g = backward_head(q[b, h], k[b, h], v[b, h], do[b, h], scale,
                              causal, block_mask, mask_block)
            for t, gt in zip(out, g):
                t[b, h] = gt
    return tuple(out)
