"""Helpers for GPU-vs-oracle parity tests (test infrastructure).

The bar, per output, is a max-abs error against the fp64 oracle run on the
same rounded inputs: O, dQ, dK, dV within 1e-5 (fp32 inputs), 5e-3 (fp16) or
1.5e-2 (bf16); lse within 1e-3.
"""

import concurrent.futures
import multiprocessing
import os

import numpy as np
import torch

import oracle

TOL = {torch.float32: 1e-5, torch.float16: 5e-3, torch.bfloat16: 1.5e-2}
LSE_TOL = 1e-3
DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    inf_a, inf_b = np.isinf(a), np.isinf(b)
    assert np.array_equal(inf_a, inf_b), "infinite entries differ"
    assert np.array_equal(a[inf_a], b[inf_b]), "infinite entries differ in sign"
    fin = ~inf_a
    assert not np.isnan(a).any(), "NaN in result"
    return float(np.max(np.abs(a[fin] - b[fin]), initial=0.0))


def assert_close(name, got, ref, tol):
    err = max_abs(got, ref)
    assert err <= tol, f"{name}: max abs err {err:.3e} > {tol:.1e}"
    return err


def mask_np(mask):
    return None if mask is None else mask.cpu().numpy()


def oracle_forward_heads(q, k, v, scale, causal, mask, heads, rows=None):
    """Oracle (o, lse) for the listed (b, h) heads; q, k, v are CPU tensors."""
    out = []
    for b, h in heads:
        out.append(oracle.forward_head(f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), scale,
                                       causal=causal, block_mask=mask_np(mask), rows=rows))
    return out


def oracle_backward_heads(q, k, v, do, scale, causal, mask, heads):
    out = []
    for b, h in heads:
        out.append(oracle.backward_head(f64(q[b, h]), f64(k[b, h]), f64(v[b, h]),
                                        f64(do[b, h]), scale, causal=causal,
                                        block_mask=mask_np(mask)))
    return out


def random_block_mask(n, frac, seed, keep_diagonal=True):
    t = -(-n // 128)
    g = torch.Generator().manual_seed(seed)
    m = torch.rand((t, t), generator=g) < frac
    if keep_diagonal:
        m |= torch.eye(t, dtype=torch.bool)
    return m.to(torch.uint8)


def sample_rows(n, count, seed, must=()):
    """Sorted distinct row indices: `must` (clipped to the range) plus random ones."""
    g = np.random.default_rng(seed)
    picks = set(int(x) for x in must if 0 <= x < n)
    while len(picks) < min(n, count):
        picks.add(int(g.integers(0, n)))
    return np.array(sorted(picks), dtype=np.int64)


def oracle_backward_sampled(q, k, v, do, scale, causal, mask, samples, workers=16):
    """oracle.backward_head_sampled for many heads at once, spread over up to
    `workers` processes (spawned, one BLAS thread each; they import only numpy
    and the oracle).  samples: {(b, h): (q_rows, k_cols)}.  Returns
    {(b, h): (dq_rows, dk_cols, dv_cols)}."""
    m = mask_np(mask)
    n_workers = max(1, min(workers, os.cpu_count() or 1, len(samples)))
    saved = {key: os.environ.get(key) for key in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS")}
    for key in saved:
        os.environ[key] = "1"
    try:
        with concurrent.futures.ProcessPoolExecutor(
                n_workers, mp_context=multiprocessing.get_context("spawn")) as ex:
            futs = {}
            for (b, h), (rows, cols) in samples.items():
                args = [t[b, h].float().numpy() for t in (q, k, v, do)]
                futs[(b, h)] = ex.submit(oracle.backward_head_sampled, *args, scale, causal, m,
                                         rows, cols)
            return {key: f.result() for key, f in futs.items()}
    finally:
        for key, val in saved.items():
            if val is None:
                os.environ.pop(key, None)
            else:
                os.environ[key] = val


# Element-wise rounding bounds for the 16-bit (and fp32) kernels, from their
# arithmetic: scores, exponentials and every sum in fp32; P rounded to the
# input type before P V and P^T dO, dS before dS K and dS^T Q; D from the
# stored O; O written in the input type, gradients in fp32.  Used where the
# flat bar above does not scale: softmax scales far from 1/sqrt(d), whose
# outputs and gradients grow with the scale.
UNIT = {torch.float32: 2.0 ** -24, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}
SUBNORMAL = {torch.float32: 0.0, torch.float16: 2.0 ** -25, torch.bfloat16: 0.0}
ACC = 2.0 ** -20          # fp32 sums of up to a few thousand terms, relative to sum |terms|


def _p_rel(t, q, k, scale):
    """Relative error of the kernel's P_ij = exp(s_ij - lse_i): fp32 score
    and row statistic, each within a few ulp of its magnitude."""
    lse = np.where(np.isfinite(t["lse"]), np.abs(t["lse"]), 0.0)
    return 2.0 ** -21 * (scale * (np.abs(q) @ np.abs(k).T) + lse[:, None]) + 2.0 ** -22


def forward_bound(t, q, k, v, scale, dtype, out_rounded=True):
    """|o_kernel - o| per element: P's rounding (and its fp32 error) weighted
    by |v|, the P V sum, and the output's own rounding (out_rounded=False for
    the fp32 output of the dropout forward).  With dropout, t["zc"] (the keep
    mask times 1 / (1 - p)) weights each P in the P V product."""
    u, sub = UNIT[dtype], SUBNORMAL[dtype]
    p, av = t["p"] * t.get("zc", 1.0), np.abs(v)
    w = (u + _p_rel(t, q, k, scale) + ACC) * p + sub * (p > 0)
    return w @ av + (u if out_rounded else ACC) * np.abs(t["o"]) + 1e-6


def backward_bound(t, q, k, v, do, o_in, scale, dtype):
    """(dq, dk, dv) per-element bounds for a backward handed the output o_in
    (the pages' backward reads O from memory and forms D_i = sum_c dO_ic O_ic
    from it).  D then differs from the oracle's by the known
    dD_i = sum_c dO_ic (o_in - o)_ic, which shifts dS_ij by -P_ij dD_i: that
    shift enters dq and dk as the signed sums it is.  The rest is bounded
    term by term: P's relative error, dP's and D's fp32 sums, dS's (and,
    for dv, P's) rounding to the input type, each weighted by |k|, |q| or
    |dO|."""
    u, sub = UNIT[dtype], SUBNORMAL[dtype]
    p, ds = t["p"], np.abs(t["ds"])
    zc = t.get("zc", 1.0)              # dropout: keep mask / (1 - p) on P in dV and on dP
    aq, ak, av, ado = np.abs(q), np.abs(k), np.abs(v), np.abs(do)
    rho = _p_rel(t, q, k, scale)
    o_in = np.asarray(o_in, dtype=np.float64)
    dd = (np.asarray(do, dtype=np.float64) * (o_in - t["o"])).sum(axis=1)
    acc = ACC * (ado @ av.T) * zc + 2 * ACC * (ado * np.abs(o_in)).sum(axis=1)[:, None]
    e_ds = (u + rho + ACC) * ds + (1 + u) * p * acc + u * p * np.abs(dd)[:, None] \
        + sub * (p > 0)
    e_dq = scale * (e_ds @ ak + np.abs(dd[:, None] * (p @ k)))
    e_dk = scale * (e_ds.T @ aq + np.abs((p * dd[:, None]).T @ q))
    pv = p * zc
    e_dv = ((u + rho + ACC) * pv + sub * (pv > 0)).T @ ado
    return e_dq + 1e-6, e_dk + 1e-6, e_dv + 1e-6


def assert_within(name, got, ref, bound):
    """Every element of got within its own bound of ref."""
    got, ref = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    assert not np.isnan(got).any(), f"{name}: NaN in result"
    excess = np.abs(got - ref) - bound
    worst = np.unravel_index(int(np.argmax(excess)), excess.shape) if excess.size else None
    assert excess.size == 0 or excess.max() <= 0, \
        f"{name}: {np.abs(got - ref)[worst]:.3e} at {worst} over its bound {bound[worst]:.3e}"
    return float(np.max(np.abs(got - ref) / bound, initial=0.0))
