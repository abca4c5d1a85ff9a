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
