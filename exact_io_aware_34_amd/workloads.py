"""Seeded synthetic inputs for the attention workloads.

This module only draws random tensors and masks; it holds none of the
attention arithmetic, so both the HIP path's tests/bench and the CPU oracle
can take their inputs from it.  All draws are fp32 ``torch.randn`` /
``torch.rand`` on the CPU from a seeded ``torch.Generator``, then rounded to
the workload's dtype (round-to-nearest-even); every consumer reads the same
rounded values.

Workloads (B, H, N, d; dtype; masking):

=============================  ==========================  =====  ==================
name                           shape                       dtype  structure
=============================  ==========================  =====  ==================
dense_n256_d64_f32             1, 1, 256, 64               f32    dense, fwd only
dense_n4096_d64_f32            1, 1, 4096, 64              f32    dense, fwd only
dense_n4096_d64_bf16           1, 1, 4096, 64              bf16   same draws as f32
causal_b4h12_n8192_d64_bf16    4, 12, 8192, 64             bf16   causal, fwd+bwd
causal_b1h12_n23400_d64_f16    1, 12, 23400, 64            f16    causal, drift
sparse_b2h16_n16384_d128_bf16  2, 16, 16384, 128           bf16   128x128 block mask
=============================  ==========================  =====  ==================

* Values are N(0, 1).  The N=4096 pair repeats the ultralytics glossary
  page's own loop inputs: seed 0, one ``randn(3, n, d)`` unbound into q, k, v.
* The long-context fp16 workload (one trading day at 1 s resolution: 23 400
  steps, the length the marketmaker.cc page motivates) adds a slow drift
  0.01 * t / N to row t of Q, K and V before rounding; dO has no drift.
* The block-sparse mask is Bernoulli(0.25) over 128 x 128 tiles with the
  diagonal tiles always kept, one mask for every (b, h).
* Scale is 1/sqrt(d) rounded to fp32 (0.125 exactly for d = 64).

Decode workloads (few new queries against a long cached history; q is
(B, H, Nq, d), k and v are (B, H, Nk, d)):

=================================  ====================  =====  ======================
name                               B, H, Nq, Nk, d       dtype  notes
=================================  ====================  =====  ======================
decode_b8h12_q1_k65536_d64_bf16    8, 12, 1, 65536, 64   bf16   1.5 GiB K/V cache
=================================  ====================  =====  ======================

Decode draws are seeded per head (see ``draw_decode``) so that any head can be
regenerated alone on the CPU.  The head geometry (12 heads of d = 64, bf16)
is the headline workload's; one new query per sequence, 8 sequences, and a
history of 65 536 keys make the cache several times larger than the MI355X's
256 MB last-level cache, so the timed scan streams from HBM.
"""

from dataclasses import dataclass, field
from typing import Optional

import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
MASK_BLOCK = 128


def scale_for(d: int) -> float:
    """1/sqrt(d) rounded to fp32, as a Python float (exactly representable)."""
    return float(torch.tensor(1.0 / d ** 0.5, dtype=torch.float32).item())


@dataclass
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    backward: bool
    seed: int
    drift: float = 0.0
    mask_frac: Optional[float] = None
    mask_seed: Optional[int] = None
    page_layout: bool = False          # randn(3, n, d) draw order of the glossary page
    notes: str = field(default="")

    @property
    def scale(self) -> float:
        return scale_for(self.d)

    @property
    def sparse(self) -> bool:
        return self.mask_frac is not None


WORKLOADS = {
    w.name: w
    for w in [
        Workload("dense_n256_d64_f32", 1, 1, 256, 64, "f32", False, False, seed=1),
        Workload("dense_n4096_d64_f32", 1, 1, 4096, 64, "f32", False, False, seed=0,
                 page_layout=True),
        Workload("dense_n4096_d64_bf16", 1, 1, 4096, 64, "bf16", False, False, seed=0,
                 page_layout=True),
        Workload("causal_b4h12_n8192_d64_bf16", 4, 12, 8192, 64, "bf16", True, True, seed=3),
        Workload("causal_b1h12_n23400_d64_f16", 1, 12, 23400, 64, "f16", True, True, seed=4,
                 drift=0.01),
        Workload("sparse_b2h16_n16384_d128_bf16", 2, 16, 16384, 128, "bf16", False, True,
                 seed=5, mask_frac=0.25, mask_seed=50),
    ]
}

HEADLINE = "causal_b4h12_n8192_d64_bf16"


def draw_qkvdo(B, H, N, d, dtype="bf16", seed=0, drift=0.0, with_do=True):
    """Seeded (q, k, v, dO) of shape (B, H, N, d) in `dtype` (CPU tensors).

    One fp32 ``randn(4 or 3, B, H, N, d)`` draw; with drift, row t of q, k, v
    gets + drift * t / N before rounding.
    """
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((4 if with_do else 3, B, H, N, d), generator=g, dtype=torch.float32)
    if drift:
        t = torch.arange(N, dtype=torch.float32).view(N, 1) * (drift / N)
        x[:3] += t
    x = x.to(TORCH_DTYPES[dtype])
    return tuple(x.unbind(0)) + ((None,) if not with_do else ())


def draw_page_qkv(n, d, seed=0):
    """q, k, v as the glossary page draws them: seed, randn(3, n, d).unbind(0)."""
    g = torch.Generator().manual_seed(seed)
    return torch.randn((3, n, d), generator=g, dtype=torch.float32).unbind(0)


def draw_block_mask(N, frac, seed, keep_diagonal=True, block=MASK_BLOCK):
    """uint8 [ceil(N/block)][ceil(N/block)]: Bernoulli(frac) tiles, diagonal kept."""
    t = -(-N // block)
    g = torch.Generator().manual_seed(seed)
    m = torch.rand((t, t), generator=g) < frac
    if keep_diagonal:
        m |= torch.eye(t, dtype=torch.bool)
    return m.to(torch.uint8)


def make(name: str):
    """Inputs of a named workload: dict with q, k, v, do (or None), mask, ..."""
    w = WORKLOADS[name]
    if w.page_layout:
        q, k, v = draw_page_qkv(w.N, w.d, w.seed)
        q, k, v = (t.view(1, 1, w.N, w.d).to(TORCH_DTYPES[w.dtype]) for t in (q, k, v))
        do = None
    else:
        q, k, v, do = draw_qkvdo(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.drift,
                                 with_do=w.backward)
    mask = draw_block_mask(w.N, w.mask_frac, w.mask_seed) if w.sparse else None
    return dict(workload=w, q=q, k=k, v=v, do=do, mask=mask, scale=w.scale, causal=w.causal)


@dataclass
class DecodeWorkload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return scale_for(self.d)


DECODE_WORKLOADS = {
    w.name: w
    for w in [
        DecodeWorkload("decode_b8h12_q1_k65536_d64_bf16", 8, 12, 1, 65536, 64, "bf16", True,
                       seed=6),
    ]
}


def draw_decode_head(b, h, H, Nq, Nk, d, dtype="bf16", seed=0):
    """(q, k, v) of head (b, h): one fp32 randn((Nq + 2 Nk) * d) from a
    generator seeded with seed * 1000003 + b * H + h, split in that order."""
    g = torch.Generator().manual_seed(seed * 1000003 + b * H + h)
    x = torch.randn(((Nq + 2 * Nk) * d,), generator=g, dtype=torch.float32)
    x = x.to(TORCH_DTYPES[dtype])
    q = x[: Nq * d].view(Nq, d)
    k = x[Nq * d: (Nq + Nk) * d].view(Nk, d)
    v = x[(Nq + Nk) * d:].view(Nk, d)
    return q, k, v


def draw_decode(B, H, Nq, Nk, d, dtype="bf16", seed=0, device="cpu"):
    """Seeded decode inputs q (B, H, Nq, d), k, v (B, H, Nk, d) on `device`,
    filled head by head from ``draw_decode_head``."""
    dt = TORCH_DTYPES[dtype]
    q = torch.empty((B, H, Nq, d), dtype=dt, device=device)
    k = torch.empty((B, H, Nk, d), dtype=dt, device=device)
    v = torch.empty((B, H, Nk, d), dtype=dt, device=device)
    for b in range(B):
        for h in range(H):
            hq, hk, hv = draw_decode_head(b, h, H, Nq, Nk, d, dtype, seed)
            q[b, h].copy_(hq)
            k[b, h].copy_(hk)
            v[b, h].copy_(hv)
    return q, k, v


def draw_rotation_signs(d, seed):
    """The d random signs (+1 / -1, int8) of the FP8 path's rotation."""
    g = torch.Generator().manual_seed(seed)
    return (torch.randint(0, 2, (d,), generator=g, dtype=torch.int8) * 2 - 1).to(torch.int8)


def draw_outlier_qkv(B, H, N, d, dtype="bf16", seed=0, frac=1e-3, sd=10.0):
    """N(0, 1) q, k, v with a fraction `frac` of the q and k entries redrawn
    from N(0, sd^2): the outliers that FP8 quantisation handles badly."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((3, B, H, N, d), generator=g, dtype=torch.float32)
    for i in (0, 1):
        m = torch.rand((B, H, N, d), generator=g) < frac
        x[i][m] = torch.randn((int(m.sum()),), generator=g) * sd
    x = x.to(TORCH_DTYPES[dtype])
    return tuple(x.unbind(0))
