"""Host-side checks of the seeded input generators (exact_io_aware_34_amd/workloads.py)."""

import torch

from exact_io_aware_34_amd import workloads as W


def test_scale_is_fp32_rounded():
    assert W.scale_for(64) == 0.125
    s = W.scale_for(128)
    assert s == float(torch.tensor(128 ** -0.5, dtype=torch.float32))
    assert s != 128 ** -0.5


def test_draws_are_reproducible_and_rounded():
    a = W.draw_qkvdo(1, 2, 33, 8, "bf16", seed=11)
    b = W.draw_qkvdo(1, 2, 33, 8, "bf16", seed=11)
    c = W.draw_qkvdo(1, 2, 33, 8, "bf16", seed=12)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (1, 2, 33, 8)
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    # rounding is round-to-nearest-even of the fp32 draw
    g = torch.Generator().manual_seed(11)
    raw = torch.randn((4, 1, 2, 33, 8), generator=g)
    assert torch.equal(raw[0].to(torch.bfloat16), a[0])


def test_glossary_page_draw_order():
    torch.manual_seed(0)
    q, k, v = torch.randn(3, 64, 16).unbind(0)
    q2, k2, v2 = W.draw_page_qkv(64, 16, seed=0)
    assert torch.equal(q, q2) and torch.equal(k, k2) and torch.equal(v, v2)
    w = W.make("dense_n4096_d64_bf16")
    w32 = W.make("dense_n4096_d64_f32")
    assert torch.equal(w["q"].float(), w32["q"].to(torch.bfloat16).float())


def test_drift_applies_to_qkv_not_do():
    q, k, v, do = W.draw_qkvdo(1, 64, 512, 16, "f32", seed=4, drift=5.0)
    t = torch.arange(512, dtype=torch.float32) * (5.0 / 512)
    for x in (q, k, v):
        m = x.mean(dim=(0, 1, 3))
        assert torch.allclose(m, t, atol=0.15)
    assert do.mean().abs() < 0.02


def test_block_mask_density_and_diagonal():
    m = W.draw_block_mask(16384, 0.25, 50)
    assert m.shape == (128, 128) and m.dtype == torch.uint8
    assert torch.all(torch.diagonal(m) == 1)
    frac = m.float().mean().item()
    assert 0.24 < frac < 0.275                 # expected 0.25 + 0.75/128 = 0.2559
    assert torch.equal(m, W.draw_block_mask(16384, 0.25, 50))
    assert W.draw_block_mask(23400, 0.5, 1).shape == (183, 183)


def test_named_workloads_shapes():
    for name, w in W.WORKLOADS.items():
        assert w.name == name
        assert w.d in (64, 128)
    w = W.WORKLOADS[W.HEADLINE]
    assert (w.B, w.H, w.N, w.d, w.dtype, w.causal) == (4, 12, 8192, 64, "bf16", True)
    small = W.make("dense_n256_d64_f32")
    assert small["q"].shape == (1, 1, 256, 64) and small["do"] is None


def test_decode_draws_are_per_head():
    q, k, v = W.draw_decode(2, 3, 4, 50, 8, "f16", seed=9)
    assert q.shape == (2, 3, 4, 8) and k.shape == (2, 3, 50, 8) and v.dtype == torch.float16
    for b in range(2):
        for h in range(3):
            hq, hk, hv = W.draw_decode_head(b, h, 3, 4, 50, 8, "f16", seed=9)
            assert torch.equal(hq, q[b, h]) and torch.equal(hk, k[b, h]) and torch.equal(hv, v[b, h])
    # one generator per head, seeded seed * 1000003 + b * H + h, split q | k | v
    g = torch.Generator().manual_seed(9 * 1000003 + 1 * 3 + 2)
    raw = torch.randn(((4 + 100) * 8,), generator=g).to(torch.float16)
    assert torch.equal(raw[32:32 + 400].view(50, 8), k[1, 2])
    assert not torch.equal(k[0, 0], k[0, 1])


def test_decode_workload_streams_from_hbm():
    w = W.DECODE_WORKLOADS["decode_b8h12_q1_k65536_d64_bf16"]
    cache_bytes = 2 * w.B * w.H * w.Nk * w.d * 2
    assert cache_bytes > 4 * 256 * 2 ** 20        # several times the 256 MB last-level cache
    assert (w.H, w.d, w.dtype) == (W.WORKLOADS[W.HEADLINE].H, W.WORKLOADS[W.HEADLINE].d, "bf16")
