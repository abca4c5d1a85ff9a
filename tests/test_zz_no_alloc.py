"""fa_decode_noalloc (the decode call that allocates nothing) against
fa_decode with a caller workspace, through the C ABI.

Both run the same kernels over the same key ranges, so the results must be
identical bit for bit.  Two calls in a row share the library's device
array; the second, smaller one must not see anything the first left there.
The call is also checked in a fresh process by running this file alone.
"""

import pytest
import torch

from exact_io_aware_34_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    from exact_io_aware_34_amd import fa as _fa
    return _fa


CALLS = [
    # B, H, Nq, Nk, d, dtype, causal, n_splits
    (2, 8, 4, 5000, 64, "bf16", True, 0),       # automatic ranges
    (1, 3, 2, 1500, 128, "f16", False, 5),      # fewer heads, explicit ranges
    (1, 1, 1, 300, 64, "bf16", True, 0),        # one range: no partials at all
    (4, 12, 16, 65536, 64, "bf16", True, 0),    # the decode workload's size class
    (1, 2, 3, 700, 64, "bf16", True, 3),
]


def _draw(B, H, Nq, Nk, d, dtype, seed):
    q, k, v = W.draw_decode(B, H, Nq, Nk, d, dtype, seed=seed)
    return q.cuda(), k.cuda(), v.cuda()


def _check(fa, B, H, Nq, Nk, d, dtype, causal, n_splits, seed):
    q, k, v = _draw(B, H, Nq, Nk, d, dtype, seed)
    need = fa.decode_workspace_size(B, H, Nq, Nk, d, n_splits)
    assert need <= fa.NOALLOC_SCRATCH_BYTES
    o_ref, l_ref = fa.decode(q, k, v, causal=causal, n_splits=n_splits)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    fa.decode_noalloc(q, k, v, causal=causal, n_splits=n_splits, out=o, lse=lse)
    torch.cuda.synchronize()
    print(f"decode_noalloc B{B} H{H} Nq{Nq} Nk{Nk} d{d} {dtype} causal={causal} "
          f"ranges={fa.decode_splits(B, H, Nq, Nk, d, n_splits)} partial bytes={need}", flush=True)
    assert torch.equal(o, o_ref)
    assert torch.equal(lse, l_ref)


def test_two_calls_in_a_row_second_smaller(fa):
    _check(fa, *CALLS[0], seed=1)
    _check(fa, *CALLS[1], seed=2)


def test_every_case_and_repeats(fa):
    for i, c in enumerate(CALLS):
        _check(fa, *c, seed=10 + i)
    for i, c in enumerate(reversed(CALLS)):
        _check(fa, *c, seed=20 + i)


def test_rejects_partials_beyond_the_array(fa):
    # 64 ranges x 32 heads x 16 queries x (128 + 1) floats > 16 MiB
    B, H, Nq, Nk, d = 1, 32, 16, 64 * 128, 128
    assert fa.decode_workspace_size(B, H, Nq, Nk, d, 64) > fa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros_like(q)
    with pytest.raises(fa.FAError) as e:
        fa.decode_noalloc(q, k, k, n_splits=64, out=o)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert torch.all(o == 0)
