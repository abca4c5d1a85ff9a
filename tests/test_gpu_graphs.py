"""The C ABI under HIP graph capture.

Every call only launches kernels on the caller's stream (no allocation, no
memset, no synchronisation), so a sequence of calls with caller-owned
buffers can be captured once and replayed.  The test captures a forward +
backward step, a split-KV decode, a split-key-run forward and a block-sparse
forward + backward (each with its work-order kernel) into one graph,
then replays it several times with new inputs copied into the captured
buffers by ordinary eager work between the replays, and checks every replay
bit for bit against the same calls made eagerly on separate buffers.
"""

import pytest
import torch

from exact_io_aware_34_amd import workloads as W
from tests.parity import random_block_mask

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    from exact_io_aware_34_amd import fa as _fa
    return _fa


def test_graph_replays_match_eager(fa):
    B, H, N, d = 1, 2, 576, 64
    Nq, Nk = 2, 1300
    q, k, v, do = (t.cuda() for t in W.draw_qkvdo(B, H, N, d, "bf16", seed=30))
    xq, xk, xv = (t.cuda() for t in W.draw_decode(B, H, Nq, Nk, d, "bf16", seed=31))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device="cuda")
    ws = torch.empty(fa.workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
    grads = tuple(torch.empty(B, H, N, d, device="cuda") for _ in range(3))
    xo = torch.empty_like(xq)
    xlse = torch.empty(B, H, Nq, device="cuda")
    xws = torch.empty(fa.decode_workspace_size(B, H, Nq, Nk, d, 3), dtype=torch.uint8, device="cuda")
    so = torch.empty_like(q)
    slse = torch.empty(B, H, N, device="cuda")
    sws = torch.empty(fa.forward_split_workspace_size(B, H, N, d, 4), dtype=torch.uint8,
                      device="cuda")
    # Block-sparse without the causal flag: the forward and backward each
    # launch the work-order kernel into their workspace first.
    mask = random_block_mask(N, 0.5, seed=32).cuda()
    mo = torch.empty_like(q)
    mlse = torch.empty(B, H, N, device="cuda")
    mws = torch.empty(fa.forward_split_workspace_size(B, H, N, d, 1), dtype=torch.uint8,
                      device="cuda")
    mbws = torch.empty(fa.workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
    mgrads = tuple(torch.empty(B, H, N, d, device="cuda") for _ in range(3))

    def step():
        fa.forward(q, k, v, causal=True, out=o, lse=lse, n_splits=1)
        fa.backward(q, k, v, o, lse, do, causal=True, workspace=ws, grads=grads)
        fa.decode(xq, xk, xv, causal=True, n_splits=3, out=xo, lse=xlse, workspace=xws)
        fa.forward(q, k, v, causal=True, out=so, lse=slse, n_splits=4, workspace=sws)
        fa.forward(q, k, v, block_mask=mask, out=mo, lse=mlse, n_splits=1, workspace=mws)
        fa.backward(q, k, v, mo, mlse, do, block_mask=mask, workspace=mbws, grads=mgrads)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    for seed in (40, 41, 42):
        nq, nk, nv, ndo = (t.cuda() for t in W.draw_qkvdo(B, H, N, d, "bf16", seed=seed))
        mq, mk, mv = (t.cuda() for t in W.draw_decode(B, H, Nq, Nk, d, "bf16", seed=seed + 100))
        for dst, src in ((q, nq), (k, nk), (v, nv), (do, ndo), (xq, mq), (xk, mk), (xv, mv)):
            dst.copy_(src)
        graph.replay()
        eo, el = fa.forward(nq, nk, nv, causal=True, n_splits=1)
        eg = fa.backward(nq, nk, nv, eo, el, ndo, causal=True)
        exo, exl = fa.decode(mq, mk, mv, causal=True, n_splits=3)
        eso, esl = fa.forward(nq, nk, nv, causal=True, n_splits=4)
        emo, eml = fa.forward(nq, nk, nv, block_mask=mask, n_splits=1)
        emg = fa.backward(nq, nk, nv, emo, eml, ndo, block_mask=mask)
        torch.cuda.synchronize()
        checks = [("o", o, eo), ("lse", lse, el), ("dq", grads[0], eg[0]), ("dk", grads[1], eg[1]),
                  ("dv", grads[2], eg[2]), ("decode o", xo, exo), ("decode lse", xlse, exl),
                  ("split o", so, eso), ("split lse", slse, esl), ("sparse o", mo, emo),
                  ("sparse lse", mlse, eml), ("sparse dq", mgrads[0], emg[0]),
                  ("sparse dk", mgrads[1], emg[1]), ("sparse dv", mgrads[2], emg[2])]
        for name, got, want in checks:
            assert torch.equal(got, want), f"replay with seed {seed}: {name} differs from eager"
