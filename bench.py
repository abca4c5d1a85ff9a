"""Throughput of exact attention forward + backward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                [--calibrate-copy] [--decode-workload NAME | --no-decode] [--no-fp8]
                [--no-dropout] [--dropout-p P]

A step is one forward pass and one backward pass (every kernel of the path:
forward, then the backward's dQ kernel -- which also computes each row's
D = rowsum(dO o O) -- and its dK/dV kernel) over the workload's synthetic
inputs, which are resident in HBM before the timed region starts.  The
default 30 untimed warm-up steps (about 60 ms of work) let the clocks settle:
after only 5 the timed mean of 20 steps is about 4 % higher.  FLOPs are
counted as 4*N^2*d per head for the forward and 10*N^2*d per head for the
backward, halved for causal masking and scaled by the fraction of 128x128
tiles the block mask keeps.  One JSON line is printed.

The other workloads (long-context fp16, block-sparse d = 128, and the
single-head N = 4096 bf16 / fp32 and N = 256 fp32 forwards) are timed the
same way after the headline steps and reported in the `workloads` object
(the single-head forwards through the library's default, which splits their
key ranges over more workgroups); each 16-bit forward + backward entry also
carries the FP8 forward on the same inputs (`fp8`: call time with the
preparation, its ratio to the 16-bit forward).

The decode path (fa_decode: a few queries against a long cached K/V history)
is timed after the steps on its own workload and reported in the `decode`
object of the same line: call time, algorithmic HBM bytes per call (16-bit K
and V read once, q read, o and lse written) over that time against the
8 TB/s HBM peak, and the oracle's rate on a few heads.

The same step with fused dropout (fa_forward_dropout + fa_backward_dropout,
probability 0.1 by default, a fixed seed) is timed after the plain steps and
reported in the `dropout` object, with the same FLOP count.

On workloads whose forward grid is too small to fill the GPU (fewer query
tiles in all than one round of workgroups), the `split_forward` object times
fa_forward_split with the library's number of key runs.

The FP8 forward (fa_forward_fp8: rotation + block quantisation, then
attention on E4M3 operands) is timed on the same workload and reported in the
`fp8` object: call time (both kernels), fa_fp8_prepare of all three
operands alone (the forward prepares K and V that way and each query
tile's Q inside its attention kernel), the
workload's forward FLOPs (same count as the 16-bit forward) over the call
time against the 5.0 PFLOP/s dense FP8 peak, and the oracle's float64
emulation of the method on a sample of heads.

`roofline.traffic` comes from profiles/hbm_traffic_<workload>.json (FETCH_SIZE
and WRITE_SIZE counter runs of this script, scaled by the same counters on a
plain device copy of known size, which --calibrate-copy adds before the timed
steps).  It is reported only while the kernel sources hash to the value
recorded with those counters; otherwise it is null.
"""

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3, "fp8": 5000.0}   # MI355X dense, published
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd/bwd TFLOPS (bf16, N=8192, d=64, causal) and % of MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads of the workload the oracle is timed on "
                         "(0: two per host core)")
    ap.add_argument("--other-workloads", default="causal_b1h12_n23400_d64_f16,"
                    "sparse_b2h16_n16384_d128_bf16,dense_n4096_d64_bf16,dense_n4096_d64_f32,"
                    "dense_n256_d64_f32",
                    help="comma-separated workloads also timed (fwd + bwd) and reported "
                         "in the `workloads` object; empty for none")
    ap.add_argument("--other-steps", type=int, default=20)
    ap.add_argument("--decode-workload", default="decode_b8h12_q1_k65536_d64_bf16")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-cpu-heads", type=int, default=24)
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-dropout", action="store_true")
    ap.add_argument("--dropout-p", type=float, default=0.1)
    ap.add_argument("--fp8-cpu-heads", type=int, default=2)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device-to-device copy before the steps "
                         "(reference kernel for HBM byte counters)")
    return ap.parse_args()


COPY_BYTES = 1 << 30


def kernel_sources_sha256():
    """Hash of the HIP sources the library is built from."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "exact_io_aware_34_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per call from committed counter runs, if they match the sources."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != kernel_sources_sha256():
        return None
    return rec


def work_fraction(w, mask):
    """Fraction of the dense N^2 score matrix the method evaluates."""
    frac = 0.5 if w.causal else 1.0
    if mask is not None:
        frac *= float(mask.float().mean())
    return frac


def flops(w, mask):
    f = work_fraction(w, mask) * w.N * w.N * w.d * w.B * w.H
    return 4.0 * f, 10.0 * f


def _cpu_pool_run(fn, jobs, procs):
    """Run fn(*job) for every job over `procs` spawned worker processes (one
    BLAS thread each; they import only numpy and the oracle).  The workers
    are started and warmed before the clock starts.  Returns wall seconds."""
    import concurrent.futures
    import multiprocessing

    import oracle
    saved = {k: os.environ.get(k) for k in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        with concurrent.futures.ProcessPoolExecutor(
                procs, mp_context=multiprocessing.get_context("spawn")) as ex:
            import numpy as np
            tiny = np.ones((2, 8))
            list(ex.map(oracle.rowsum_do_o, [tiny] * (4 * procs), [tiny] * (4 * procs)))
            t0 = time.perf_counter()
            for f in [ex.submit(fn, *job) for job in jobs]:
                f.result()
            return time.perf_counter() - t0
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def cpu_baseline(w, inputs, n_heads=None):
    """Time the fp64 oracle on a sample of heads of the same workload, the
    heads spread over os.cpu_count() processes with one BLAS thread each.

    All sampled heads' forwards run as one batch of jobs, then all their
    backwards; `value` is their combined FLOPs over the combined wall time
    (the same ratio as the GPU step).
    """
    import oracle
    procs = max(1, os.cpu_count() or 1)
    n = min(w.B * w.H, n_heads or 2 * procs)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)][:n]
    mask = None if inputs["mask"] is None else inputs["mask"].numpy()
    fwd_jobs, bwd_jobs = [], []
    for b, h in heads:
        a = [inputs[x][b, h].float().numpy() for x in ("q", "k", "v")]
        fwd_jobs.append((*a, w.scale, w.causal, mask))
        if w.backward:
            bwd_jobs.append((*a, inputs["do"][b, h].float().numpy(), w.scale, w.causal, mask))
    procs = min(procs, len(heads))
    t_fwd = _cpu_pool_run(oracle.forward_head, fwd_jobs, procs)
    t_bwd = _cpu_pool_run(oracle.backward_head, bwd_jobs, procs) if w.backward else 0.0
    f_fwd, f_bwd = flops(w, inputs["mask"])
    per_head_fwd = f_fwd / (w.B * w.H)
    per_head_bwd = (f_bwd if w.backward else 0.0) / (w.B * w.H)
    out = {"value": (per_head_fwd + per_head_bwd) * n / (t_fwd + t_bwd) / 1e12, "unit": "TFLOPS",
           "cores": procs, "kind": "oracle", "seconds": round(t_fwd + t_bwd, 3),
           "fwd_tflops": per_head_fwd * n / t_fwd / 1e12, "fwd_seconds": round(t_fwd, 3),
           "sample": f"{n} of {w.B * w.H} heads, forward"
                     f"{' + backward' if w.backward else ''}, numpy float64, "
                     f"{procs} processes x 1 BLAS thread, os.cpu_count()={os.cpu_count()}"}
    if w.backward:
        out["bwd_tflops"] = per_head_bwd * n / t_bwd / 1e12
        out["bwd_seconds"] = round(t_bwd, 3)
    return out


def time_passes(fa, w, tensors, mask, steps, warmup, dropout_p=0.0, seed=0):
    """Per-step forward and backward times (ms, HIP events on the launch stream)."""
    import torch
    q, k, v, do, o, lse, ws, grads = tensors
    stream = torch.cuda.current_stream()
    # With dropout the forward also writes O in fp32 for the backward's D.
    o_acc = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dropout_p else None
    # Without dropout fa.forward splits the key range of grids too small to
    # fill the GPU (the library's choice); its workspace is allocated here.
    ws_f = None
    if not dropout_p and fa.forward_splits(w.B, w.H, w.N, w.d, 0, q.dtype) > 1:
        ws_f = torch.empty(fa.forward_split_workspace_size(w.B, w.H, w.N, w.d, 0, q.dtype),
                           dtype=torch.uint8, device=q.device)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.forward(q, k, v, causal=w.causal, scale=w.scale, block_mask=mask, out=o, lse=lse,
                   dropout_p=dropout_p, seed=seed, o_acc=o_acc, workspace=ws_f)
        if ev is not None:
            ev[1].record(stream)
        if w.backward:
            fa.backward(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, block_mask=mask,
                        workspace=ws, grads=grads, dropout_p=dropout_p, seed=seed, o_acc=o_acc)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [e[0].elapsed_time(e[1]) for e in events]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in events] if w.backward else [0.0]
    return fwd_ms, bwd_ms, wall


def decode_bytes(w):
    """Algorithmic HBM bytes of one fa_decode call: K and V read once, q read,
    o written (16-bit), lse written (fp32)."""
    e = 2
    return w.B * w.H * (2 * w.Nk * w.d * e + 2 * w.Nq * w.d * e + 4 * w.Nq)


def decode_cpu_baseline(w, n_heads):
    """The oracle's decode on `n_heads` heads, as bytes-equivalent GB/s."""
    from threadpoolctl import threadpool_info

    import oracle
    from exact_io_aware_34_amd import workloads as W
    heads = [(b, h) for b in range(w.B) for h in range(w.H)][:n_heads]
    t = 0.0
    for b, h in heads:
        q, k, v = (x.double().numpy() for x in
                   W.draw_decode_head(b, h, w.H, w.Nq, w.Nk, w.d, w.dtype, seed=w.seed))
        t0 = time.perf_counter()
        oracle.decode_head(q, k, v, w.scale, w.causal)
        t += time.perf_counter() - t0
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    per_head = decode_bytes(w) / (w.B * w.H)
    return {"value": round(per_head * len(heads) / t / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds": round(t, 3),
            "sample": f"{len(heads)} of {w.B * w.H} heads, numpy float64 on the 16-bit "
                      f"inputs, os.cpu_count()={os.cpu_count()}"}


def bench_decode(fa, name, steps, warmup, cpu_heads, with_cpu):
    import torch

    from exact_io_aware_34_amd import workloads as W
    w = W.DECODE_WORKLOADS[name]
    q, k, v = W.draw_decode(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, seed=w.seed, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=q.device)
    n = fa.decode_splits(w.B, w.H, w.Nq, w.Nk, w.d, 0)
    ws = torch.empty(max(1, fa.decode_workspace_size(w.B, w.H, w.Nq, w.Nk, w.d, 0)),
                     dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()

    def call():
        fa.decode(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    mean_ms = sum(ms) / len(ms)
    byts = decode_bytes(w)
    gbs = byts / (mean_ms * 1e-3) / 1e9
    rec = recorded_traffic(name)
    out = {"workload": name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
           "causal": w.causal, "dtype": w.dtype, "key_ranges": n, "workgroups": w.B * w.H * n,
           "ms": round(mean_ms, 4),
           "ms_median_min": [round(statistics.median(ms), 4), round(min(ms), 4)],
           "keys_per_s": round(w.B * w.H * w.Nk / (mean_ms * 1e-3), 1),
           "roofline": {"bound": "hbm", "kernel": "fa_decode (dec_kernel + dec_combine)",
                        "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_call": byts,
                        "traffic": None if rec is None else rec["bytes_per_call"].get("decode"),
                        "avg_ms": round(mean_ms, 4)}}
    if with_cpu:
        out["cpu_baseline"] = decode_cpu_baseline(w, cpu_heads)
    del q, k, v, o, ws
    torch.cuda.empty_cache()
    return out


def fp8_cpu_baseline(w, inputs, signs, n_heads):
    """The oracle's float64 emulation of the FP8 forward on `n_heads` heads
    (query rows in chunks of 1024), as equivalent TFLOP/s."""
    from threadpoolctl import threadpool_info

    import oracle
    heads = [(b, h) for b in range(w.B) for h in range(w.H)][:n_heads]
    sg = signs.numpy().astype("float64")
    t = 0.0
    for b, h in heads:
        a = [inputs[n][b, h].double().numpy() for n in ("q", "k", "v")]
        for r0 in range(0, w.N, 1024):
            rows = list(range(r0, min(w.N, r0 + 1024)))
            t0 = time.perf_counter()
            oracle.fp8_forward_head(*a, w.scale, w.causal, None, sg, rows=rows)
            t += time.perf_counter() - t0
    f_fwd, _ = flops(w, inputs["mask"])
    per_head = f_fwd / (w.B * w.H)
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] + [1])
    return {"value": round(per_head * len(heads) / t / 1e12, 5), "unit": "TFLOPS", "cores": threads,
            "kind": "oracle", "seconds": round(t, 3),
            "sample": f"{len(heads)} of {w.B * w.H} heads, float64 emulation of the FP8 method "
                      f"(operands quantised whole, query rows in chunks of 1024), "
                      f"os.cpu_count()={os.cpu_count()}"}


def bench_split(fa, w, tensors, mask, steps, warmup, fwd_ms):
    """fa_forward_split with the library's run count, for workloads whose
    plain forward grid is too small to fill the GPU."""
    import torch
    q, k, v, _, o, lse, _, _ = tensors
    n = fa.forward_splits(w.B, w.H, w.N, w.d, 0, q.dtype)
    ws = torch.empty(max(1, fa.forward_split_workspace_size(w.B, w.H, w.N, w.d, 0, q.dtype)),
                     dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()

    def call():
        fa.forward(q, k, v, causal=w.causal, scale=w.scale, block_mask=mask, out=o, lse=lse,
                   n_splits=0, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    mean = sum(ms) / len(ms)
    f_fwd, _ = flops(w, mask.cpu() if mask is not None else None)
    tf = f_fwd / (mean * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    return {"n_splits": n, "workgroups": ((w.N + 127) // 128) * w.B * w.H * n,
            "ms": round(mean, 4),
            "ms_median_min": [round(statistics.median(ms), 4), round(min(ms), 4)],
            "tflops": round(tf, 2), "frac_peak": round(tf / peak, 4),
            "vs_plain_forward": round(fwd_ms / mean, 3),
            "kernels": "forward kernel over key runs + dec_combine merge"}


def bench_fp8(fa, w, inputs, tensors, mask, steps, warmup, cpu_heads, with_cpu):
    import torch

    from exact_io_aware_34_amd import workloads as W
    q, k, v, _, o, lse, _, _ = tensors
    signs = W.draw_rotation_signs(w.d, seed=7)
    sd = signs.to(q.device)
    ws = torch.empty(fa.fp8_workspace_size(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    call = timed(lambda: fa.forward_fp8(q, k, v, signs=sd, causal=w.causal, scale=w.scale,
                                        block_mask=mask, out=o, lse=lse, workspace=ws))
    prep = timed(lambda: fa.fp8_prepare(q, k, v, sd, scale=w.scale, workspace=ws))
    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    f_fwd, _ = flops(w, mask.cpu() if mask is not None else None)
    tf = f_fwd / (mean(call) * 1e-3) / 1e12
    rec = recorded_traffic(w.name)
    out = {"workload": w.name, "rotation": "random Hadamard (seeded signs)",
           "ms": round(mean(call), 4),
           "ms_median_min": [round(statistics.median(call), 4), round(min(call), 4)],
           "prep_ms": round(mean(prep), 4), "tflops": round(tf, 2),
           "vs_bf16_forward": None,
           "roofline": {"bound": "mfma", "kernel": "fa_forward_fp8 (fp8_prep + fwd8)",
                        "achieved": round(tf, 2), "peak": PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_TFLOPS["fp8"], 4),
                        "traffic": None if rec is None else rec["bytes_per_call"].get("fp8"),
                        "avg_ms": round(mean(call), 4)}}
    if with_cpu:
        out["cpu_baseline"] = fp8_cpu_baseline(w, inputs, signs, cpu_heads)
    return out


def bench_dropout(fa, w, tensors, mask, steps, warmup, p, plain_ms):
    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    seed = 20260101
    fwd_ms, bwd_ms, wall = time_passes(fa, w, tensors, mask, steps, warmup, dropout_p=p, seed=seed)
    f_fwd, f_bwd = flops(w, mask.cpu() if mask is not None else None)
    ms_step = wall * 1e3 / steps
    tf_bwd = f_bwd / (mean(bwd_ms) * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    rec = recorded_traffic(w.name)
    out = {"dropout_p": p, "seed": seed, "value": round((f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12, 2),
           "unit": "TFLOPS", "ms_per_step": round(ms_step, 4),
           "fwd_ms": round(mean(fwd_ms), 4), "bwd_ms": round(mean(bwd_ms), 4),
           "fwd_tflops": round(f_fwd / (mean(fwd_ms) * 1e-3) / 1e12, 2),
           "bwd_tflops": round(tf_bwd, 2),
           "step_time_vs_plain": round(ms_step / plain_ms, 3),
           "roofline": {"bound": "mfma", "kernel": "fa_backward_dropout (bwd_dq + bwd_dkdv)",
                        "achieved": round(tf_bwd, 2), "peak": peak, "unit": "TFLOP/s",
                        "frac": round(tf_bwd / peak, 4),
                        "traffic": None if rec is None else rec["bytes_per_call"].get("dropout_backward"),
                        "avg_ms": round(mean(bwd_ms), 4)}}
    return out


def pass_summary(w, mask_cpu, fwd_ms, bwd_ms, wall, steps):
    """Per-pass times, TFLOP/s, fractions of peak and the roofline of the
    dominant call (the backward when present: its kernels run back to back
    on the stream and are timed together; else the forward kernel)."""
    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    f_fwd, f_bwd = flops(w, mask_cpu)
    if not w.backward:
        f_bwd = 0.0
    ms_step = wall * 1e3 / steps
    peak = PEAK_TFLOPS[w.dtype]
    fwd_tf = f_fwd / (mean(fwd_ms) * 1e-3) / 1e12
    bwd_tf = f_bwd / (mean(bwd_ms) * 1e-3) / 1e12 if w.backward else None
    if w.backward and mean(bwd_ms) >= mean(fwd_ms):
        dom, dom_key, dom_ms, dom_flops = ("fa_backward (bwd_dq + bwd_dkdv)", "backward",
                                           mean(bwd_ms), f_bwd)
    else:
        dom, dom_key, dom_ms, dom_flops = "fa_forward (fwd kernel)", "forward", mean(fwd_ms), f_fwd
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    rec = recorded_traffic(w.name)
    traffic = None if rec is None else rec["bytes_per_call"].get(dom_key)
    return {
        "value": round((f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12, 2),
        "ms_per_step": round(ms_step, 4),
        "fwd_ms": round(mean(fwd_ms), 4), "bwd_ms": round(mean(bwd_ms), 4),
        "fwd_ms_median_min": [round(statistics.median(fwd_ms), 4), round(min(fwd_ms), 4)],
        "bwd_ms_median_min": [round(statistics.median(bwd_ms), 4), round(min(bwd_ms), 4)],
        "fwd_tflops": round(fwd_tf, 2), "fwd_frac_peak": round(fwd_tf / peak, 4),
        "bwd_tflops": None if bwd_tf is None else round(bwd_tf, 2),
        "bwd_frac_peak": None if bwd_tf is None else round(bwd_tf / peak, 4),
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic, "avg_ms": round(dom_ms, 4)},
    }


def skip_efficiency(fa, w, tensors, mask, steps, fwd_ms, bwd_ms):
    """(T_dense / T_sparse) / (1 / kept fraction), the dense time from the
    same kernels with no mask."""
    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    d_fwd, d_bwd, _ = time_passes(fa, w, tensors, None, max(3, steps // 2), 2)
    kept = float(mask.float().mean())
    return {"kept_tile_fraction": round(kept, 5),
            "fwd": round(mean(d_fwd) / mean(fwd_ms) * kept, 4),
            "bwd": round(mean(d_bwd) / mean(bwd_ms) * kept, 4) if w.backward else None,
            "dense_fwd_ms": round(mean(d_fwd), 4),
            "dense_bwd_ms": round(mean(d_bwd), 4) if w.backward else None}


def workload_tensors(fa, w, inputs, dev):
    import torch
    q, k, v = (inputs[n].to(dev) for n in ("q", "k", "v"))
    do = inputs["do"].to(dev) if w.backward else None
    mask = None if inputs["mask"] is None else inputs["mask"].to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device=dev)
                  for _ in range(3)) if w.backward else None
    ws = torch.empty(max(1, fa.workspace_size(w.B, w.H, w.N, w.d)), dtype=torch.uint8, device=dev)
    return (q, k, v, do, o, lse, ws, grads), mask


def bench_other(fa, name, steps, warmup):
    """Forward + backward of another workload: the same fields as the line."""
    import torch

    from exact_io_aware_34_amd import workloads as W
    w = W.WORKLOADS[name]
    inputs = W.make(name)
    tensors, mask = workload_tensors(fa, w, inputs, torch.device("cuda:0"))
    fwd_ms, bwd_ms, wall = time_passes(fa, w, tensors, mask, steps, warmup)
    out = {"B": w.B, "H": w.H, "N": w.N, "d": w.d, "dtype": w.dtype, "causal": w.causal,
           "block_sparse": w.sparse, "steps": steps, "warmup": warmup,
           "work_fraction": round(work_fraction(w, inputs["mask"]), 5),
           "forward_key_runs": fa.forward_splits(w.B, w.H, w.N, w.d, 0, W.TORCH_DTYPES[w.dtype])}
    out.update(pass_summary(w, inputs["mask"], fwd_ms, bwd_ms, wall, steps))
    if w.sparse:
        out["skip_efficiency"] = skip_efficiency(fa, w, tensors, mask, steps, fwd_ms, bwd_ms)
    if w.backward and w.dtype in ("bf16", "f16"):
        # The FP8 forward on the same inputs (rotation + quantisation included).
        f8 = bench_fp8(fa, w, inputs, tensors, mask, steps, warmup, 0, False)
        out["fp8"] = {k_: f8[k_] for k_ in ("ms", "ms_median_min", "prep_ms", "tflops")}
        out["fp8"]["frac_fp8_peak"] = f8["roofline"]["frac"]
        out["fp8"]["vs_16bit_forward"] = round(sum(fwd_ms) / len(fwd_ms) / f8["ms"], 3)
    del tensors, mask
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard over independent (batch, head) pairs with no "
              "communication; that sharding is not built)", file=sys.stderr)
        sys.exit(2)
    import torch

    from exact_io_aware_34_amd import build as _build
    if not os.path.exists(_build.LIB):
        _build.build()
    from exact_io_aware_34_amd import fa
    from exact_io_aware_34_amd import workloads as W

    name = args.workload or W.HEADLINE
    w = W.WORKLOADS[name]
    inputs = W.make(name)
    dev = torch.device("cuda:0")
    B, H, N, d = w.B, w.H, w.N, w.d
    tensors, mask = workload_tensors(fa, w, inputs, dev)
    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    fwd_ms, bwd_ms, wall = time_passes(fa, w, tensors, mask, args.steps, args.warmup)

    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    summary = pass_summary(w, inputs["mask"], fwd_ms, bwd_ms, wall, args.steps)
    ms_step = summary["ms_per_step"]
    out = {
        "metric": METRIC if name == W.HEADLINE else f"attention TFLOPS ({name})",
        "value": summary["value"], "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "block_sparse": w.sparse, "passes": "fwd+bwd" if w.backward else "fwd",
                   "work_fraction": round(work_fraction(w, inputs["mask"]), 5)},
    }
    out.update({k_: v_ for k_, v_ in summary.items() if k_ not in ("value", "ms_per_step")})
    if w.sparse:
        out["skip_efficiency"] = skip_efficiency(fa, w, tensors, mask, args.steps, fwd_ms, bwd_ms)
    if fa.forward_splits(B, H, N, d, 0, W.TORCH_DTYPES[w.dtype]) > 1:
        out["split_forward"] = bench_split(fa, w, tensors, mask, args.steps, args.warmup,
                                           mean(fwd_ms))
    if not args.no_dropout and w.dtype in ("bf16", "f16") and w.backward:
        out["dropout"] = bench_dropout(fa, w, tensors, mask, args.steps, args.warmup,
                                       args.dropout_p, ms_step)
    if not args.no_fp8 and w.dtype in ("bf16", "f16"):
        out["fp8"] = bench_fp8(fa, w, inputs, tensors, mask, args.steps, args.warmup,
                               args.fp8_cpu_heads, not args.no_cpu_baseline)
        out["fp8"]["vs_bf16_forward"] = round(mean(fwd_ms) / out["fp8"]["ms"], 3)
    if not args.no_decode:
        out["decode"] = bench_decode(fa, args.decode_workload, args.steps, args.warmup,
                                     args.decode_cpu_heads, not args.no_cpu_baseline)
    others = [x for x in args.other_workloads.split(",") if x and x != name]
    if others:
        del tensors, mask
        torch.cuda.empty_cache()
        out["workloads"] = {x: bench_other(fa, x, args.other_steps, max(5, args.other_steps // 2))
                            for x in others}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_heads or None)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
