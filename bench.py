"""Anchor-attention throughput on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--plan auto|fused|split]
                [--pass forward|backward|block|linear|nystrom] [--head-dim D] [--anchors M]
                [--no-cpu-baseline]

One step = one forward of the whole hot path (logits, softmax, column sums and A^T V,
normalisation, H = A W) over one batch of the workload; with --pass backward, one
backward (dQ, dU, dV for a given dL/dH) instead; with --pass block, one attention block
(Q|V projection, the layer on the projection in place, output projection) with the
workload's B, n, h, m, d; with --pass linear, the ReLU kernel linear attention (L2ViT
page) on the workload's Q, K, V.  Inputs are resident in HBM:
R copies of the batch (R * bytes >= 1 GiB, well beyond the 256 MB Infinity Cache) are
cycled so every step reads cold HBM.  K steps are bracketed by events on the launch
stream.  Prints one JSON line; for the forward it carries `parity`, the output of the last
timed launch against the fp64 oracle on sampled slices, and the run exits with status 1
when that error is past the gate.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # dense MFMA bf16, published
FP32_PEAK_TFLOPS = 157.3       # fp32 matrix, published
ROTATE_BYTES = 1 << 30

# HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (each scaled by the
# reading of a plain copy kernel of known size; see profiles/).  Valid only while the
# kernel's sources hash to the recorded fingerprint; otherwise traffic is reported null.
MEASURED_TRAFFIC = {
    ("vit_s16_224", "fused"): {"sources": ["efficient_vision_transformer_amd/csrc/fused_bf16.hip",
                                           "efficient_vision_transformer_amd/csrc/tile_ops.h",
                                           "efficient_vision_transformer_amd/csrc/device_common.h",
                                           "efficient_vision_transformer_amd/csrc/geometry.h"],
                               "sha": "84710bd8b22f54c8", "read_bytes": 19471753,
                               "write_bytes": 10890544},
}
# the split plan's three kernels per step (pass 1, finalize, pass 2)
_SPLIT_SOURCES = ["efficient_vision_transformer_amd/csrc/split_bf16.hip",
                  "efficient_vision_transformer_amd/csrc/tile_ops.h",
                  "efficient_vision_transformer_amd/csrc/device_common.h",
                  "efficient_vision_transformer_amd/csrc/geometry.h",
                  "efficient_vision_transformer_amd/csrc/pass2_layout.h",
                  "efficient_vision_transformer_amd/csrc/split_plan.h"]   # the chunking
MEASURED_TRAFFIC[("dense_64x64", "split")] = {"sources": _SPLIT_SOURCES, "sha": "fcab4de23b77c240",
                                             "read_bytes": 111445946, "write_bytes": 46439736}
MEASURED_TRAFFIC[("long_16k_bf16", "split")] = {"sources": _SPLIT_SOURCES, "sha": "fcab4de23b77c240",
                                               "read_bytes": 244297780, "write_bytes": 111275950}


def measured_traffic(workload: str, plan: str):
    import hashlib
    rec = MEASURED_TRAFFIC.get((workload, plan))
    if rec is None:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest()[:16] != rec["sha"]:
        return None
    return rec["read_bytes"] + rec["write_bytes"]


# Device-side delay queued just before the start event (GPU clock ticks of torch's spin
# kernel; tens of microseconds to a few milliseconds depending on the counter's rate).
LEAD_IN_CYCLES = 1_000_000


def timed_steps(step, warmup: int, steps: int, stream, sets: int = 0) -> float:
    """Average milliseconds per step on `stream`.

    step(i) enqueues step i (callers rotate over `sets` buffer sets with i).  First every
    set is touched once by an untimed step (so no timed step meets pages the device has
    not mapped since their allocation); then warm-up steps 0 .. warmup - 1 run untimed and
    the timed steps are warmup .. warmup + steps - 1, so with enough sets none of them
    reuses a set still in the caches.  Both ends are bracketed by a device
    synchronisation.  A spin kernel is queued right before the start event: while it runs,
    the host enqueues the first timed launches, so the window holds the K launches back to
    back rather than the host's latency to its first launch on an idle GPU."""
    import torch
    torch.cuda.synchronize()
    for i in range(sets):
        step(i)
    torch.cuda.synchronize()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(LEAD_IN_CYCLES)
    e0.record(stream)
    for i in range(steps):
        step(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def host_info() -> dict:
    """Threads this process may use, nproc, the host's CPU count and its CPU model."""
    import subprocess
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = int(subprocess.run(["nproc"], capture_output=True, text=True, check=True).stdout)
    except (OSError, ValueError, subprocess.CalledProcessError):
        nproc = None
    return {"affinity_cores": len(os.sched_getaffinity(0)), "nproc": nproc,
            "cpu_count": os.cpu_count(), "cpu_model": model}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--plan", default="auto", choices=["auto", "fused", "split"])
    ap.add_argument("--pass", dest="which", default="forward",
                    choices=["forward", "backward", "block", "linear", "nystrom"])
    ap.add_argument("--head-dim", type=int, default=0,
                    help="override the workload's head dim (32, 64 or 128)")
    ap.add_argument("--anchors", type=int, default=0,
                    help="override the workload's anchor count (up to 512)")
    ap.add_argument("--landmarks", type=int, default=0,
                    help="landmarks for --pass nystrom (default: per workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="instead of the benchmark, run a plain device copy of this many MiB "
                         "(reference reading for the HBM byte counters)")
    return ap.parse_args()


def calibrate_copy(mib: int, reps: int = 5) -> None:
    """A plain copy kernel of known size: reads and writes `mib` MiB per launch."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(mib << 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": mib << 20,
                      "bytes_written_per_launch": mib << 20, "launches": reps}), flush=True)


def cpu_baseline(x, seconds: float) -> dict:
    """The fp64 oracle as it stands, on this host's cores: whole batches of the same
    workload repeated until `seconds` of wall clock have elapsed, on the threads one GPU's
    share of the host allows (all cores this process may use, at most 16); then once on a
    single thread, over the whole batch when it has at most 2^30 multiply-adds per logits
    product, else over its first four slices, extrapolated to the batch."""
    import numpy as np
    import oracle
    cores = oracle.default_threads()
    Q, U, V = (np.asarray(a, dtype=np.float64) for a in (x.Q, x.U, x.V))
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.anchor_attn(Q, U, V, nthreads=cores)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    w = x.workload
    whole = w.B * w.h * w.n * w.m * w.d <= (1 << 30)
    if whole:
        q1, v1, scale, what = Q, V, 1.0, "the whole batch"
    else:
        q1 = Q.reshape(w.B * w.h, w.n, w.d)[:4].reshape(1, 4, w.n, w.d)
        v1 = V.reshape(w.B * w.h, w.n, w.d)[:4].reshape(1, 4, w.n, w.d)
        u1 = np.stack([U[j % w.h] for j in range(4)])
        scale, what = w.B * w.h / 4.0, f"4 of {w.B * w.h} slices, extrapolated"
    t1 = time.perf_counter()
    if whole:
        oracle.anchor_attn(q1, U, v1, nthreads=1)
    else:
        oracle.anchor_attn(q1, u1, v1, nthreads=1)
    el1 = (time.perf_counter() - t1) * scale
    out = {"value": reps * w.B * w.n / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"{reps} full batch(es) of {w.name} (B={w.B} h={w.h} n={w.n} m={w.m} d={w.d}) "
                     f"in fp64 on {cores} threads, {el:.1f} s wall",
           "value_1thread": w.B * w.n / el1,
           "sample_1thread": f"{what} on one thread, {el1:.2f} s per batch"}
    out.update(host_info())
    return out


def cpu_baseline_backward(x, G, seconds: float) -> dict:
    """The fp64 oracle's gradients as they stand, timed like cpu_baseline."""
    import numpy as np
    import oracle
    cores = oracle.default_threads()
    Q, U, V, G = (np.asarray(a, dtype=np.float64) for a in (x.Q, x.U, x.V, G))
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.anchor_backward(Q, U, V, G, nthreads=cores)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    w = x.workload
    return {"value": reps * w.B * w.n / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} full backward(s) of {w.name} (B={w.B} h={w.h} n={w.n} m={w.m} "
                      f"d={w.d}) in fp64, {el:.1f} s wall"}


def backward_bytes_flops(w) -> tuple[int, int]:
    """Algorithmic bytes and flops of one backward: Q, V, dH read and dQ, dV written once,
    U read and dU written once; 2nmd flops each for the logits, A^T V, A^T dH, dH W^T,
    V dP^T, dS U, A dP and dS^T Q per slice."""
    es = w.elem_bytes
    act = w.B * w.h * w.n * w.d * es
    return 5 * act + 2 * w.h * w.m * w.d * es, 16 * w.B * w.h * w.n * w.m * w.d


def bench_backward(args, ctx, x, dev, plan_desc) -> dict:
    import numpy as np
    import torch
    from efficient_vision_transformer_amd.inputs import make_upstream_grad
    w = x.workload
    G, gbits = make_upstream_grad(x, w.seed + 1)
    if w.dtype == "bf16":
        up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
        Q0, U, V0, G0 = up(x.bits["Q"]), up(x.bits["U"]), up(x.bits["V"]), up(gbits)
    else:
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
        Q0, U, V0, G0 = up(x.Q), up(x.U), up(x.V), up(G)
    algo_bytes, flops = backward_bytes_flops(w)
    R = max(1, -(-ROTATE_BYTES // algo_bytes))
    mk = lambda q, v, g: (q, v, g, (torch.empty_like(q), torch.empty_like(U), torch.empty_like(v)))
    sets = [mk(Q0, V0, G0)] + [mk(Q0.clone(), V0.clone(), G0.clone()) for _ in range(R - 1)]
    stream = torch.cuda.current_stream(dev)

    def step(i):
        q, v, g, o = sets[i % R]
        ctx.backward(q, U, v, g, out=o, stream=stream)
    ms = timed_steps(step, args.warmup, args.steps, stream, R)
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    # the bound is whichever floor is higher: the bytes at HBM peak or the flops at the
    # dense MFMA peak of the dtype (the long and dense workloads' many anchors, and fp32,
    # make it the latter)
    peak_tf = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    if flops / (peak_tf * 1e12) > algo_bytes / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak_tf,
                "unit": "TFLOP/s", "frac": round(tflops / peak_tf, 4), "traffic": None}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}
    roof.update({
            "kernel": ("whole backward (pass1 x2 + finalize + tokens + dU reduction)"
                       if w.dtype == "bf16" else
                       "whole backward (pass1 x2 + finalize + tokens + dS^T Q + dU reduction)"),
            "per_launch": {"algorithmic_bytes": algo_bytes, "algorithmic_flops": flops,
                           "avg_duration_us": round(ms * 1e3, 3)}})
    out = {
        "metric": f"anchor-attention backward tokens/sec ({w.name})",
        "value": round(w.B * w.n / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "backward", "B": w.B, "h": w.h, "n": w.n,
                   "m": w.m, "d": w.d, "global_batch": w.B, "seq_len": w.n,
                   "parallelism": "single-gpu", "forward_plan": plan_desc, "rotating_sets": R},
        "achieved_hbm_gbs": round(gbs, 1),
        "achieved_tflops": round(tflops, 3),
        "roofline": roof,
    }
    ref = copy_reference(algo_bytes, min(args.steps, 200), min(args.warmup, 20))
    ref["frac_of_copy"] = round(gbs / ref["gbs"], 4) if ref["gbs"] > 0 else None
    out["copy_reference"] = ref
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_backward(x, G, args.cpu_seconds)
    return out


def block_bytes_flops(w) -> tuple[int, int]:
    """Algorithmic bytes and flops of one attention block (C = h*d, T = B*n tokens): X
    read, [Q|V] written and read, H written and read, Y written, the weights and biases
    read once; flops of the two projections (2*T*C*2C and 2*T*C*C) plus the layer."""
    C, T, es = w.h * w.d, w.B * w.n, w.elem_bytes
    act = T * C * es
    return (act + 2 * 2 * act + 2 * act + act + (3 * C * C + 3 * C + w.h * w.m * w.d) * es,
            6 * T * C * C + w.algorithmic_flops())


def cpu_baseline_block(x, seconds: float) -> dict:
    """The fp64 oracle's block as it stands, timed like cpu_baseline."""
    import oracle
    cores = oracle.default_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.anchor_block_forward(x.X, x.Wqv, x.bqv, x.U, x.Wo, x.bo)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": reps * x.B * x.n / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} full block(s) (B={x.B} n={x.n} h={x.h} m={x.m} d={x.d}) in fp64 "
                      f"with numpy projections, {el:.1f} s wall"}


def bench_block(args, ctx, w, dev) -> dict:
    import numpy as np
    import torch
    from efficient_vision_transformer_amd.inputs import make_block_inputs
    if w.dtype != "bf16":
        raise SystemExit("the block runs in bf16 only")
    x = make_block_inputs(w.B, w.n, w.h, w.m, w.d, seed=w.seed)
    conv = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    t = {k: conv(v) for k, v in x.bits.items()}
    algo_bytes, flops = block_bytes_flops(w)
    act = w.B * w.n * w.h * w.d * 2
    R = max(1, -(-ROTATE_BYTES // (2 * act)))
    sets = [(t["X"], torch.empty_like(t["X"]))] + [(t["X"].clone(), torch.empty_like(t["X"]))
                                                   for _ in range(R - 1)]
    stream = torch.cuda.current_stream(dev)
    step = lambda i: ctx.block_forward(sets[i % R][0], t["Wqv"], t["bqv"], t["U"], t["Wo"],
                                       t["bo"], out=sets[i % R][1], stream=stream)
    ms = timed_steps(step, args.warmup, args.steps, stream, R)
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    hbm_bound = algo_bytes / (HBM_PEAK_GBS * 1e9) >= flops / (BF16_PEAK_TFLOPS * 1e12)
    roof = ({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(gbs / HBM_PEAK_GBS, 4)} if hbm_bound else
            {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4)})
    roof.update({"traffic": None,
                 "kernel": "whole block (Q|V projection fused into the layer's kernel, hipBLASLt "
                           "output projection)" if (w.m <= 32 and w.n <= 256 and w.d <= 64 and
                                                   args.plan != "split")
                 else "whole block (hipBLASLt projection, the layer, hipBLASLt projection)",
                 "per_launch": {"algorithmic_bytes": algo_bytes, "algorithmic_flops": flops,
                                "avg_duration_us": round(ms * 1e3, 3)}})
    out = {
        "metric": f"anchor-attention block tokens/sec ({w.name} shape, C={w.h * w.d})",
        "value": round(w.B * w.n / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "block", "B": w.B, "n": w.n, "h": w.h, "m": w.m,
                   "d": w.d, "C": w.h * w.d, "global_batch": w.B, "seq_len": w.n,
                   "parallelism": "single-gpu", "rotating_sets": R},
        "achieved_hbm_gbs": round(gbs, 1), "achieved_tflops": round(tflops, 3),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_block(x, args.cpu_seconds)
    return out


def bench_linear(args, ctx, x, dev) -> dict:
    import numpy as np
    import torch
    w = x.workload
    if w.dtype != "bf16":
        raise SystemExit("the linear attention runs in bf16 only")
    conv = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    Q0, K0, V0 = conv(x.bits["Q"]), conv(x.bits["K"]), conv(x.bits["V"])
    act = w.B * w.h * w.n * w.d * 2
    algo_bytes, flops = 4 * act, 4 * w.B * w.h * w.n * w.d * w.d
    R = max(1, -(-ROTATE_BYTES // algo_bytes))
    sets = [(Q0, K0, V0, torch.empty_like(Q0))] + [
        (Q0.clone(), K0.clone(), V0.clone(), torch.empty_like(Q0)) for _ in range(R - 1)]
    stream = torch.cuda.current_stream(dev)
    step = lambda i: ctx.relu_linear(*sets[i % R][:3], 100.0, 1.0, out=sets[i % R][3], stream=stream)
    ms = timed_steps(step, args.warmup, args.steps, stream, R)
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": f"ReLU linear attention tokens/sec ({w.name} shape)",
        "value": round(w.B * w.n / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "linear", "B": w.B, "h": w.h, "n": w.n, "d": w.d,
                   "cmin": 100.0, "global_batch": w.B, "seq_len": w.n,
                   "parallelism": "single-gpu", "rotating_sets": R},
        "achieved_hbm_gbs": round(gbs, 1),
        "achieved_tflops": round(flops / (ms * 1e-3) / 1e12, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "relu_linear_bf16 (the whole step is this one kernel)",
                     "per_launch": {"algorithmic_bytes": algo_bytes, "algorithmic_flops": flops,
                                    "avg_duration_us": round(ms * 1e3, 3)}},
    }
    ref = copy_reference(algo_bytes, min(args.steps, 200), min(args.warmup, 20))
    ref["frac_of_copy"] = round(gbs / ref["gbs"], 4) if ref["gbs"] > 0 else None
    out["copy_reference"] = ref
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_limits
        reps, t0 = 0, time.perf_counter()
        with threadpool_limits(limits=1):
            while True:
                oracle.relu_linear_attn(x.Q, x.K, x.V)
                reps += 1
                el = time.perf_counter() - t0
                if el >= args.cpu_seconds:
                    break
        out["cpu_baseline"] = {"value": reps * w.B * w.n / el, "unit": "tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{reps} full batch(es) of {w.name} in fp64 numpy, {el:.1f} s wall"}
    return out


# Landmarks per workload for the Nystrom leg: the page's sample sizes are 32 to 64.
NYSTROM_LANDMARKS = {"vit_s16_224": 32, "vit_b16_384": 64, "dense_64x64": 64,
                     "long_16k_bf16": 64}


def bench_nystrom(args, ctx, x, dev) -> dict:
    """Nystrom attention with given landmarks (token 0 plus seeded distinct tokens per batch
    element): one step = gather, landmark maxima, landmark pass, solve, output pass."""
    import numpy as np
    import torch
    from efficient_vision_transformer_amd.inputs import make_landmarks
    w = x.workload
    if w.dtype != "bf16":
        raise SystemExit("Nystrom attention runs in bf16 only")
    s = args.landmarks or NYSTROM_LANDMARKS.get(w.name, 64)
    idx = torch.from_numpy(make_landmarks(w.B, w.n, s, seed=w.seed + 77)).to(dev)
    conv = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    Q0, K0, V0 = conv(x.bits["Q"]), conv(x.bits["K"]), conv(x.bits["V"])
    act = w.B * w.h * w.n * w.d * 2
    # Q, K, V read once and H written once; 2nsd flops for each of Q k^T, q K^T, F3 V, F1 Z
    algo_bytes = 4 * act
    flops = 8 * w.B * w.h * w.n * s * w.d
    R = max(1, -(-ROTATE_BYTES // algo_bytes))
    sets = [(Q0, K0, V0, torch.empty_like(Q0))] + [
        (Q0.clone(), K0.clone(), V0.clone(), torch.empty_like(Q0)) for _ in range(R - 1)]
    stream = torch.cuda.current_stream(dev)
    step = lambda i: ctx.nystrom(*sets[i % R][:3], idx, out=sets[i % R][3], stream=stream)
    ms = timed_steps(step, args.warmup, args.steps, stream, R)
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    out = {
        "metric": f"Nystrom attention tokens/sec ({w.name} shape, s={s} landmarks)",
        "value": round(w.B * w.n / (ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "nystrom", "B": w.B, "h": w.h, "n": w.n, "d": w.d,
                   "landmarks": s, "global_batch": w.B, "seq_len": w.n,
                   "parallelism": "single-gpu", "rotating_sets": R},
        "achieved_hbm_gbs": round(gbs, 1),
        "achieved_tflops": round(flops / (ms * 1e-3) / 1e12, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "the whole step (three launches)",
                     "per_launch": {"algorithmic_bytes": algo_bytes, "algorithmic_flops": flops,
                                    "avg_duration_us": round(ms * 1e3, 3)}},
    }
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_limits
        idx_h = idx.cpu().numpy()
        reps, t0 = 0, time.perf_counter()
        with threadpool_limits(limits=1):
            while True:
                oracle.nystrom_attn(x.Q, x.K, x.V, idx_h)
                reps += 1
                el = time.perf_counter() - t0
                if el >= args.cpu_seconds:
                    break
        out["cpu_baseline"] = {"value": reps * w.B * w.n / el, "unit": "tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{reps} full batch(es) of {w.name} in fp64 numpy, {el:.1f} s wall"}
    return out


def timed_output_parity(x, H) -> dict:
    """The output of the last timed launch against the fp64 oracle on a sample of whole
    slices (first, last and seeded others): normwise max-relative error for fp32 (gate
    1e-5), relative Frobenius error for bf16 (gate 1e-2), over the sample."""
    import numpy as np
    import oracle
    w = x.workload
    k = 4 if w.n > 8192 else 8
    all_s = [(b, j) for b in range(w.B) for j in range(w.h)]
    rng = np.random.default_rng(0)
    pick = sorted({all_s[0], all_s[-1]} | {all_s[int(i)] for i in rng.integers(0, len(all_s), 3 * k)})[:k]
    q = np.stack([x.Q[b, j] for b, j in pick])[None]
    v = np.stack([x.V[b, j] for b, j in pick])[None]
    u = np.stack([x.U[j] for _, j in pick])
    ref = oracle.anchor_attn(q, u, v)[0]
    got = np.stack([H[b, j] for b, j in pick])
    if w.dtype == "fp32":
        metric, gate = "normwise_max_relative", 1e-5
        err = float(np.abs(got - ref).max() / np.abs(ref).max())
    else:
        metric, gate = "relative_frobenius", 1e-2
        err = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    return {"metric": metric, "error": err, "gate": gate, "ok": bool(err <= gate),
            "slices": [list(p) for p in pick], "output": "last timed launch"}


def full_attention_gap(x, H, slices=4) -> dict:
    """Report-only: relative Frobenius gap between softmax(QK^T/sqrt(d))V and H on a few
    slices (inputs exactly as stored)."""
    import numpy as np
    import oracle
    w = x.workload
    num = den = 0.0
    picked = [(b, j) for b in range(w.B) for j in range(w.h)][:slices]
    rows = None
    if w.n > 4096:
        rows = np.random.default_rng(0).choice(w.n, 2048, replace=False)
    for b, j in picked:
        full = oracle.full_attention_slice(x.Q[b, j], x.K[b, j], x.V[b, j], rows)
        mine = H[b, j] if rows is None else H[b, j][rows]
        num += float(((full - mine) ** 2).sum())
        den += float((full ** 2).sum())
    return {"full_attention_rel_frobenius_gap": (num / den) ** 0.5, "slices": len(picked),
            "rows": "all" if rows is None else "2048 sampled"}


def copy_reference(algo_bytes: int, steps: int, warmup: int) -> dict:
    """A plain device copy moving the same bytes (half read, half written) per launch,
    rotated over >= 1 GiB like the benchmark: the bandwidth a single kernel of this size
    reaches on this machine, for context beside the roofline fraction."""
    import torch
    dev = torch.device("cuda:0")
    n = max(1, (algo_bytes // 2) // 4)
    R = max(1, -(-ROTATE_BYTES // (8 * n)))
    pairs = [(torch.ones(n, dtype=torch.int32, device=dev), torch.empty(n, dtype=torch.int32, device=dev))
             for _ in range(R)]
    stream = torch.cuda.current_stream(dev)

    def step(i):
        s, d = pairs[i % R]
        d.copy_(s)
    us = timed_steps(step, warmup, steps, stream, R) * 1e3
    return {"bytes_per_launch": 8 * n, "avg_duration_us": round(us, 3),
            "gbs": round(8 * n / (us * 1e-6) / 1e9, 1)}


def stream_reference(tensor_bytes: int, steps: int, warmup: int) -> dict:
    """The forward's byte pattern with no arithmetic: two tensors of `tensor_bytes` read and
    one written per launch by the library's streaming reference kernel (one 16-byte chunk
    of each buffer per thread), rotated over >= 1 GiB like the benchmark: the practical
    bandwidth floor of one launch moving these bytes on this machine."""
    import ctypes
    import torch
    from efficient_vision_transformer_amd import anchor_attn
    lib = anchor_attn.load_library()
    fn = lib.anchor_attn_stream_reference
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong,
                   ctypes.c_void_p]
    fn.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    nb = tensor_bytes // 16 * 16
    R = max(1, -(-ROTATE_BYTES // (3 * nb)))
    sets = [tuple(torch.full((nb // 2,), 3, dtype=torch.int16, device=dev) for _ in range(3))
            for _ in range(R)]
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    call = lambda i: fn(sets[i % R][0].data_ptr(), sets[i % R][1].data_ptr(),
                        sets[i % R][2].data_ptr(), nb, sp)
    bad = []

    def step(i):
        if call(i) != 0:
            bad.append(i)
    us = timed_steps(step, warmup, steps, stream, R) * 1e3
    if bad:
        raise RuntimeError(f"stream reference launch failed at step {bad[0]}")
    return {"bytes_per_launch": 3 * nb, "avg_duration_us": round(us, 3),
            "gbs": round(3 * nb / (us * 1e-6) / 1e9, 1),
            "kernel": "two buffers read, one written, one 16-byte chunk per thread"}


def main():
    args = parse()
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch
    from efficient_vision_transformer_amd import AnchorAttention
    from efficient_vision_transformer_amd.inputs import HEADLINE, WORKLOADS, make_inputs

    name = args.workload or HEADLINE
    w = WORKLOADS[name]
    if args.head_dim or args.anchors:
        # the workload's value structure at another head dim or anchor count
        from efficient_vision_transformer_amd.inputs import Workload
        over = {}
        if args.head_dim:
            over["d"] = args.head_dim
        if args.anchors:
            over["m"] = args.anchors
        tag = "".join(f"_{k}{v}" for k, v in over.items())
        w = Workload(**{**w.__dict__, **over, "name": f"{w.name}{tag}"})
        name = w.name
    dev = torch.device("cuda:0")
    x = make_inputs(w, with_k=True)
    ctx = AnchorAttention(dev, plan=args.plan)
    plan_desc = ctx.describe(w.B, w.h, w.n, w.m, w.d, w.dtype)
    if args.which == "linear":
        out = bench_linear(args, ctx, x, dev)
        ctx.close()
        print(json.dumps(out), flush=True)
        return
    if args.which == "nystrom":
        out = bench_nystrom(args, ctx, x, dev)
        ctx.close()
        print(json.dumps(out), flush=True)
        return
    if args.which == "block":
        out = bench_block(args, ctx, w, dev)
        ctx.close()
        print(json.dumps(out), flush=True)
        return
    if args.which == "backward":
        out = bench_backward(args, ctx, x, dev, plan_desc)
        ctx.close()
        print(json.dumps(out), flush=True)
        return

    if w.dtype == "bf16":
        up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
        Q0, U, V0 = up(x.bits["Q"]), up(x.bits["U"]), up(x.bits["V"])
    else:
        Q0, U, V0 = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (x.Q, x.U, x.V))
    algo_bytes = w.algorithmic_bytes()
    R = max(1, -(-ROTATE_BYTES // algo_bytes))
    sets = [(Q0, V0, torch.empty_like(V0))] + [
        (Q0.clone(), V0.clone(), torch.empty_like(V0)) for _ in range(R - 1)]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    # Each step is one anchor_attn_forward call through the C ABI with its arguments
    # marshalled once up front (the binding's per-call Python checks stay out of the loop).
    import ctypes
    from efficient_vision_transformer_amd import anchor_attn
    lib = anchor_attn.load_library()
    sv = ctypes.c_void_p(stream.cuda_stream)
    dcode = anchor_attn.BF16 if w.dtype == "bf16" else anchor_attn.FP32
    calls = [(ctx._h, q.data_ptr(), U.data_ptr(), v.data_ptr(), hh.data_ptr(), w.B, w.h, w.n,
              w.m, w.d, dcode, sv) for q, v, hh in sets]
    bad = []

    def step(i):
        rc = lib.anchor_attn_forward(*calls[i % R])
        if rc != 0:
            bad.append(rc)
    ms = timed_steps(step, args.warmup, args.steps, stream, R)
    if bad:
        raise RuntimeError(f"anchor_attn_forward: {anchor_attn.status_string(bad[0])}")
    # the output of the last timed launch, checked against the oracle below (not timed)
    last = (args.warmup + args.steps - 1) % R
    H = sets[last][2].float().cpu().numpy().astype(np.float64)

    tokens = w.B * w.n
    value = tokens / (ms * 1e-3)
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    flops = w.algorithmic_flops()
    peak_tf = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    tflops = flops / (ms * 1e-3) / 1e12
    hbm_bound = (algo_bytes / (HBM_PEAK_GBS * 1e9)) >= (flops / (peak_tf * 1e12))
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(tflops / peak_tf, 4), "traffic": None}
    plan_kind = plan_desc.split(":")[0]
    roof["traffic"] = measured_traffic(name, plan_kind)
    roof["kernel"] = ("fused_bf16 (the whole forward is this one kernel)" if plan_kind == "fused"
                      else f"whole forward ({plan_kind} plan: pass1 + finalize + pass2)")
    roof["per_launch"] = {"algorithmic_bytes": algo_bytes, "algorithmic_flops": flops,
                          "avg_duration_us": round(ms * 1e3, 3)}

    out = {
        "metric": "anchor-attention tokens/sec and achieved HBM GB/s (n=196, m=30, bf16)"
        if name == HEADLINE else f"anchor-attention tokens/sec ({name})",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "h": w.h, "n": w.n, "m": w.m, "d": w.d,
                   "global_batch": w.B, "seq_len": w.n, "parallelism": "single-gpu",
                   "plan": plan_desc, "rotating_sets": R},
        "achieved_hbm_gbs": round(gbs, 1),
        "achieved_tflops": round(tflops, 3),
        "roofline": roof,
    }
    # the other roofline, for workloads near the ridge (the long bf16 one: HBM and MFMA
    # time floors within 20% of each other)
    out["roofline_secondary"] = (
        {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak_tf, "unit": "TFLOP/s",
         "frac": round(tflops / peak_tf, 4)} if hbm_bound else
        {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(gbs / HBM_PEAK_GBS, 4)})
    out["slice_tokens_per_s"] = round(w.B * w.h * w.n / (ms * 1e-3), 1)
    ref = copy_reference(algo_bytes, min(args.steps, 200), min(args.warmup, 20))
    ref["frac_of_copy"] = round(gbs / ref["gbs"], 4) if ref["gbs"] > 0 else None
    out["copy_reference"] = ref
    sref = stream_reference(algo_bytes // 3, min(args.steps, 200), min(args.warmup, 20))
    sref["frac_of_stream"] = round(gbs / sref["gbs"], 4) if sref["gbs"] > 0 else None
    out["stream_reference"] = sref
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    out["diagnostic"] = full_attention_gap(x, H)
    out["parity"] = timed_output_parity(x, H)
    ctx.close()
    print(json.dumps(out), flush=True)
    if not out["parity"]["ok"]:
        sys.exit(1)


if __name__ == "__main__":
    main()
