#!/usr/bin/env python3
"""Throughput of the Hyena long-convolution chain forward on one MI355X.

One step = one ``hyena_forward`` call (every stage of the order-N chain:
transform, spectral product with feedthrough, inverse, gate) over one batch of
synthetic inputs already resident in HBM.  Filter spectra are computed once
before timing (``hyena_filter_spectrum`` is timed separately and reported).

Prints one JSON line.  ``value`` is token*channels per second of the headline
workload (B=2, N=8192, d=768, order 2, bfloat16 storage, float32 arithmetic);
the other workloads are reported under ``workloads``.  Inputs rotate over
several buffer sets so that the working set of the timed loop exceeds the
256 MB last-level cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME]
                    [--no-cpu-baseline] [--copy-calibration-mb MB]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Hyena FFTConv fwd token·channels/s + HBM GB/s (% peak) at N=8K and 64K"
HBM_PEAK_GBPS = 8000.0
# float32 vector peak with packed-FP32 instructions disabled (all HIP code is
# compiled that way):
# 256 CUs x 4 SIMDs x 16 lanes x 2 flop (FMA) x 2.4 GHz
ALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
# MI355X's published dense fp32 vector figure (with packed FP32), for context
FP32_PUBLISHED_TFLOPS = 157.3
HEADLINE = 2
SECOND = 3  # the metric's second length (64K tokens)
ORDER_OF_RUN = [2, 1, 3, 4, 5]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# accounting (algorithmic bytes and flops per forward)
# ---------------------------------------------------------------------------

def io_bytes(dtype):
    return 2 if dtype == "bf16" else 4


def grid_points(cfg):
    """Tokens per batch row: N (1D), X Y (2D) or X Y Z (3D)."""
    if cfg["kind"] == "1d":
        return cfg["N"]
    if cfg["kind"] == "2d":
        return cfg["X"] * cfg["Y"]
    return cfg["X"] * cfg["Y"] * cfg["Z"]


def spectrum_reals(cfg):
    """Reals of one filter's Hermitian half-spectrum: 2N (1D), 4XY (2D), 8XYZ (3D)."""
    return (2 ** (1 if cfg["kind"] == "1d" else 2 if cfg["kind"] == "2d" else 3)) * grid_points(cfg)


def algorithmic_bytes(cfg, spec_dtype):
    """(2 + order) activations (u, gates, y) + order spectra + order*d
    feedthrough scalars; each read or written once."""
    s_io = io_bytes(cfg["dtype"])
    s_sp = io_bytes(spec_dtype)
    order, d, B = cfg["order"], cfg["d"], cfg["B"]
    tokens = B * grid_points(cfg)
    return (2 + order) * tokens * d * s_io + order * d * spectrum_reals(cfg) * s_sp + order * d * 4


def transform_points(cfg):
    if cfg["kind"] == "1d":
        M = 1
        while M < 2 * cfg["N"]:
            M *= 2
        return M
    return spectrum_reals(cfg)


def algorithmic_flops(cfg):
    """Radix-2 model: 5 M log2 M per complex length-M transform, halved for
    real data; a forward and an inverse per stage; 9 flops per output for the
    spectral product, feedthrough and gate."""
    M = transform_points(cfg)
    tokens = cfg["B"] * grid_points(cfg)
    per_tc = cfg["order"] * (2 * 5 * (M / 2) * math.log2(M) / (M / 2) + 9)
    return per_tc * tokens * cfg["d"]


def kernel_source_sha():
    """Hash of the kernel sources and of the build script (its compiler flags
    shape the generated code as much as the sources do)."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "long_convolution_sequence_rfft_amd")
    for f in sorted(glob.glob(os.path.join(pkg, "csrc", "*"))) + [os.path.join(pkg, "build.py")]:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, kernel):
    """Measured HBM bytes per launch of `kernel` (FETCH_SIZE + WRITE_SIZE,
    each scaled by the plain copy kernel's reading) from the committed
    rocprofv3 counter summary, or None if there is none for this kernel or the
    kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    if not os.path.exists(path):
        return None
    sha = None
    for line in open(path):
        line = line.rstrip("\n")
        if line.startswith("# kernel_source_sha"):
            sha = line.split()[-1]
        if not line or line.startswith("#"):
            continue
        f = line.split("\t")
        if len(f) >= 4 and f[0] == workload and f[1] == kernel:
            if sha != kernel_source_sha():
                return None
            return int(float(f[2]) + float(f[3]))
    return None


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def hold_stream():
    """Enqueue a short spin kernel on the current stream (outside any timed
    region): while it runs the host enqueues the first forwards, so a timed
    region that starts after it holds K forwards running back to back on the
    GPU rather than also the host's latency to its first launch (the
    blocking-kernel method of GPU benchmark harnesses).  The host enqueues a
    forward in less time than the GPU runs one, so the GPU does not wait on it
    later in the region."""
    import torch
    torch.cuda._sleep(1_000_000)


def make_inputs(idx, seed):
    from long_convolution_sequence_rfft_amd import synth
    return synth.make_workload(idx, seed=seed)


def run_workload(idx, steps, warmup, min_rotation_bytes=600 << 20):
    import torch
    from long_convolution_sequence_rfft_amd import hyena, synth
    from long_convolution_sequence_rfft_amd.synth import WORKLOADS, WORKLOAD_NAMES

    cfg = dict(WORKLOADS[idx])
    name = WORKLOAD_NAMES[idx]
    io = hyena.HYENA_F32 if cfg["dtype"] == synth.F32 else hyena.HYENA_BF16
    spec_dtype = io
    dims = {"1d": lambda: (cfg["N"],), "2d": lambda: (cfg["X"], cfg["Y"]),
            "3d": lambda: (cfg["X"], cfg["Y"], cfg["Z"])}[cfg["kind"]]()
    log(f"[bench] {name}: building plan")
    try:
        plan = hyena.Plan(cfg["B"], cfg["d"], cfg["order"], dims, io_dtype=io,
                          spectrum_dtype=spec_dtype)
    except hyena.HyenaError as e:
        log(f"[bench] {name}: skipped ({e})")
        return None
    t0 = time.time()
    inp = make_inputs(idx, seed=idx)
    log(f"[bench] {name}: inputs synthesised in {time.time() - t0:.1f}s")

    def dev(a):
        if cfg["dtype"] == synth.BF16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    h = dev(inp.h)
    D = torch.from_numpy(inp.D).cuda()
    # filter spectrum, timed separately
    try:
        H = plan.spectrum(h)
    except hyena.HyenaError as e:
        log(f"[bench] {name}: skipped ({e})")
        return None
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        plan.spectrum(h, H)
    e1.record()
    torch.cuda.synchronize()
    spectrum_ms = e0.elapsed_time(e1) / 3
    del h
    # spectrum from an implicit filter (sine MLP over positions, K = 8
    # frequencies, width 64): the taps are generated on the device
    implicit_ms = None
    if cfg["kind"] == "1d":
        w = synth.make_implicit(cfg["d"], cfg["order"], K=8, H=64, seed=idx)
        devw = {k: torch.from_numpy(v).cuda() for k, v in w.arrays().items()}
        Hi = plan.spectrum_implicit(omega=w.omega, **devw)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(3):
            plan.spectrum_implicit(omega=w.omega, H=Hi, **devw)
        e1.record()
        torch.cuda.synchronize()
        implicit_ms = e0.elapsed_time(e1) / 3
        del Hi, devw

    bytes_alg = algorithmic_bytes(cfg, "bf16" if spec_dtype == hyena.HYENA_BF16 else "f32")
    nsets = max(1, min(4, int(math.ceil(min_rotation_bytes / bytes_alg))))
    sets = []
    for s in range(nsets):
        u = dev(inp.u)
        gates = [dev(inp.gates[n]) for n in range(cfg["order"])]
        Hs = H if s == 0 else H.clone()
        sets.append((u, gates, Hs, torch.empty_like(u)))
    del inp

    def step(i):
        u, gates, Hs, y = sets[i % nsets]
        plan.forward(u, gates, Hs, D, y)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # Timed region: exactly `steps` forwards between two events on the launch
    # stream (torch's current stream, which the plan launches on).
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    hold_stream()
    start.record()
    h0 = time.perf_counter()
    for i in range(steps):
        step(i)
    stop.record()
    host_us = (time.perf_counter() - h0) * 1e6 / steps  # host time to enqueue one forward
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    # The same `steps` forwards again with every kernel launch bracketed by
    # its own pair of events on that stream (hyena_timing_*): per-kernel
    # launch durations.  The event markers add a few microseconds between
    # launches, so the whole-job time above comes from the clean region.
    # Per-step distribution: the same `steps` forwards with an event between
    # consecutive steps (one marker per step; the whole-job time above stays
    # the clean region's).
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    hold_stream()
    marks[0].record()
    for i in range(steps):
        step(i)
        marks[i + 1].record()
    torch.cuda.synchronize()
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))

    def pct(q):
        # nearest-rank percentile of the per-step times
        return step_ms[min(len(step_ms) - 1, max(0, int(math.ceil(q * len(step_ms))) - 1))]

    hyena.hyena_timing_begin(steps * 64)
    start2, stop2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_stream()
    start2.record()
    for i in range(steps):
        step(i)
    stop2.record()
    torch.cuda.synchronize()
    kernels, dropped = hyena.hyena_timing_end()
    hyena.hyena_timing_release()
    traced_ms = start2.elapsed_time(stop2)
    if dropped:
        log(f"[bench] {name}: {dropped} launches not timed")

    tokens = cfg["B"] * grid_points(cfg)
    tc = tokens * cfg["d"]
    ms = total_ms / steps
    flops = algorithmic_flops(cfg)
    res = {
        "workload": name,
        "path": {1: "LDS1D", 2: "FOURSTEP1D", 3: "ROWCOL2D", 4: "ROWCOL3D"}[plan.path],
        "B": cfg["B"], "d": cfg["d"], "order": cfg["order"],
        "dims": list(dims), "storage": cfg["dtype"],
        "spectrum": "bf16" if spec_dtype == hyena.HYENA_BF16 else "f32",
        "ms_per_step": ms,
        "step_ms_p10": pct(0.10), "step_ms_p50": pct(0.50), "step_ms_p90": pct(0.90),
        "host_enqueue_us_per_step": round(host_us, 1),
        "tc_per_s": tc / (ms * 1e-3),
        "spectrum_ms": spectrum_ms,
        "implicit_spectrum_ms": implicit_ms,
        "rotation_sets": nsets,
        "algorithmic_bytes": bytes_alg,
        "algorithmic_flops": flops,
        "hbm_GBps": bytes_alg / (ms * 1e-3) / 1e9,
        "hbm_frac": bytes_alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "alu_TFLOPs": flops / (ms * 1e-3) / 1e12,
        "alu_frac": flops / (ms * 1e-3) / 1e12 / ALU_PEAK_TFLOPS,
        "traced_ms_per_step": traced_ms / steps,
        "kernels": {k: {"launches_per_forward": v["launches"] / steps,
                        "avg_launch_ms": v["total_ms"] / v["launches"],
                        "ms_per_forward": v["total_ms"] / steps}
                    for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["total_ms"])},
        "cfg": cfg,
    }
    log(f"[bench] {name}: {ms * 1e3:.1f} us/step, {res['tc_per_s'] / 1e9:.1f} G tc/s, "
        f"{res['hbm_GBps']:.0f} GB/s ({100 * res['hbm_frac']:.1f}% HBM), "
        f"{res['alu_TFLOPs']:.1f} TFLOP/s ({100 * res['alu_frac']:.1f}% fp32 VALU)")
    del sets, H
    torch.cuda.empty_cache()
    return res


def kernel_share(cfg, kernel):
    """Algorithmic (flops, bytes) per forward attributed to one kernel.

    Per token*channel and stage the flop model gives 5 log2 M to each of the
    forward and the inverse transform and 9 to the spectral product,
    feedthrough and gate; a multi-pass transform of length M = La * Lb
    splits its 5 log2 M as 5 log2 La (outer pass) + 5 log2 Lb (inner pass),
    and on 3D grids M = P3 P2 P1 as outer, middle and inner passes.
    Bytes: the activations, spectra and feedthrough a kernel consumes or
    produces; staging copies move no algorithmic bytes."""
    tc = cfg["B"] * cfg["d"] * grid_points(cfg)
    s_io = io_bytes(cfg["dtype"])
    s_sp = io_bytes(cfg["dtype"])
    order, d = cfg["order"], cfg["d"]
    spec = order * d * spectrum_reals(cfg) * s_sp + order * d * 4
    act = tc * s_io
    M = transform_points(cfg)
    short = kernel.split("<")[0].replace("hy::", "")
    args = [a.strip() for a in kernel[kernel.index("<") + 1:kernel.rindex(">")].split(",")] \
        if "<" in kernel else []
    if short in ("hyena_lds1d_forward", "hyena_lds1d_real_forward"):
        # the whole chain runs in this one kernel (on staged copies of the
        # activations, which move the same bytes) -- except, for float32
        # storage on the single-channel kernels, the last gate, which the
        # gated stage-out applies
        f, b_ = algorithmic_flops(cfg), algorithmic_bytes(cfg, cfg["dtype"])
        if short == "hyena_lds1d_real_forward" and len(args) > 1 and args[1] == "float":
            return f - tc, b_ - act
        return f, b_
    if short == "hyena_stage" and len(args) > 2 and args[2] == "true":
        # float32 stage-out with the chain's last gate: one multiply and the
        # gate read per token*channel
        return float(tc), act
    if short == "hyena_mp_outer":
        la, mode = int(args[0]), int(args[2])
        lg = math.log2(la)
        table = {0: (5 * lg, act),                                   # u -> forward outer
                 1: ((order - 1) * (10 * lg + 1), (order - 1) * act),  # inverse, gate, forward
                 2: (5 * lg + 1, 2 * act)}                            # inverse, gate -> y
        if mode in table:
            f, b = table[mode]
            return f * tc, b
        return 0.0, 0.0
    if short == "hyena_mp_mid":
        # 3D: the transforms along y, one forward and one inverse per stage
        ly, mode = int(args[0]), int(args[1])
        return order * 5 * math.log2(ly) * tc, 0.0
    if short == "hyena_mp_inner":
        lb, mode = int(args[0]), int(args[2])
        if mode == 0:
            return order * (10 * math.log2(lb) + 8) * tc, spec
        return 0.0, 0.0
    return 0.0, 0.0


def roofline_of(res):
    """Roofline of the workload's dominant kernel (largest time per forward):
    its algorithmic flops or bytes per launch over its average launch duration,
    both from the timed region."""
    cfg = res["cfg"]
    name, k = next(iter(res["kernels"].items()))
    flops, nbytes = kernel_share(cfg, name)
    per_launch_f = flops / k["launches_per_forward"]
    per_launch_b = nbytes / k["launches_per_forward"]
    sec = k["avg_launch_ms"] * 1e-3
    traffic = load_traffic(res["workload"], name)
    t_hbm = per_launch_b / (HBM_PEAK_GBPS * 1e9)
    t_alu = per_launch_f / (ALU_PEAK_TFLOPS * 1e12)
    out = {"kernel": name, "launches_per_forward": k["launches_per_forward"],
           "avg_launch_us": round(k["avg_launch_ms"] * 1e3, 2)}
    a_alu = per_launch_f / sec / 1e12
    a_hbm = per_launch_b / sec / 1e9
    if t_alu >= t_hbm:
        out.update({"bound": "alu", "achieved": round(a_alu, 3), "peak": round(ALU_PEAK_TFLOPS, 2),
                    "unit": "TFLOP/s", "frac": round(a_alu / ALU_PEAK_TFLOPS, 4),
                    "peak_kind": "fp32 VALU without packed-FP32 instructions "
                                 "(256 CU x 4 SIMD x 16 lanes x 2 flop x 2.4 GHz)",
                    "frac_of_published_fp32": round(a_alu / FP32_PUBLISHED_TFLOPS, 4)})
    else:
        out.update({"bound": "hbm", "achieved": round(a_hbm, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(a_hbm / HBM_PEAK_GBPS, 4)})
    # the metric's own roofline (HBM), whatever bounds the kernel
    out["hbm"] = {"achieved": round(a_hbm, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                  "frac": round(a_hbm / HBM_PEAK_GBPS, 4)}
    out["alu"] = {"achieved": round(a_alu, 3), "peak": round(ALU_PEAK_TFLOPS, 2),
                  "unit": "TFLOP/s", "frac": round(a_alu / ALU_PEAK_TFLOPS, 4)}
    out["algorithmic_per_launch"] = {"flops": per_launch_f, "bytes": per_launch_b}
    out["traffic"] = traffic
    # Summed launch durations per forward over the wall time of the same
    # (event-bracketed) forwards.  Above 1, launches overlap: chains of
    # several chunks run them on two streams, and each launch's duration then
    # includes the time it shares the GPU with the other stream's, so the
    # fractions above understate the kernel's own rate.
    if res.get("traced_ms_per_step"):
        busy = sum(v["ms_per_forward"] for v in res["kernels"].values())
        out["kernel_time_over_step_time"] = round(busy / res["traced_ms_per_step"], 3)
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def cpu_baseline(idx, max_channels, min_seconds=10.0, max_seconds=30.0):
    """The float64 oracle on the workload's first `max_channels` channels (all
    tokens), repeated until about `min_seconds` of wall time have passed."""
    import oracle
    from long_convolution_sequence_rfft_amd.synth import WORKLOADS, WORKLOAD_NAMES
    cfg = WORKLOADS[idx]
    inp = make_inputs(idx, seed=idx)
    ch = np.arange(min(max_channels, cfg["d"]))
    u, g, h, D = inp.f64()
    u, g, D = np.ascontiguousarray(u[..., ch]), np.ascontiguousarray(g[..., ch]), D[:, ch]
    h = np.ascontiguousarray(h[:, ch])
    method = oracle.DIRECT if (cfg["kind"] == "1d" and cfg["N"] <= 2048) else oracle.FFT
    tokens = cfg["B"] * grid_points(cfg)
    reps = 0
    t0 = time.time()
    while True:
        {"1d": oracle.hyena1d, "2d": oracle.hyena2d, "3d": oracle.hyena3d}[cfg["kind"]](
            u, g, h, D, method)
        reps += 1
        dt = time.time() - t0
        if dt >= min_seconds or dt * (reps + 1) / reps > max_seconds:
            break
    tc = tokens * len(ch) * reps
    return {"value": tc / dt, "unit": "token·channels/s", "cores": oracle.num_threads(),
            "kind": "oracle", "workload": WORKLOAD_NAMES[idx], **host_info(),
            "sample": f"{len(ch)} of {cfg['d']} channels, all {tokens} tokens per channel, "
                      f"{'direct Toeplitz sum' if method == oracle.DIRECT else 'radix-2 FFT'}"
                      f" route, float64, {reps} repetitions; {dt:.1f} s wall"}


def host_info():
    """The host the oracle ran on: CPUs this process may use, the CPU model,
    and the OpenMP thread setting."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count()
    return {"host_cpus_available": affinity, "cpu_model": model,
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


# ---------------------------------------------------------------------------

def copy_rate(mib=1024, reps=10):
    """Device-to-device copy rate of a plain contiguous copy (torch), GB/s of
    bytes read plus written: the practical streaming rate, as context."""
    import torch
    n = (mib << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_moved": 2 * (mib << 20), "GBps": round(2 * (mib << 20) / (ms * 1e-3) / 1e9, 1),
            "kind": "torch copy_, float32, read + write"}


def copy_calibration(mb):
    """A plain elementwise kernel of known traffic (reads mb MiB, writes mb MiB;
    torch's negation kernel, a name no other kernel in the run carries), so
    counter runs can scale FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch
    n = (mb << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {mb} MiB read + {mb} MiB written")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", type=str, default=None, help="run only this workload name")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-channels", type=int, default=768)
    ap.add_argument("--copy-calibration-mb", type=int, default=0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "bench.py runs on one GPU only; the path shards over "
                          "channels with no communication between GPUs, but no multi-GPU "
                          "run is provided", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch
    from long_convolution_sequence_rfft_amd.synth import WORKLOAD_NAMES
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb)

    results = {}
    for idx in ORDER_OF_RUN:
        if args.only and WORKLOAD_NAMES[idx] != args.only and str(idx) != args.only:
            continue
        r = run_workload(idx, args.steps, args.warmup)
        if r is not None:
            results[idx] = r

    head_idx = HEADLINE if HEADLINE in results else (next(iter(results)) if results else None)
    if head_idx is None:
        print(json.dumps({"error": "no workload ran"}), flush=True)
        sys.exit(1)
    head = results[head_idx]

    cpu = None
    cpu_64k = None
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle) ...")
        cpu = cpu_baseline(head_idx, args.cpu_channels)
        log(f"[bench] oracle: {cpu['value'] / 1e6:.2f} M tc/s on {cpu['cores']} threads")
        if SECOND in results and SECOND != head_idx:
            # the metric names both lengths: the oracle at 64K tokens too
            cpu_64k = cpu_baseline(SECOND, args.cpu_channels)
            log(f"[bench] oracle at 64K: {cpu_64k['value'] / 1e6:.2f} M tc/s")
    copy = copy_rate()
    log(f"[bench] plain copy: {copy['GBps']:.0f} GB/s")

    workloads = {}
    for idx, r in results.items():
        w = {k: v for k, v in r.items() if k != "cfg"}
        w["roofline"] = roofline_of(r)
        workloads[r["workload"]] = w
    line = {
        "metric": METRIC,
        "value": head["tc_per_s"],
        "unit": "token·channels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage_dtype": head["storage"],
        "data": "synthetic (seeded; damped-sinusoid filters, N(0,1) activations)",
        "config": {"workload": head["workload"], "B": head["B"], "dims": head["dims"],
                   "d": head["d"], "order": head["order"], "storage": head["storage"],
                   "spectrum": head["spectrum"], "path": head["path"],
                   "parallelism": "single GPU"},
        "hbm": {"achieved": round(head["hbm_GBps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(head["hbm_frac"], 4)},
        "step_ms": {"p10": head["step_ms_p10"], "p50": head["step_ms_p50"],
                    "p90": head["step_ms_p90"]},
        "roofline": roofline_of(head),
        "roofline_hbm": roofline_of(head)["hbm"],
        "cpu_baseline": cpu,
        "cpu_baseline_64k": cpu_64k,
        "plain_copy": copy,
        "second_length": ({"workload": results[SECOND]["workload"],
                           "value": results[SECOND]["tc_per_s"],
                           "ms_per_step": results[SECOND]["ms_per_step"],
                           "hbm_frac": round(results[SECOND]["hbm_frac"], 4),
                           "roofline": roofline_of(results[SECOND])}
                          if SECOND in results else None),
        "workloads": workloads,
        "kernel_source_sha": kernel_source_sha(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
