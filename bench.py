"""Benchmark of the fused conv / GEMM-logsumexp library on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME|baseline] [--cpu-seconds S]
                    [--cpu-seconds-each S] [--cold-steps C]

A step is one call of the fused operation (all of its kernels) on one batch of
synthetic input already resident in HBM. Prints ONE JSON line.

The default (--workload baseline) measures the five baseline configurations in one
process. The line's top-level fields are the headline: the fp32 conv3x3 + bias +
erf-GELU + global average pool on x (64, 16, 224, 224) -> (64, 64). Its "configs"
object holds the same figures for the other four: the tiny conv (2, 3, 16, 16) -> (2, 8),
the fp32 conv + Mish∘Mish with the full (32, 128, 190, 190) output, the bf16 conv +
GELU + pool on (16, 128, 128, 128) -> (16, 256), and the fp32 GEMM (2048 x 4096 x 6144)
+ scale + clamp + row logsumexp + z*mish(z). Each carries the whole-step throughput
(TFLOP/s of the algorithmic contraction), the roofline of its dominant kernel (average
launch time from HIP events recorded on the launch stream during timed steps) against
the spec peak and against the sustained MFMA rate measured on this part at the start of
the run, and a CPU baseline: the fp64 oracle timed on this host's cores on a bounded
sample of the same workload, with the GPU-over-oracle speed-up. --workload NAME measures
one workload only (the form the profiler runs use).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}  # MI355X dense MFMA peaks
HBM_GBPS = 8000.0
DEFAULT_WORKLOAD = "baseline"
HEADLINE = "conv_gelu_pool_f32"
# the other baseline configurations, in their listed order
BASELINE_OTHERS = ["conv_tiny", "conv_mish2_full_f32", "conv_gelu_pool_bf16", "gemm_lse_mish_f32"]
_CSRC = "gemm_activation_reduction_amd/csrc/"
# The sources each measured kernel is compiled from: a traffic summary counts only while
# they are unchanged since its counters were taken.
KERNEL_SOURCES = {
    "conv3x3_fused": [_CSRC + "conv3x3.hip", _CSRC + "conv_common.h", _CSRC + "device_math.h"],
    "conv3x3_wide_bf16": [_CSRC + "conv3x3.hip", _CSRC + "conv_common.h", _CSRC + "device_math.h"],
    "conv_general_fused": [_CSRC + "conv_general.hip", _CSRC + "conv_general_kernel.h", _CSRC + "conv_general_k1.hip",
                           _CSRC + "conv_general_k3.hip", _CSRC + "conv_general_k5.hip", _CSRC + "conv_common.h",
                           _CSRC + "device_math.h"],
    "gemm_lse_partials": [_CSRC + "gemm_lse.hip", _CSRC + "device_math.h"],
    "act_pool_map": [_CSRC + "epilogue.hip", _CSRC + "device_math.h"],
    "act_elementwise": [_CSRC + "epilogue.hip", _CSRC + "device_math.h"],
    "scale_clamp_lse": [_CSRC + "epilogue.hip", _CSRC + "device_math.h"],
    "mfma_rate_probe": [_CSRC + "probe.hip"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def conv_flops(s) -> float:
    K = synth.conv_geometry(s)[0]
    OH, OW = synth.conv_out_size(s)
    return 2.0 * s["N"] * s["Cout"] * OH * OW * s["Cin"] * K * K


def conv_bytes(s) -> float:
    esz = 2 if s["dtype"] == "bf16" else 4
    K = synth.conv_geometry(s)[0]
    OH, OW = synth.conv_out_size(s)
    out = s["N"] * s["Cout"] * (1 if s["pool"] else OH * OW)
    return esz * (s["N"] * s["Cin"] * s["H"] * s["W"] + s["Cout"] * s["Cin"] * K * K) + 4 * s["Cout"] + 4 * out


def gemm_flops(s) -> float:
    return 2.0 * s["M"] * s["K"] * s["N"]


def gemm_bytes(s) -> float:
    esz = 2 if s.get("dtype", "f32") == "bf16" else 4
    return esz * (s["M"] * s["K"] + s["N"] * s["K"]) + 4.0 * (s["N"] + s["M"])


def read_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or None when the
    summary is missing or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_hash") != source_hash(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_pool_sample(spec, x, w, b, n, oc):
    import oracle
    K, S, P = synth.conv_geometry(spec)
    if (K, S, P) == (3, 1, 0):
        return oracle.conv_pool_sample(x, w, b, spec["act"], n, oc)
    return oracle.conv2d_pool_sample(x, w, b, S, P, spec["act"], n, oc)


def oracle_point_sample(spec, x, w, b, n, oc, oh, ow):
    import oracle
    K, S, P = synth.conv_geometry(spec)
    if (K, S, P) == (3, 1, 0):
        return oracle.conv_point_sample(x, w, b, spec["act"], n, oc, oh, ow)
    return oracle.conv2d_point_sample(x, w, b, S, P, spec["act"], n, oc, oh, ow)


def cpu_baseline_conv(spec, x, w, b, got_pool, seconds):
    """fp64 oracle on a bounded sample of (n, oc) maps of the same workload."""
    import oracle
    N, Cout = spec["N"], spec["Cout"]
    order = np.random.default_rng(1).permutation(N * Cout)
    flops_per_map = conv_flops(spec) / (N * Cout)
    done, t0, errs = 0, time.perf_counter(), []
    batch = max(1, oracle.num_threads())
    while done < len(order) and time.perf_counter() - t0 < seconds:
        sel = order[done:done + batch]
        n, oc = sel // Cout, sel % Cout
        ref = oracle_pool_sample(spec, x, w, b, n, oc)
        if got_pool is not None:
            errs.append(np.max(np.abs(got_pool[n, oc] - ref) / (1 + np.abs(ref))))
        done += len(sel)
    el = time.perf_counter() - t0
    return {"value": round(done * flops_per_map / el / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(el, 3),
            "sample": f"{done} of {N * Cout} (n, oc) output maps ({done * flops_per_map / 1e9:.2f} GFLOP, fp64)",
            "sample_max_err": float(max(errs)) if errs else None}


def cpu_baseline_conv_points(spec, x, w, b, out_dev, seconds):
    import oracle
    import torch
    N, Cout = spec["N"], spec["Cout"]
    OH, OW = synth.conv_out_size(spec)
    r = np.random.default_rng(2)
    flops_per_pt = 2.0 * spec["Cin"] * synth.conv_geometry(spec)[0] ** 2
    done, t0, errs, batch = 0, time.perf_counter(), [], 200000
    while time.perf_counter() - t0 < seconds:
        n, oc = r.integers(0, N, batch), r.integers(0, Cout, batch)
        oh, ow = r.integers(0, OH, batch), r.integers(0, OW, batch)
        ref = oracle_point_sample(spec, x, w, b, n, oc, oh, ow)
        idx = [torch.from_numpy(a.astype(np.int64)).to(out_dev.device) for a in (n, oc, oh, ow)]
        got = out_dev[idx[0], idx[1], idx[2], idx[3]].cpu().numpy()
        errs.append(np.max(np.abs(got - ref) / (1 + np.abs(ref))))
        done += batch
    el = time.perf_counter() - t0
    return {"value": round(done * flops_per_pt / el / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(el, 3),
            "sample": f"{done} random output points of {N * Cout * OH * OW} ({done * flops_per_pt / 1e9:.2f} GFLOP, fp64)",
            "sample_max_err": float(max(errs)) if errs else None}


def cpu_baseline_gemm(spec, X, W, b, got, seconds):
    import oracle
    M = spec["M"]
    order = np.random.default_rng(3).permutation(M)
    flops_per_row = gemm_flops(spec) / M
    done, t0, errs = 0, time.perf_counter(), []
    batch = max(1, oracle.num_threads())
    while done < M and time.perf_counter() - t0 < seconds:
        rows = order[done:done + batch]
        ref, _ = oracle.gemm_lse_mish(X, W, b, spec["scale"], spec["cmin"], spec["cmax"], rows=rows)
        errs.append(np.max(np.abs(got[rows] - ref) / (1 + np.abs(ref))))
        done += len(rows)
    el = time.perf_counter() - t0
    return {"value": round(done * flops_per_row / el / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(el, 3),
            "sample": f"{done} of {M} rows ({done * flops_per_row / 1e9:.2f} GFLOP, fp64)",
            "sample_max_err": float(max(errs)) if errs else None}


def calibration_copies(args, torch, dev) -> None:
    """Plain device copies of a known size: the reference a --pmc run scales HBM counters by."""
    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print(f"bench: calibration copies of {args.calib_copy_mb} MiB done", file=sys.stderr, flush=True)


def epilogue_bytes(spec) -> float:
    """Algorithmic bytes of one epilogue-only launch: read the tensor once, write the result."""
    shape = spec["shape"]
    total = int(np.prod(shape))
    if spec["kind"] == "pool":
        return 4.0 * (total + shape[0] * shape[1])
    if spec["kind"] == "elementwise":
        return 8.0 * total
    return 4.0 * (total + shape[0])


def per_step_ms(step, n, torch, stream, flush=None):
    """Per-step times (ms) from torch events on the launch stream. With `flush`, it runs
    before each step's first event (outside the timed interval)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        if flush is not None:
            flush()
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


COLD_FLUSH_MIB = 512


def warm_and_cold(step, steps, cold_steps, torch, dev):
    """(median warm step ms, median cold step ms, cold steps). Cold: each step follows a
    512 MiB read stream over a scratch buffer (a sum), which evicts L2 and the 256 MB MALL
    with clean lines (inputs of up to ~256 MB otherwise stay in the MALL between steps; a
    read + write stream would leave dirty lines whose write-back lands in the timed step)."""
    stream = torch.cuda.current_stream()
    warm = per_step_ms(step, steps, torch, stream)
    if cold_steps <= 0:
        return float(np.median(warm)), None, 0
    flushbuf = torch.zeros(COLD_FLUSH_MIB << 18, dtype=torch.float32, device=dev)
    cold = per_step_ms(step, cold_steps, torch, stream, flush=lambda: flushbuf.sum())
    del flushbuf
    return float(np.median(warm)), float(np.median(cold)), cold_steps


def bench_epilogue(args, name, spec, torch, fc, dev) -> int:
    """HBM-bound epilogue-only kernels: GB/s of algorithmic traffic against 8 TB/s."""
    print(f"bench: generating inputs for {name}", file=sys.stderr, flush=True)
    base = synth.epilogue_base(spec)
    shape = spec["shape"]
    total = int(np.prod(shape))
    reps = total // base.size
    bd = torch.from_numpy(base).to(dev)
    xd = torch.cat([bd.repeat(reps), bd[: total - reps * base.size]]).view(*shape)
    del bd
    kind = spec["kind"]
    if kind == "pool":
        N, C, H, W = shape
        out = torch.empty((N, C), dtype=torch.float32, device=dev)
        nbytes, kernel = epilogue_bytes(spec), "act_pool_map"
        step = lambda: fc.fact_pool(xd, N, C, H, W, spec["act"], out)  # noqa: E731
    elif kind == "elementwise":
        out = torch.empty_like(xd)
        nbytes, kernel = epilogue_bytes(spec), "act_elementwise"
        step = lambda: fc.fact_elementwise(xd, total, spec["act"], out)  # noqa: E731
    else:
        M, N = shape
        out = torch.empty((M, 1), dtype=torch.float32, device=dev)
        nbytes, kernel = epilogue_bytes(spec), "scale_clamp_lse"
        step = lambda: fc.flse_mish_rows(xd, M, N, spec["scale"], spec["cmin"], spec["cmax"], out)  # noqa: E731
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    fc.fconv_profile(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kms, kl = fc.fconv_profile_read(kernel)
    fc.fconv_profile(False)
    med_ms, cold_ms, ncold = warm_and_cold(step, args.steps, args.cold_steps, torch, dev)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kernel_ms = kms / max(1, kl)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    cold_txt = (f", cold-cache median {cold_ms:.4f} ms ({nbytes / (cold_ms * 1e-3) / 1e9:.1f} GB/s)"
                if ncold else "")
    print(f"bench: {ms_per_step:.4f} ms/step, {kernel} {kernel_ms:.4f} ms/launch, {achieved:.1f} GB/s; "
          f"median step {med_ms:.4f} ms{cold_txt}", file=sys.stderr, flush=True)
    calibration_copies(args, torch, dev)
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        r = np.random.default_rng(4)
        t0, done, work = time.perf_counter(), 0, 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            if kind == "pool":
                hw = shape[2] * shape[3]
                p = int(r.integers(0, shape[0] * shape[1]))
                oracle.act_mean(base[synth.epilogue_element_indices(spec, p * hw + np.arange(hw))], spec["act"])
                work += 4 * hw
            elif kind == "elementwise":
                idx = r.integers(0, total, 1 << 20)
                oracle.act_elementwise(base[synth.epilogue_element_indices(spec, idx)], spec["act"])
                work += 8 * len(idx)
            else:
                N = shape[1]
                m = int(r.integers(0, shape[0]))
                y = base[synth.epilogue_element_indices(spec, m * N + np.arange(N))].reshape(1, N)
                oracle.scale_clamp_lse_mish(y, spec["scale"], spec["cmin"], spec["cmax"])
                work += 4 * N
            done += 1
        el = time.perf_counter() - t0
        cpu = {"value": round(work / el / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
               "seconds": round(el, 3), "sample": f"{done} sampled {'maps' if kind == 'pool' else 'batches/rows'}",
               "cpu_model": cpu_model()}
        cpu["speedup"] = round(value / cpu["value"], 1) if cpu["value"] > 0 else None
    line = {
        "metric": f"epilogue-only {name} GB/s", "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "shape": list(shape), "kind": kind},
        "median_ms_per_step": round(med_ms, 5),
        "cold": {"median_ms_per_step": round(cold_ms, 5), "value": round(nbytes / (cold_ms * 1e-3) / 1e9, 1),
                 "unit": "GB/s", "steps": ncold, "flush_mib": COLD_FLUSH_MIB} if ncold else None,
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_GBPS, 4), "traffic": read_traffic(name, kernel),
                     "kernel_ms": round(kernel_ms, 5), "algorithmic_bytes": nbytes},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def measure_sustained_peaks(fc, torch, dev, iters=(2048, 4096)):
    """Sustained dense MFMA rate (TFLOP/s) of this part for fp32 and bf16: the MFMA-only
    probe kernel, timed with HIP events on the launch stream (median of 10 launches after 3
    warm-up launches)."""
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    out = {}
    for dtype, code, it in (("f32", fc.DT_F32, iters[0]), ("bf16", fc.DT_BF16, iters[1])):
        for _ in range(3):
            fc.fconv_mfma_rate_probe(code, it, sink)
        torch.cuda.synchronize()
        fc.fconv_profile(True)
        times = []
        flops = 0.0
        for _ in range(10):
            flops = fc.fconv_mfma_rate_probe(code, it, sink)
            torch.cuda.synchronize()
            ms, n = fc.fconv_profile_read("mfma_rate_probe")
            times.append(ms)
            fc.fconv_profile(True)
        fc.fconv_profile(False)
        med = float(np.median(times))
        out[dtype] = {"value": round(flops / (med * 1e-3) / 1e12, 1), "unit": "TFLOP/s", "kernel_ms": round(med, 4),
                      "spec": PEAK_TFLOPS[dtype], "frac_of_spec": round(flops / (med * 1e-3) / 1e12 / PEAK_TFLOPS[dtype], 4)}
        print(f"bench: sustained {dtype} MFMA rate {out[dtype]['value']} TFLOP/s "
              f"({100 * out[dtype]['frac_of_spec']:.1f} % of {PEAK_TFLOPS[dtype]})", file=sys.stderr, flush=True)
    del sink
    return out


def prepare(name, torch, fc, dev):
    """Inputs resident on the device and a step closure for one conv or GEMM workload."""
    is_conv = name in synth.CONV_WORKLOADS
    spec = synth.CONV_WORKLOADS[name] if is_conv else synth.GEMM_WORKLOADS[name]
    print(f"bench: generating inputs for {name}", file=sys.stderr, flush=True)
    w_ = {"name": name, "spec": spec, "is_conv": is_conv}
    if is_conv:
        x, w, b = synth.conv_inputs(spec)
        bf16 = spec["dtype"] == "bf16"
        to = (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)) if bf16 else \
            (lambda a: torch.from_numpy(a).to(dev))
        xd, wd, bd = to(x), to(w), torch.from_numpy(b).to(dev)
        act = {0: "none", 1: "gelu", 2: "mish2", 3: "gelu_tanh"}[spec["act"]]
        OH, OW = synth.conv_out_size(spec)
        K, S, P = synth.conv_geometry(spec)
        out = torch.empty((spec["N"], spec["Cout"]) if spec["pool"] else
                          (spec["N"], spec["Cout"], OH, OW), dtype=torch.float32, device=dev)

        def step():
            fc.conv2d_act_pool(xd, wd, bd, stride=S, pad=P, act=act, pool=bool(spec["pool"]), out=out)
        # the 3x3 path runs the wide kernel for bf16 with Cout >= 256, also with pad 1 (the
        # library's timer names whichever ran)
        kernels = (["conv3x3_fused", "conv3x3_wide_bf16"] if (K, S, P) == (3, 1, 0) else
                   ["conv3x3_wide_bf16", "conv_general_fused"] if (K, S, P) == (3, 1, 1) else ["conv_general_fused"])
        w_.update(host=(x, w, b), step=step, out=out, flops=conv_flops(spec), nbytes=conv_bytes(spec),
                  kernels=kernels, dtype=spec["dtype"],
                  cfg={"workload": name, "x": [spec["N"], spec["Cin"], spec["H"], spec["W"]], "cout": spec["Cout"],
                       "kernel": f"{K}x{K} stride {S} pad {P}", "act": act, "pool": bool(spec["pool"]),
                       "dtype": spec["dtype"]})
    else:
        X, W, b = synth.gemm_inputs(spec)
        dtype = spec.get("dtype", "f32")
        to = (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)) if dtype == "bf16" else \
            (lambda a: torch.from_numpy(a).to(dev))
        xd, wd, bd = to(X), to(W), torch.from_numpy(b).to(dev)
        out = torch.empty((spec["M"], 1), dtype=torch.float32, device=dev)

        def step():
            fc.gemm_lse_mish(xd, wd, bd, spec["scale"], spec["cmin"], spec["cmax"], out=out)
        w_.update(host=(X, W, b), step=step, out=out, flops=gemm_flops(spec), nbytes=gemm_bytes(spec),
                  kernels=["gemm_lse_partials"], dtype=dtype,
                  cfg={"workload": name, "M": spec["M"], "K": spec["K"], "N": spec["N"], "scale": spec["scale"],
                       "clamp": [spec["cmin"], spec["cmax"]], "dtype": dtype})
    return w_


def time_workload(wl, args, torch, fc, dev, sustained):
    """Warm-up, whole-step timing, per-kernel event timing, warm/cold medians."""
    step, flops, nbytes, dtype = wl["step"], wl["flops"], wl["nbytes"], wl["dtype"]
    print(f"bench: {wl['name']}: warmup {args.warmup}, timing {args.steps} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # timed region 1: the whole step, nothing else on the stream
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # timed region 2: the same steps with every kernel bracketed by HIP events recorded by
    # the library on the launch stream (per-kernel average launch time)
    fc.fconv_profile(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kernel, kms, klaunches = wl["kernels"][0], 0.0, 0
    for k in wl["kernels"]:
        kms, klaunches = fc.fconv_profile_read(k)
        if klaunches:
            kernel = k
            break
    others = {k: fc.fconv_profile_read(k) for k in ("pack_weights", "pool_finalize", "lse_merge_mish")}
    fc.fconv_profile(False)
    if klaunches == 0:
        raise RuntimeError(f"none of the kernels {wl['kernels']} was timed for {wl['name']}")
    # timed regions 3 and 4: per-step events with warm caches (median), then cold caches
    med_ms, cold_ms, ncold = warm_and_cold(step, args.steps, args.cold_steps, torch, dev)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    ev_ms_per_step = ev0.elapsed_time(ev1) / args.steps
    kernel_ms = kms / max(1, klaunches)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]
    sus = sustained.get(dtype, {}).get("value") if sustained else None
    for k, (ms, nl) in others.items():
        if nl:
            print(f"bench: {wl['name']}: {k} {ms / nl * 1e3:.2f} us/launch", file=sys.stderr, flush=True)
    print(f"bench: {wl['name']}: {ms_per_step:.4f} ms/step (events {ev_ms_per_step:.4f}), {kernel} {kernel_ms:.4f} "
          f"ms/launch over {klaunches} launches, {achieved:.2f} TFLOP/s ({100 * achieved / peak:.1f} % of spec"
          + (f", {100 * achieved / sus:.1f} % of sustained" if sus else "") + "), "
          f"{nbytes / (kernel_ms * 1e-3) / 1e9:.1f} GB/s algorithmic; median step {med_ms:.4f} ms"
          + (f", cold-cache median {cold_ms:.4f} ms ({flops / (cold_ms * 1e-3) / 1e12:.2f} TFLOP/s)" if ncold else ""),
          file=sys.stderr, flush=True)
    return {
        "value": round(value, 3), "unit": "TFLOP/s", "ms_per_step": round(ms_per_step, 5), "dtype": dtype,
        "pct_mfma_peak": round(100.0 * value / peak, 2),
        "median_ms_per_step": round(med_ms, 5),
        "cold": {"median_ms_per_step": round(cold_ms, 5), "value": round(flops / (cold_ms * 1e-3) / 1e12, 3),
                 "unit": "TFLOP/s", "steps": ncold, "flush_mib": COLD_FLUSH_MIB} if ncold else None,
        "roofline": {"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "peak_sustained": sus, "frac_sustained": round(achieved / sus, 4) if sus else None,
                     "traffic": read_traffic(wl["name"], kernel),
                     "kernel_ms": round(kernel_ms, 5), "algorithmic_bytes": nbytes,
                     "algorithmic_gbps": round(nbytes / (kernel_ms * 1e-3) / 1e9, 1)},
    }


def cpu_baseline(wl, seconds, gpu_value):
    """The fp64 oracle on a bounded sample of the workload, with the GPU-over-oracle speed-up."""
    if seconds <= 0:
        return None
    print(f"bench: {wl['name']}: CPU oracle baseline (~{seconds:.0f} s)", file=sys.stderr, flush=True)
    spec, out = wl["spec"], wl["out"]
    if wl["is_conv"]:
        x, w, b = wl["host"]
        if spec["pool"]:
            cpu = cpu_baseline_conv(spec, x, w, b, out.cpu().numpy(), seconds)
        else:
            cpu = cpu_baseline_conv_points(spec, x, w, b, out, seconds)
    else:
        X, W, b = wl["host"]
        cpu = cpu_baseline_gemm(spec, X, W, b, out.cpu().numpy()[:, 0], seconds)
    cpu["cpu_model"] = cpu_model()
    cpu["speedup"] = round(gpu_value / cpu["value"], 1) if cpu["value"] > 0 else None
    return cpu


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the shader clock ramps up over the first ~30 back-to-back steps (measured on the 3x3
    # GELU+pool fp32 workload: 0.64 ms falling to 0.55 ms per step), so the default warm-up
    # covers the ramp
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="steps timed after evicting L2 and the MALL (0: skip)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=["baseline"] + sorted(list(synth.CONV_WORKLOADS) + list(synth.GEMM_WORKLOADS)
                                                  + list(synth.EPILOGUE_WORKLOADS)))
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time budget for the headline workload (0: skip every CPU baseline)")
    ap.add_argument("--cpu-seconds-each", type=float, default=5.0,
                    help="oracle time budget for each of the other baseline configurations")
    ap.add_argument("--no-sustained", action="store_true", help="skip the sustained MFMA rate probe")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after timing, run plain device copies of this size (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding the work over several GPUs is not implemented", file=sys.stderr)
        return 2

    import torch
    import gemm_activation_reduction_amd as fc

    dev = torch.device("cuda:0")
    # Everything runs on a stream of its own (default priority), as a serving loop would:
    # on torch's default (null) stream every launch also synchronizes with the other
    # blocking streams, which measured 2-5 % longer per step.
    torch.cuda.set_stream(torch.cuda.Stream(device=dev))
    name = args.workload
    if name in synth.EPILOGUE_WORKLOADS:
        return bench_epilogue(args, name, synth.EPILOGUE_WORKLOADS[name], torch, fc, dev)
    sustained = None if args.no_sustained else measure_sustained_peaks(fc, torch, dev)
    head_name = HEADLINE if name == "baseline" else name
    others = BASELINE_OTHERS if name == "baseline" else []

    wl = prepare(head_name, torch, fc, dev)
    res = time_workload(wl, args, torch, fc, dev, sustained)
    calibration_copies(args, torch, dev)
    cpu = cpu_baseline(wl, args.cpu_seconds, res["value"])
    line = {
        "metric": "fused conv+act+pool TFLOP/s and % MFMA peak; GEMM-LSE TFLOP/s",
        "value": res["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res["dtype"],
        "data": "synthetic",
        "config": wl["cfg"],
        "pct_mfma_peak": res["pct_mfma_peak"],
        "median_ms_per_step": res["median_ms_per_step"],
        "cold": res["cold"],
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
    }
    del wl
    if others:
        configs = {}
        for other in others:
            torch.cuda.empty_cache()
            owl = prepare(other, torch, fc, dev)
            ores = time_workload(owl, args, torch, fc, dev, sustained)
            ores["config"] = owl["cfg"]
            ores["cpu_baseline"] = cpu_baseline(owl, args.cpu_seconds_each if args.cpu_seconds > 0 else 0,
                                                ores["value"])
            configs[other] = ores
            del owl
        line["configs"] = configs
    line["sustained_mfma"] = sustained
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
