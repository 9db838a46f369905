"""Throughput benchmark of the fused transform + dynamic quantization operator on one GPU.

A step is one fq_run over a whole workload: every slice x_k of x[K, M, N] is transformed
(P1 . x_k . P2) and quantized, codes and scales written to HBM.  The headline workload is
the largest one, K=32768, M=N=256 (hidden 65536), bf16 activations N(0,1) with 1% of the
channels x20, random orthogonal P1/P2, per-token int4 (2 codes a byte), clipRatio 0.95 --
bound by the bf16 matrix cores.  The other four workloads (K=64 M=N=16; K=8192 M=N=64
per-token INT32 clip 0.9; K=16384 M=64 N=128 fp16 MXFP4; K=16384 M=N=256 left-only MXFP4
V2) are measured the same way and reported as sub-records of the same line.  Inputs are
resident in HBM before the timed region; for the small workloads several input/output sets
are rotated so the 256 MB last-level cache cannot serve the reads.

Per workload: `steps` launches back to back on one stream, bracketed by HIP events on that
stream (the step time), then `steps` more launches each bracketed by its own event pair (the
launch-duration distribution: mean, median, p10, p90; an event pair around every launch
adds a few microseconds to the short ones).  The roofline record divides the algorithmic
bytes (HBM-bound workloads) or flops (the 256 x 256 two-sided one) by the step time of the
back-to-back launches, which includes the gaps between them.  HBM traffic, MFMA busy and the shader clock come from the committed
rocprofv3 summaries under profiles/ when their kernel source hash matches the build.  The
CPU baseline is the oracle on the host cores on a bounded sample of the workload; the same
leg compares a sample of the timed run's outputs with the oracle (the bit-exact rule with
its tie tolerance) and reports the result.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16/fp16 MFMA, TFLOP/s
MFMA_FP4_PEAK_TFS = 10100.0    # MI355X dense fp4 MFMA, TFLOP/s
MFMA_INT8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, TOP/s


def algorithmic_bytes(w, K=None) -> int:
    """Bytes one launch must move: read x, P1, P2 once; write codes (0.5 B/elem, 1 B/elem for
    the 8-bit modes) and scales."""
    K = w.K if K is None else K
    MN = w.M * w.N
    codes = K * MN if w.mode in ("int8", "e4m3", "e5m2") else K * MN // 2
    b = 2 * K * MN + 2 * w.M * w.M + (2 * w.N * w.N if w.two_sided else 0) + codes
    if w.mode == "fp4":
        b += K * 2 * (-(-MN // 64))
    else:
        b += 4 * K
    return b


def dequant_bytes(w, K=None) -> int:
    """Bytes one dequantization launch must move: read the codes (0.5 B/elem, 1 B/elem for
    the 8-bit modes) and scales, write the values (2 B/elem)."""
    K = w.K if K is None else K
    MN = w.M * w.N
    codes = K * MN if w.mode in ("int8", "e4m3", "e5m2") else K * MN // 2
    b = codes + 2 * K * MN
    b += K * 2 * (-(-MN // 64)) if w.mode == "fp4" else 4 * K
    return b


def algorithmic_flops(w, K=None) -> int:
    K = w.K if K is None else K
    f = 2 * w.M * w.M * w.N
    if w.two_sided:
        f += 2 * w.M * w.N * w.N
    return K * f


# the source file of each profiled kernel
KERNEL_SOURCES = {"generic": "fq_generic.hip", "mfma_small": "fq_mfma_small.hip", "mfma_wide1": "fq_mfma_wide.hip",
                  "mfma_wide2": "fq_mfma_wide.hip", "mfma_wide2t": "fq_mfma_wide2t.hip",
                  "mfma_wide1s": "fq_mfma_wide1s.hip", "dequant": "fq_dequant.hip",
                  "mx_gemm_kernel": "fq_mx_gemm.hip", "int4_gemm_kernel": "fq_int4_gemm.hip"}


def kernel_source_hash(kernel: str | None = None) -> str:
    """Hash of a kernel's device code: its HIP source and every device header (not the host
    code); all HIP sources when no kernel is named.  The profile summaries record it beside
    their counters."""
    import glob
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "flatquant_transform_quant_amd", "csrc")
    hips = ([os.path.join(csrc, KERNEL_SOURCES[kernel])] if kernel in KERNEL_SOURCES
            else glob.glob(os.path.join(csrc, "*.hip")))
    hips = [f for f in hips if os.path.exists(f)]  # no sources beside the library: no match
    for f in sorted(hips + glob.glob(os.path.join(csrc, "*.h"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profile_info(w, op="quantize", kernel: str | None = None):
    """The machine-readable record of the committed rocprofv3 summary of this workload's
    kernel (profiles/<kernel>_<workload>.md; `kernel`, when given, names the one launched),
    or None when there is none or the kernel's device code has changed since it was taken."""
    import glob

    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{w.name}.md"))):
        if os.path.basename(f).startswith("dequant_") != (op == "dequant"):
            continue
        with open(f, encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("machine-readable:"):
                    info = json.loads(line.split(":", 1)[1])
                    # (a GEMM summary's name ends with the workload its A came from; it has no
                    # workload of its own)
                    if kernel is not None and info.get("kernel") != kernel:
                        continue
                    if info.get("workload") == w.name and info.get("source_hash") == kernel_source_hash(info.get("kernel")):
                        return info
    return None


def profiled_traffic(w, op="quantize"):
    """HBM bytes per launch from the committed counter summary (FETCH_SIZE and WRITE_SIZE,
    each scaled against a copy kernel of known size), or None."""
    info = profile_info(w, op)
    return info.get("traffic_bytes_per_dispatch") if info else None


def profiled_gemm_traffic(kernel: str, product: str):
    """Bytes beyond L2 per launch of a GEMM (2 x FETCH_SIZE + WRITE_SIZE) from its committed
    profile summary for this T x O x H product, or None (no summary, or the kernel changed)."""
    import glob

    for f in glob.glob(os.path.join(ROOT, "profiles", f"{kernel.replace('_kernel', '')}_*.md")):
        with open(f, encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("machine-readable:"):
                    info = json.loads(line.split(":", 1)[1])
                    if info.get("product") == product and info.get("source_hash") == kernel_source_hash(kernel):
                        return info.get("traffic_bytes_per_dispatch")
    return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x_host, p1, p2, budget_s: float = 10.0, gpu_slices=None):
    """The oracle (codes and scales only) on the host cores, on a bounded sample of
    slices of the same workload, scaled to Gelem/s.  With `gpu_slices` (a function giving
    the timed run's packed codes and scales for a list of slice indices) the same leg also
    checks a sample of the timed outputs against the oracle."""
    import oracle

    threads = max(1, min(os.cpu_count() or 1, 64))
    n0 = min(w.K, max(threads, 16 if w.M * w.N > 16384 else 64))
    t = time.perf_counter()
    oracle.run_codes_only(x_host[:n0], p1, p2, w.dtype, w.mode, w.clip_ratio, w.dst_type_max, threads)
    dt0 = time.perf_counter() - t
    n = min(w.K, max(n0, int(n0 * budget_s / max(dt0, 1e-6))))
    if n > n0:
        t = time.perf_counter()
        oracle.run_codes_only(x_host[:n], p1, p2, w.dtype, w.mode, w.clip_ratio, w.dst_type_max, threads)
        dt = time.perf_counter() - t
    else:
        n, dt = n0, dt0
    # the whole workload takes less than the budget: repeat passes over it
    reps = 1
    if n == w.K and dt < 0.5 * budget_s:
        reps = max(1, min(200, int(budget_s / max(dt, 1e-6))))
        t = time.perf_counter()
        for _ in range(reps):
            oracle.run_codes_only(x_host, p1, p2, w.dtype, w.mode, w.clip_ratio, w.dst_type_max, threads)
        dt = time.perf_counter() - t
    elems = reps * n * w.M * w.N
    what = f"{reps} passes over all {w.K} slices" if reps > 1 else f"first {n} of {w.K} slices"
    rec = {"value": elems / dt / 1e9, "unit": "Gelem/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{what} ({elems} elements), {dt:.2f} s wall on {threads} threads"}
    if gpu_slices is not None:
        import numpy as np

        from oracle.compare import compare

        rng = np.random.default_rng(0)
        count = 8 if w.M * w.N > 16384 else 128
        idx = sorted({0, w.K // 2, w.K - 1, *rng.integers(0, w.K, count).tolist()})
        packed, scale = gpu_slices(idx)
        orc = oracle.run(x_host[idx], p1, p2, w.dtype, w.mode, w.clip_ratio, w.dst_type_max, nthreads=threads)
        rep = compare(orc, packed, scale)
        rec["parity_of_timed_outputs"] = {
            "slices": len(idx), "elements": rep["elements"], "ok": rep["ok"], "mismatch": rep["mismatch"],
            "mismatch_cap": rep["mismatch_cap"], "outside_tie_window": rep["mismatch_out_of_window"],
            "outside_tie_window_cap": rep["out_of_window_cap"], "scale_ties": rep.get("scale_ties"),
            "alt_groups": rep.get("alt_groups"), "errors": rep["errors"][:3]}
    return rec


def cpu_baseline_dequant(w, packed, scale, budget_s: float = 10.0):
    """The oracle's dequantization (single thread) on the host, over as many passes of the
    workload's codes as fit the budget, scaled to Gelem/s."""
    import oracle

    t = time.perf_counter()
    oracle.dequant(packed, scale, w.M, w.N, w.dtype, w.mode)
    dt0 = time.perf_counter() - t
    reps = max(1, min(50, int(budget_s / max(dt0, 1e-6))))
    t = time.perf_counter()
    for _ in range(reps):
        oracle.dequant(packed, scale, w.M, w.N, w.dtype, w.mode)
    dt = time.perf_counter() - t
    elems = reps * w.K * w.M * w.N
    return {"value": elems / dt / 1e9, "unit": "Gelem/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} passes over all {w.K} slices ({elems} elements), {dt:.2f} s wall on 1 thread"}


def percentile_summary(ms):
    import numpy as np

    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"mean": round(float(a.mean()), 3), "median": round(float(np.median(a)), 3),
            "p10": round(float(np.percentile(a, 10)), 3), "p90": round(float(np.percentile(a, 90)), 3),
            "unit": "us"}


def time_launches(step, steps, warmup, stream):
    """`steps` calls of step(i) back to back on `stream` bracketed by one event pair (the
    step time), then `steps` more, each bracketed by its own pair (the launch durations)."""
    import torch

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return total_ms, [a.elapsed_time(b) for a, b in ev]


def launch_floor(stream, steps):
    """Duration of a minimal kernel (a one-element add) launched the same way: the fixed cost
    every launch pays."""
    import torch

    t = torch.zeros(1, device=torch.device("cuda:0"))

    def step(i):
        with torch.cuda.stream(stream):
            t.add_(1.0)

    total, each = time_launches(step, steps, 10, stream)
    return {"what": "one-element torch add on the same stream", "step_us": round(total / steps * 1e3, 3),
            "launch_us": percentile_summary(each)}


def copy_reference(nbytes, nsets, stream, steps, dev):
    """A torch device copy moving the same bytes as one launch (half read, half written),
    over as many rotating buffer sets: what plain streaming reaches at this transfer size."""
    import torch

    half = max(1, nbytes // 2)
    bufs = [(torch.empty(half, dtype=torch.uint8, device=dev), torch.empty(half, dtype=torch.uint8, device=dev))
            for _ in range(nsets)]

    def step(i):
        src, dst = bufs[i % nsets]
        with torch.cuda.stream(stream):
            dst.copy_(src)

    total, each = time_launches(step, steps, 5, stream)
    lat = percentile_summary(each)
    step_us = total / steps * 1e3
    del bufs
    torch.cuda.empty_cache()
    return {"what": "torch copy of the same bytes (half read, half written), rotating sets as above",
            "bytes": 2 * half, "step_us": round(step_us, 3), "frac": round(2 * half / (step_us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "launch_us": lat}


def measure_workload(key, args, dev):
    """One workload: inputs resident, timed launches, roofline, CPU baseline + parity."""
    import numpy as np
    import torch

    import flatquant_transform_quant_amd as fq
    import synth

    w = synth.WORKLOADS[key]
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to(dev)

    print(f"[bench] {key}: generating K={w.K} M={w.M} N={w.N}", file=sys.stderr, flush=True)
    x_host, p1, p2 = synth.make_inputs(w)
    # rotate input/output sets so one lap touches > 2x the 256 MB last-level cache
    per_set = algorithmic_bytes(w)
    nsets = int(max(1, min(8, -(-(600 * 2 ** 20) // per_set))))
    xs = [to_dev(x_host)]
    for _ in range(1, nsets):
        xs.append(xs[0].clone())  # distinct buffers with the same values
    p1d = to_dev(p1)
    p2d = to_dev(p2) if p2 is not None else None
    outs = [fq.empty_outputs(w.K, w.M, w.N, w.mode, dev) for _ in range(nsets)]
    execs = [fq.Executor(xs[i], p1d, p2d, outs[i][0], outs[i][1], w.mode, w.clip_ratio,
                         w.dst_type_max, kernel=args.kernel) for i in range(nsets)]
    kernel_id = execs[0].kernel
    stream = torch.cuda.Stream(dev)  # the kernels' stream; every event is recorded on it
    torch.cuda.synchronize()
    total_ms, each_ms = time_launches(lambda i: execs[i % nsets].run(stream), args.steps, args.warmup, stream)
    ms_per_step = total_ms / args.steps
    lat = percentile_summary(each_ms)
    mean_s = ms_per_step / 1e3  # back-to-back launches: the kernel time plus the gaps
    elems = w.K * w.M * w.N
    bytes_ = algorithmic_bytes(w)
    flops = algorithmic_flops(w)
    gbs = bytes_ / mean_s / 1e9
    tfs = flops / mean_s / 1e12
    hbm_frac = gbs / HBM_PEAK_GBS
    mfma_frac = tfs / MFMA_BF16_PEAK_TFS
    bound = "hbm" if bytes_ / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFS * 1e12) else "mfma"
    kname = {1: "generic_kernel", 2: "mfma_small_kernel", 3: "mfma_wide_kernel", 4: "mfma_wide2t_kernel",
             5: "mfma_wide1s_kernel"}.get(kernel_id)
    # the summaries name a kernel by its source family; the two forms of mfma_wide_kernel by side count
    short = {"mfma_wide_kernel": "mfma_wide2" if w.two_sided else "mfma_wide1"}.get(kname, (kname or "")[:-len("_kernel")])
    info = profile_info(w, kernel=short or None)
    roof = ({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(hbm_frac, 4)}
            if bound == "hbm" else
            {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
             "frac": round(mfma_frac, 4)})
    roof["traffic"] = info.get("traffic_bytes_per_dispatch") if info else None
    roof["kernel"] = kname
    roof["avg_launch_us"] = round(ms_per_step * 1e3, 3)
    roof["algorithmic_bytes"] = bytes_
    roof["algorithmic_flops"] = flops
    roof["other_frac"] = round(mfma_frac if bound == "hbm" else hbm_frac, 4)
    if info:
        roof["profile"] = {"avg_us": round(info["avg_ns"] / 1e3, 3), "mfma_busy": info.get("mfma_busy"),
                           "shader_clock_ghz": info.get("clock_ghz_est"), "source_hash": info["source_hash"]}
    rec = {"workload": w.name, "K": w.K, "M": w.M, "N": w.N, "dtype": w.dtype, "mode": w.mode,
           "clip_ratio": w.clip_ratio, "dst_type_max": w.dst_type_max, "two_sided": w.two_sided,
           "buffer_sets": nsets, "value": round(elems * args.steps / (total_ms / 1e3) / 1e9, 2),
           "unit": "Gelem/s", "ms_per_step": round(ms_per_step, 5), "launch_us": lat, "roofline": roof}
    if w.K * w.M * w.N <= 2 ** 16:
        rec["launch_floor"] = launch_floor(stream, args.steps)
    if bound == "hbm":
        rec["copy_reference"] = copy_reference(bytes_, nsets, stream, args.steps, dev)
    for e in execs:
        e.destroy()
    out0, sc0 = outs[(args.steps - 1) % nsets]  # the last timed launch's outputs

    def gpu_slices(idx):
        t = torch.as_tensor(idx, device=dev)
        packed = out0.contiguous().view(torch.uint8).reshape(w.K, -1)[t].cpu().numpy()
        sc = sc0.contiguous()
        scale = (sc.view(torch.uint8).reshape(w.K, -1)[t] if w.mode == "fp4" else sc[t]).cpu().numpy()
        return packed, scale

    rec["cpu_baseline"] = (None if args.no_cpu else
                           cpu_baseline(w, x_host, p1, p2, args.cpu_budget, gpu_slices=gpu_slices))
    del xs, outs, execs, out0, sc0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


HEADLINE = "c4"
SUB_RECORDS = ("c1", "c2", "c3", "c5")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="all",
                    help="all (the headline c4 with c1, c2, c3, c5 as sub-records) or one workload key")
    ap.add_argument("--kernel", type=int, default=0, help="0 auto, 1 generic, 2 mfma-small, 3 mfma-wide, 4 mfma-wide pipelined (256x256 two-sided per-token), 5 mfma-wide streaming (256x256 left-only per-group)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline (and its parity check)")
    ap.add_argument("--cpu-budget", type=float, default=8.0)
    ap.add_argument("--op", default="quantize", choices=["quantize", "dequant", "mxgemm", "i4gemm"],
                    help="quantize (the fused operator, default), dequant (codes + scales -> values), "
                         "mxgemm / i4gemm (the GEMMs consuming a workload's output)")
    ap.add_argument("--gemm-out", type=int, default=8192, help="mxgemm / i4gemm: output features O")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this operator shards over K with no communication, and "
              "the benchmark runs and reports a single MI355X only (--gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.op != "quantize":
        key = HEADLINE if args.config == "all" else args.config
        w = synth.WORKLOADS[key]
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float16

        def to_dev(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to(dev)

        x_host, p1, p2 = synth.make_inputs(w)
        if args.op == "dequant":
            return bench_dequant(args, w, x_host, p1, p2, to_dev, dev, tdt)
        if args.op == "mxgemm":
            return bench_mx_gemm(args, w, x_host, p1, p2, to_dev, dev)
        return bench_int4_gemm(args, w, x_host, p1, p2, to_dev, dev)

    keys = [HEADLINE, *SUB_RECORDS] if args.config == "all" else [args.config]
    recs = [measure_workload(k, args, dev) for k in keys]
    head = recs[0]
    line = {
        "metric": "Gelem/s quantized (x[K,M,N] elems) + % of HBM/MFMA roofline, 1 MI355X",
        "value": head["value"],
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": {"workload": head["workload"], "K": head["K"], "M": head["M"], "N": head["N"],
                   "mode": head["mode"], "clip_ratio": head["clip_ratio"], "dst_type_max": head["dst_type_max"],
                   "two_sided": head["two_sided"], "buffer_sets": head["buffer_sets"], "parallelism": "none"},
        "launch_us": head["launch_us"],
        "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "sub_records": recs[1:],
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_dequant(args, w, x_host, p1, p2, to_dev, dev, tdt):
    """Times fq_dequant on the codes and scales the quantizer makes for the workload."""
    import torch

    import flatquant_transform_quant_amd as fq

    per_set = dequant_bytes(w)
    nsets = int(max(1, min(8, -(-(600 * 2 ** 20) // per_set))))
    x = to_dev(x_host)
    p1d = to_dev(p1)
    p2d = to_dev(p2) if p2 is not None else None
    codes = [fq.empty_outputs(w.K, w.M, w.N, w.mode, dev) for _ in range(nsets)]
    for out, sc in codes:
        fq.quantize(x, p1d, p2d, out, sc, w.mode, w.clip_ratio, w.dst_type_max)
    del x
    vals = [torch.empty((w.K, w.M, w.N), dtype=tdt, device=dev) for _ in range(nsets)]
    stream = torch.cuda.Stream(dev)
    torch.cuda.synchronize()

    def step(i):
        out, sc = codes[i % nsets]
        fq.dequantize(out, sc, w.mode, w.M, w.N, tdt, out=vals[i % nsets], stream=stream)

    for i in range(args.warmup):
        step(i)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms = total_ms / args.steps  # one launch per step, back to back on `stream`
    elems = w.K * w.M * w.N
    bytes_ = dequant_bytes(w)
    gbs = bytes_ / (ms / 1e3) / 1e9
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(w, "dequant"),
            "kernel": (("dequant8_kernel" if (w.M * w.N) % 8 == 0 else "dequant8_each_kernel")
                       if w.mode in ("int8", "e4m3", "e5m2") else
                       ("dequant32_kernel" if (w.M * w.N) % 32 == 0 else "dequant_bytes_kernel")),
            "avg_launch_us": round(ms * 1e3, 3), "algorithmic_bytes": bytes_}
    cpu = None
    if not args.no_cpu:
        import numpy as np

        out, sc = codes[0]
        packed = out.contiguous().view(torch.uint8).reshape(w.K, -1).cpu().numpy()
        scale = (sc.contiguous().view(torch.uint8).reshape(w.K, -1) if w.mode == "fp4" else sc).cpu().numpy()
        cpu = cpu_baseline_dequant(w, np.ascontiguousarray(packed), np.ascontiguousarray(scale), args.cpu_budget)
    line = {
        "metric": "Gelem/s dequantized (codes of x[K,M,N] -> values) + % of HBM roofline, 1 MI355X",
        "value": round(elems * args.steps / (total_ms / 1e3) / 1e9, 2),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "op": "dequant", "K": w.K, "M": w.M, "N": w.N, "mode": w.mode,
                   "buffer_sets": nsets, "parallelism": "none"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_mx_gemm(args, w, x_host, p1, p2, to_dev, dev):
    """Times fq_mx_gemm with A = the workload's per-group quantizer output (T = K tokens,
    H = M*N) and synthetic MXFP4 weights W [O, H] (seeded random codes and e8m0 scales)."""
    import numpy as np
    import torch

    import flatquant_transform_quant_amd as fq

    if w.mode != "fp4":
        print("--op mxgemm needs a per-group (fp4) workload", file=sys.stderr)
        return 2
    T, H, O = w.K, w.M * w.N, args.gemm_out
    x = to_dev(x_host)
    a, a_sc = fq.empty_outputs(T, w.M, w.N, "fp4", dev)
    fq.quantize(x, to_dev(p1), to_dev(p2) if p2 is not None else None, a, a_sc, "fp4", w.clip_ratio, w.dst_type_max)
    del x
    rng = np.random.default_rng(1234)
    wc = torch.from_numpy(rng.integers(0, 256, (O, H // 2), dtype=np.uint8)).to(dev)
    ws = torch.from_numpy(rng.integers(118, 128, (O, -(-H // 64), 2), dtype=np.uint8)).to(dev)
    c = torch.empty((T, O), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.Stream(dev)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        fq.mx_gemm(a, a_sc, wc, ws, H, out=c, stream=stream)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        fq.mx_gemm(a, a_sc, wc, ws, H, out=c, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms = total_ms / args.steps
    flops = 2 * T * O * H
    tfs = flops / (ms / 1e3) / 1e12
    bytes_ = T * H // 2 + O * H // 2 + (T + O) * 2 * (-(-H // 64)) + 2 * T * O
    roof = {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_FP4_PEAK_TFS, "unit": "TFLOP/s",
            "frac": round(tfs / MFMA_FP4_PEAK_TFS, 4), "traffic": profiled_gemm_traffic("mx_gemm_kernel", f"{T}x{O}x{H}"),
            "kernel": "mx_gemm_kernel",
            "avg_launch_us": round(ms * 1e3, 3), "algorithmic_flops": flops, "algorithmic_bytes": bytes_,
            "other_frac": round(bytes_ / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    cpu = None
    if not args.no_cpu:
        import oracle

        rows = 4
        a_h = a[:rows].cpu().numpy()
        ae_h = a_sc[:rows].reshape(rows, -1).cpu().numpy()
        t = time.perf_counter()
        oracle.mx_gemm(a_h, ae_h, wc.cpu().numpy(), ws.reshape(O, -1).cpu().numpy(), H)
        dt = time.perf_counter() - t
        cpu = {"value": 2 * rows * O * H / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
               "sample": f"{rows} of {T} rows of C ({rows * O} outputs, H = {H}), {dt:.2f} s wall on 1 thread"}
    line = {
        "metric": "TFLOP/s of the MXFP4 GEMM consuming the quantizer output + % of the fp4 MFMA roofline, 1 MI355X",
        "value": round(tfs, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "data": "synthetic",
        "config": {"workload": w.name, "op": "mxgemm", "T": T, "H": H, "O": O, "c": "bf16", "parallelism": "none"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_int4_gemm(args, w, x_host, p1, p2, to_dev, dev):
    """Times fq_int4_gemm with A = the workload's per-token int4 quantizer output (T = K
    tokens, H = M*N) and its scales, and synthetic int4 weights W [O, H] with per-channel fp32
    scales (seeded)."""
    import numpy as np
    import torch

    import flatquant_transform_quant_amd as fq

    if w.mode not in ("int32", "int4"):
        print("--op i4gemm needs a per-token int4 workload", file=sys.stderr)
        return 2
    T, H, O = w.K, w.M * w.N, args.gemm_out
    x = to_dev(x_host)
    a, a_sc = fq.empty_outputs(T, w.M, w.N, "int4", dev)
    fq.quantize(x, to_dev(p1), to_dev(p2), a, a_sc, "int4", w.clip_ratio, w.dst_type_max)
    del x
    a = a.reshape(T, H // 2)
    rng = np.random.default_rng(1235)
    wc = torch.from_numpy(rng.integers(0, 256, (O, H // 2), dtype=np.uint8)).to(dev)
    ws = torch.from_numpy(np.abs(rng.standard_normal(O)).astype(np.float32) * np.float32(0.01)).to(dev)
    c = torch.empty((T, O), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.Stream(dev)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        fq.int4_gemm(a, a_sc, wc, ws, H, out=c, stream=stream)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        fq.int4_gemm(a, a_sc, wc, ws, H, out=c, stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms = total_ms / args.steps
    ops = 2 * T * O * H
    tops = ops / (ms / 1e3) / 1e12
    bytes_ = T * H // 2 + O * H // 2 + 4 * (T + O) + 2 * T * O
    roof = {"bound": "mfma", "achieved": round(tops, 1), "peak": MFMA_INT8_PEAK_TOPS, "unit": "TOP/s",
            "frac": round(tops / MFMA_INT8_PEAK_TOPS, 4),
            "traffic": profiled_gemm_traffic("int4_gemm_kernel", f"{T}x{O}x{H}"), "kernel": "int4_gemm_kernel",
            "avg_launch_us": round(ms * 1e3, 3), "algorithmic_ops": ops, "algorithmic_bytes": bytes_,
            "other_frac": round(bytes_ / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    cpu = None
    if not args.no_cpu:
        import oracle

        rows = 4
        t = time.perf_counter()
        oracle.int4_gemm(a[:rows].cpu().numpy(), a_sc[:rows].cpu().numpy(), wc.cpu().numpy(), ws.cpu().numpy(), H)
        dt = time.perf_counter() - t
        cpu = {"value": 2 * rows * O * H / dt / 1e12, "unit": "TOP/s", "cores": 1, "kind": "oracle",
               "sample": f"{rows} of {T} rows of C ({rows * O} outputs, H = {H}), {dt:.2f} s wall on 1 thread"}
    line = {
        "metric": "TOP/s of the int4 GEMM consuming the quantizer output + % of the int8 MFMA roofline, 1 MI355X",
        "value": round(tops, 1),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "data": "synthetic",
        "config": {"workload": w.name, "op": "i4gemm", "T": T, "H": H, "O": O, "c": "bf16", "parallelism": "none"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
