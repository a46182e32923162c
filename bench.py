#!/usr/bin/env python3
"""Benchmark of the LLM.int8() mixed-precision linear layer on one MI355X.

A step is one llmint8_linear call: outlier detection, row-wise quantization of
X, K-compaction when the outlier share calls for it, the int8 GEMM with its
fused fp16 outlier product, dequantization and merge. Weights are quantized
once before timing (the method quantizes them at load), and that pass is
reported on its own. Inputs are resident in HBM when the timed region starts.
To keep the 256 MB Infinity Cache from serving the weights, consecutive steps
cycle through distinct copies of the weight set (and of the activation).

The timed region replays a HIP graph that holds one call per weight set and
activation of that rotation, so the step rate is the GPU's, not that of the
Python launch loop (the eager rate is reported beside it). The GEMM kernel's
duration comes from event pairs that the kernel's own dispatch stamps, one pair
per call, over a run of eager calls.

Prints one JSON line. `value` is the whole-step rate in the workload's unit:
GB/s of algorithmic bytes for the HBM-bound decode and tiny shapes, TOPS of
algorithmic work (int8 ops + fp16 flops) for the prefill shapes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

# Kernel arguments in device memory for eager launches too, as a HIP graph
# keeps them: the GEMM's event-timed eager calls then run like the graph's
# (with host-resident arguments each launch's first argument load crosses
# PCIe; measured 9.1 against 8.2 us for the decode GEMM, same graph rate).
# Set before anything initializes HIP; a value the caller set is kept.
os.environ.setdefault("HIP_FORCE_DEV_KERNARG", "1")

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LLM.int8() linear TOPS & GB/s at 7B/13B shapes; % of int8 MFMA / HBM peak"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
FP16_PEAK_TFLOPS = 2500.0
HBM_BOUND = ("tiny", "decode")
DECODE_MAX_M = 64  # row count up to which the library takes its small-M path
PROFILES = os.path.join(ROOT, "profiles")
# the sources that define the GEMM kernels (small-M and large-M)
# Sources of the GEMM kernels whose HBM counters are committed: the split-K
# small-M kernels (up to 64 rows; the single-kernel path runs none of the
# workloads with counters) and the large-M ones, digested separately so that a
# change to one family leaves the other's counters valid.
_CSRC = os.path.join(ROOT, "bit_quantized_matmul_col_amd", "csrc")
KERNEL_SOURCES = {
    "small_m": [os.path.join(_CSRC, f) for f in ("common.hpp", "internal.hpp", "decode.hip")],
    "large_m": [os.path.join(_CSRC, f) for f in
                ("common.hpp", "internal.hpp", "gemm_core.hpp", "gemm.hip", "gemm_narrow.hip")],
}
SMALL_M_MAX = 64  # rows up to which the layer runs the small-M kernels


def _code_only(text: str) -> str:
    """Source text without comments and blank space, so that editing a comment
    does not mark the counters as taken on a different kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_family(workload: str) -> str:
    import workloads
    return "small_m" if workloads.WORKLOADS[workload].M <= SMALL_M_MAX else "large_m"


def kernel_source_digest(family: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[family]:
        with open(p, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str, variant: str = "int8"):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    or None when it is missing or was taken on a different kernel source."""
    tag = workload if variant == "int8" else f"{variant}_{workload}"
    path = os.path.join(PROFILES, f"gemm_{tag}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_digest") != kernel_source_digest(kernel_family(workload)):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def uses_compaction(M, K, n_out, any_m=False):
    """The library's rule for running the 8-bit GEMM on the K - |O| kept columns
    (the small-M int8 path never compacts; the FP8 layer runs the large-M
    kernels at every M)."""
    return ((any_m or M > DECODE_MAX_M) and n_out > 0 and K <= 32768
            and M * n_out * 16 > 5000 * (2 * K - n_out))


def step_work(M, K, N, n_out, compacted, int8w=False, large_m=False):
    """Algorithmic bytes and work of one layer call, and the algorithmic bytes of
    its GEMM kernel. The small-M GEMM kernel quantizes fp16 X itself and writes
    int32 sums, so its minimum traffic is Wq + X + C; the large-M kernel reads
    Xq, Wq (or their compacted copies), the scales and the outlier operands and
    writes Y. With int8 outlier weights the outlier rows come out of Wq, which
    the call reads anyway, so the fp16 rows drop out of the call's bytes."""
    k_int8 = K - n_out
    w_o = 0 if int8w else 2 * n_out * N
    call_bytes = 2 * M * K + K * N + 4 * N + w_o + 2 * M * N
    if M <= DECODE_MAX_M and not large_m:
        gemm_bytes = N * K + 2 * M * K + 4 * M * N
    else:
        k_loop = k_int8 if compacted else K
        gemm_bytes = (N * k_loop + 4 * N + M * k_loop + 4 * M + 2 * M * n_out
                      + 2 * n_out * N + 2 * M * N)
    int8_ops = 2 * M * N * k_int8
    fp16_flops = 2 * M * N * n_out
    return call_bytes, gemm_bytes, int8_ops, fp16_flops


def accuracy(torch, lm, X_host, W_host, Xd, Wd, threshold, n_rows=16):
    """Output error of each variant of the layer against the exact product X.W
    (fp64) on sampled rows: mean absolute error (the per-layer error measure of
    the Lightning Fabric page, section 3.12), its ratio to the mean |X.W|, and
    the largest absolute error."""
    import numpy as np

    M = X_host.shape[0]
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(M).choice(
        M, size=min(n_rows, M), replace=False)]))
    exact = X_host[rows].astype(np.float64) @ W_host.astype(np.float64)
    scale = float(np.abs(exact).mean())
    rt = torch.from_numpy(rows).to(Xd.device)
    Wq, s = lm.llmint8_quantize_colwise(Wd)
    Wqt, sw = lm.llmint8_quantize_tensorwise(Wd)
    Wq8, s8 = lm.llmint8_quantize_colwise_fp8(Wd)
    variants = {
        "llm_int8": lambda: lm.llmint8_linear(Xd, Wq, s, Wd, threshold),
        "llm_int8_int8_weights": lambda: lm.llmint8_linear(Xd, Wq, s, None, threshold,
                                                           outlier_weights="int8"),
        "vector_wise_no_outliers": lambda: lm.llmint8_linear(Xd, Wq, s, None, math.inf),
        "per_tensor": lambda: lm.llmint8_linear_tensorwise(Xd, Wqt, sw),
        "fp8_e4m3_decomposition": lambda: lm.llmint8_linear_fp8(Xd, Wq8, s8, Wd, threshold),
    }
    out = {"rows": int(rows.size), "reference": "fp64 X.W on the same rows",
           "mean_abs_X_W": round(scale, 6)}
    for name, run in variants.items():
        y = run().index_select(0, rt).cpu().numpy().astype(np.float64)
        err = np.abs(y - exact)
        out[name] = {"mean_abs_err": float(f"{err.mean():.6g}"),
                     "rel_mean_abs_err": float(f"{err.mean() / scale:.6g}"),
                     "max_abs_err": float(f"{err.max():.6g}")}
        torch.cuda.empty_cache()
    return out


def vendor_int8_gemm(torch, M, K, N, dev, reps=20):
    """Reference point, not part of the layer: the plain int8 GEMM of the same
    shape (Xq . Wq^T over all of K, int32 out, no outlier product, no
    dequantization) through torch._int_mm, which ROCm runs on hipBLASLt."""
    a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev)
    b = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev)
    try:
        for _ in range(3):
            torch._int_mm(a, b.t())
    except Exception as e:  # not every shape is supported by the library
        return {"library": "torch._int_mm (hipBLASLt)", "error": repr(e)[:120]}
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch._int_mm(a, b.t())
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tops = 2 * M * N * K / (ms * 1e-3) / 1e12
    return {"library": "torch._int_mm (hipBLASLt)", "work": "2MNK int8 ops, int32 out",
            "ms": round(ms, 6), "TOPS": round(tops, 2),
            "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}


def cpu_baseline(wl, X, W, threshold, budget_s, hbm_bound, n_out, fp8=False):
    """The oracle as it stands, single-threaded, on a bounded sample. Its weight
    quantization (load time, like the GPU's) is done first and not timed."""
    import numpy as np
    import oracle

    if fp8:
        Wq8, s8 = oracle.quantize_colwise_fp8(W)

        def layer(rows):
            return oracle.linear_fp8(X, W, threshold, Wq8=Wq8, s=s8, rows=rows)
    else:
        Wq, s = oracle.quantize_colwise(W)

        def layer(rows):
            return oracle.linear_rows(X, W, threshold, rows, Wq=Wq, s=s)
    rows = wl.M
    if not hbm_bound:
        rows = 4
    sample_rows = np.arange(rows)
    reps, elapsed = 0, 0.0
    while reps == 0 or (elapsed < budget_s and reps < 50):
        t0 = time.perf_counter()
        layer(sample_rows)
        elapsed += time.perf_counter() - t0
        reps += 1
    per = elapsed / reps
    if hbm_bound:
        call_bytes = step_work(wl.M, wl.K, wl.N, n_out, False, large_m=fp8)[0]
        value, unit = call_bytes / per / 1e9, "GB/s"
        sample = f"{reps} whole layer calls on the {wl.M}x{wl.K}x{wl.N} workload"
    else:
        work = 2 * rows * wl.N * wl.K
        value, unit = work / per / 1e12, "TOPS"
        sample = (f"outlier scan over all {wl.M} rows + rows 0..{rows - 1} of the "
                  f"{wl.M}x{wl.K}x{wl.N} workload, {reps} repetitions")
    return {"value": round(value, 6), "unit": unit, "cores": 1, "kind": "oracle",
            "sample": sample, "seconds": round(elapsed, 2)}


def main():
    import workloads

    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--threshold", type=float, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-accuracy", action="store_true",
                    help="skip the output-error comparison of the layer's variants")
    ap.add_argument("--variant", default="int8", choices=("int8", "fp8"),
                    help="int8: the LLM.int8() layer; fp8: its E4M3 variant")
    ap.add_argument("--outlier-weights", default="fp16", choices=("fp16", "int8"),
                    help="fp16: outlier rows of the fp16 weight; int8: from Wq (no fp16 W kept)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the layer on one GPU; a run on several GPUs is not "
              "provided (how the layer would shard is described, not measured). "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_quantized_matmul_col_amd as lm

    lm.lib()
    wl = workloads.WORKLOADS[args.workload]
    threshold = wl.threshold if args.threshold is None else args.threshold
    hbm_bound = args.workload in HBM_BOUND
    steps = args.steps if args.steps is not None else (2000 if hbm_bound else 100)
    warmup = args.warmup if args.warmup is not None else max(10, steps // 10)
    dev = torch.device("cuda:0")

    # inputs: weight sets and activations, resident before timing
    W_host = workloads.make_w(wl)
    W0 = torch.from_numpy(W_host).to(dev)
    wq_bytes = wl.N * wl.K
    n_sets = max(2, min(32, math.ceil(600e6 / wq_bytes)))
    x_pool = 4
    X_host = [workloads.make_x(wl, c) for c in range(x_pool)] if wl.per_call else \
        [workloads.make_x(wl)]
    Xs = [torch.from_numpy(X_host[c % len(X_host)]).to(dev) for c in range(x_pool)]

    fp8 = args.variant == "fp8"
    if fp8 and args.outlier_weights != "fp16":
        sys.exit("the FP8 layer takes its outlier rows from the fp16 weight")
    quantize = lm.llmint8_quantize_colwise_fp8 if fp8 else lm.llmint8_quantize_colwise
    # load-time weight quantization, timed on its own
    Wq0, s0 = quantize(W0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        quantize(W0)
    e1.record()
    torch.cuda.synchronize()
    colwise_ms = e0.elapsed_time(e1) / reps
    colwise_bytes = 3 * wl.K * wl.N + 4 * wl.N

    int8w = args.outlier_weights == "int8"
    sets = [(Wq0, s0, None if int8w else W0)] + [
        (Wq0.clone(), s0.clone(), None if int8w else W0.clone()) for _ in range(n_sets - 1)]
    Y = torch.empty((wl.M, wl.N), dtype=torch.float16, device=dev)
    ws_size = (lm.llmint8_linear_fp8_workspace_size if fp8 else lm.llmint8_workspace_size)
    ws = torch.empty((ws_size(wl.M, wl.K, wl.N),), dtype=torch.uint8, device=dev)
    cnt = torch.zeros((1,), dtype=torch.int32, device=dev)

    def step(i, opts=None):
        Wq, s, W = sets[i % n_sets]
        if fp8:
            lm.llmint8_linear_fp8(Xs[i % x_pool], Wq, s, W, threshold, Y=Y, workspace=ws,
                                  outlier_count=cnt, opts=opts)
        else:
            lm.llmint8_linear(Xs[i % x_pool], Wq, s, W, threshold, Y=Y, workspace=ws,
                              outlier_count=cnt, opts=opts, outlier_weights=args.outlier_weights)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: replays of a HIP graph holding graph_len consecutive layer
    # calls (every weight set and activation of the rotation), so the rate is the
    # GPU's and not the Python launch loop's.
    graph_len = n_sets * x_pool // math.gcd(n_sets, x_pool)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(graph_len):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(graph_len):
            step(i)
    replays = max(1, math.ceil(steps / graph_len))
    steps = replays * graph_len
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(replays):
        graph.replay()
    t_stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_stop)
    ms_per_step = total_ms / steps

    # The same calls launched one by one from Python (no graph), for reference.
    eager_steps = min(steps, 1000)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(eager_steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / eager_steps

    # GEMM kernel duration: events stamped by the GEMM kernel's own dispatch on
    # the library's stream, one pair per call, over eager calls.
    kt_steps = min(steps, 500)
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(kt_steps)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(kt_steps)]
    for e in ev_b + ev_e:
        e.record()  # creates the underlying hipEvent
    torch.cuda.synchronize()
    # A spin kernel holds the queue while Python enqueues the calls, so they
    # run back to back as in the timed region instead of one by one behind the
    # Python loop (an idle GPU between calls stretches each kernel's events).
    spin_ms = 1.5 * eager_ms * kt_steps
    torch.cuda._sleep(int(spin_ms * 1e-3 * 2.4e9))
    for i in range(kt_steps):
        step(i, lm.LinearOpts(gemm_begin_event=ev_b[i].cuda_event,
                              gemm_end_event=ev_e[i].cuda_event))
    torch.cuda.synchronize()
    gemm_ms = sum(ev_b[i].elapsed_time(ev_e[i]) for i in range(kt_steps)) / kt_steps

    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        a = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    n_out = int(cnt.item())
    compacted = uses_compaction(wl.M, wl.K, n_out, any_m=fp8)
    call_bytes, gemm_bytes, int8_ops, fp16_flops = step_work(wl.M, wl.K, wl.N, n_out, compacted,
                                                             int8w, large_m=fp8)
    if hbm_bound:
        value, unit = call_bytes / (ms_per_step * 1e-3) / 1e9, "GB/s"
        achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        value, unit = (int8_ops + fp16_flops) / (ms_per_step * 1e-3) / 1e12, "TOPS"
        # fp16 flops weigh double: the fp16 MFMA peak is half the int8 one
        achieved = (int8_ops + 2 * fp16_flops) / (gemm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS,
                "unit": "TFLOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4)}
    roof["traffic"] = read_traffic(args.workload, args.variant)

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3" if fp8 else "i8",
        "data": "synthetic",
        "config": {"workload": wl.description, "M": wl.M, "K": wl.K, "N": wl.N,
                   "threshold": threshold, "outlier_columns": n_out,
                   "variant": "fp8 (E4M3) decomposition" if fp8 else "LLM.int8()",
                   "outlier_weights": args.outlier_weights,
                   "k_compacted": compacted, "weight_sets_cycled": n_sets,
                   "activation_pool": x_pool, "parallelism": "single GPU"},
        "roofline": roof,
        "gemm_kernel_ms": round(gemm_ms, 6),
        "timing": {"timed_region": f"{replays} replays of a HIP graph of {graph_len} layer calls",
                   "eager_ms_per_step": round(eager_ms, 6),
                   "gemm_kernel_timing": f"dispatch-stamped events around the GEMM kernel "
                                         f"of {kt_steps} eager calls queued behind a spin "
                                         f"kernel (run back to back)"},
        "whole_step": {"algorithmic_bytes": call_bytes, "int8_ops": int8_ops,
                       "fp16_flops": fp16_flops,
                       "GB_per_s": round(call_bytes / (ms_per_step * 1e-3) / 1e9, 2),
                       "TOPS": round((int8_ops + fp16_flops) / (ms_per_step * 1e-3) / 1e12, 3),
                       "wall_s": round(wall, 4)},
        "quantize_colwise": {"ms": round(colwise_ms, 5), "algorithmic_bytes": colwise_bytes,
                             "GB_per_s": round(colwise_bytes / (colwise_ms * 1e-3) / 1e9, 2)},
    }
    if not hbm_bound:
        out["vendor_int8_gemm"] = vendor_int8_gemm(torch, wl.M, wl.K, wl.N, dev)
    if not args.no_accuracy:
        del graph
        out["accuracy"] = accuracy(torch, lm, X_host[0], W_host, Xs[0], W0, threshold)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, X_host[0], W_host, threshold, args.cpu_seconds,
                                           hbm_bound, n_out, fp8)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
