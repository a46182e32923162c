#!/usr/bin/env python3
"""Benchmark of the LLM.int8() mixed-precision linear layer on one MI355X.

A step is one llmint8_linear call: outlier detection, row-wise quantization of
X, K-compaction when the outlier share calls for it, the int8 GEMM with its
fused fp16 outlier product, dequantization and merge. Weights are quantized
once before timing (the method quantizes them at load), and that pass is
reported on its own. Inputs are resident in HBM when the timed region starts.
To keep the 256 MB Infinity Cache from serving the weights of the decode-sized
workloads, consecutive steps cycle through distinct copies of the weight set
(and of the activation).

The timed region replays HIP graphs holding exactly --steps layer calls, so
the step rate is the GPU's, not that of the Python launch loop (the eager rate
and a sustained rate over at least 1000 calls are reported beside it). The
GEMM kernel's duration comes from event pairs that the kernel's own dispatch
stamps, one pair per call, over a run of eager calls.

By default the line also carries, for the prefill, 13b and 70b workloads (70b
at thresholds 6, 4 and inf), the step time, TOPS, the GEMM kernel's time and
roofline fraction, and the standalone bandwidth of the three quantize passes.

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
import subprocess
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
# dense int8 MFMA ops per CU per clock on gfx950: the 5.0 POPS figure is
# 256 CUs x 2.4 GHz x 8192
INT8_OPS_PER_CU_CLOCK = 8192
HBM_BOUND = ("tiny", "decode")
DECODE_MAX_M = 256  # rows up to which the library may take its small-M path (65-256: shape-dependent)
PROFILES = os.path.join(ROOT, "profiles")
# Sources of the GEMM kernels whose HBM counters are committed: the split-K
# small-M kernels (up to 64 rows, or 256 when they stream K in one pass; the
# single-kernel path runs none of the workloads with counters) and the
# large-M ones, digested separately so that a change to one family leaves the
# other's counters valid.
_CSRC = os.path.join(ROOT, "bit_quantized_matmul_col_amd", "csrc")
KERNEL_SOURCES = {
    "small_m": [os.path.join(_CSRC, f) for f in ("common.hpp", "internal.hpp", "decode.hip")],
    "large_m": [os.path.join(_CSRC, f) for f in
                ("common.hpp", "internal.hpp", "gemm_core.hpp", "gemm.hip", "gemm_narrow.hip")],
}
SMALL_M_MAX = 256  # rows up to which the layer runs the small-M kernels
# the larger workloads measured by default next to the headline one
SWEEP = (("prefill", (6.0,)), ("13b", (6.0,)), ("70b", (6.0, 4.0, math.inf)))


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
    its GEMM kernel. The small-M GEMM kernel must read Wq and the fp16 X (its
    int32 split sums are the kernel's own intermediate, not algorithmic);
    the large-M kernel reads Xq, Wq (or their compacted copies), the scales
    and the outlier operands and writes Y. With int8 outlier weights the
    outlier rows come out of Wq, which the call reads anyway, so the fp16 rows
    drop out of the call's bytes."""
    k_int8 = K - n_out
    w_o = 0 if int8w else 2 * n_out * N
    call_bytes = 2 * M * K + K * N + 4 * N + w_o + 2 * M * N
    if M <= DECODE_MAX_M and not large_m:
        gemm_bytes = N * K + 2 * M * K
    else:
        k_loop = k_int8 if compacted else K
        gemm_bytes = (N * k_loop + 4 * N + M * k_loop + 4 * M + 2 * M * n_out
                      + 2 * n_out * N + 2 * M * N)
    int8_ops = 2 * M * N * k_int8
    fp16_flops = 2 * M * N * n_out
    return call_bytes, gemm_bytes, int8_ops, fp16_flops


def pass_bytes(M, K, N):
    """Algorithmic bytes of the three quantize passes: each tensor read or
    written once (find_outliers reads X; quantize_rowwise reads X, writes Xq
    and m; quantize_colwise reads W, writes Wq and s)."""
    return {"find_outliers": 2 * M * K, "quantize_rowwise": 3 * M * K + 4 * M,
            "quantize_colwise": 3 * K * N + 4 * N}


def host_facts():
    """CPU model and thread counts of the host the benchmark runs on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "cpu_count": os.cpu_count()}


def device_facts(torch, dev):
    """The GPU as the runtime reports it, and the int8 MFMA peak derived from
    its compute-unit count and the peak engine clock rocminfo lists."""
    p = torch.cuda.get_device_properties(dev)
    facts = {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
             "compute_units": p.multi_processor_count,
             "hbm_bytes": int(p.total_memory)}
    mhz = None
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
        arch = facts["arch"].split(":")[0]
        for block in out.split("*******"):
            if arch and arch in block and "Compute Unit" in block:
                m = re.search(r"Max Clock Freq\. \(MHz\):\s*(\d+)", block)
                if m:
                    mhz = int(m.group(1))
                break
    except (OSError, subprocess.SubprocessError):
        pass
    facts["max_clock_mhz"] = mhz
    if mhz:
        facts["int8_peak_derived_tops"] = round(
            facts["compute_units"] * mhz * 1e6 * INT8_OPS_PER_CU_CLOCK / 1e12, 1)
    return facts


def copy_ceiling(torch, dev, mib=1024, reps=10):
    """Plain device-to-device copy of a buffer far larger than the caches:
    bytes read + bytes written per second, the practical HBM ceiling for a
    stream that reads and writes once."""
    n = mib << 20
    a = torch.empty((n,), dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(2):
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
    return {"what": f"device copy of {mib} MiB, read + write bytes", "ms": round(ms, 4),
            "GB_per_s": round(2 * n / (ms * 1e-3) / 1e9, 1)}


def graph_time(torch, calls, steps, warmup_replays=1):
    """Time exactly `steps` calls of `calls(i)` (i = 0 .. steps-1) replayed from
    HIP graphs: one graph of min(steps, 1024) calls replayed, plus one graph of
    the remainder. Returns (ms per call, description)."""
    glen = min(steps, 1024)
    reps, tail = divmod(steps, glen)

    def capture(n, offset):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # allocations and lazy setup outside the capture
            for i in range(n):
                calls(offset + i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                calls(offset + i)
        return g

    g = capture(glen, 0)
    gt = capture(tail, reps * glen) if tail else None
    for _ in range(warmup_replays):
        g.replay()
        if gt is not None:
            gt.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    if gt is not None:
        gt.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    desc = f"{reps} replay(s) of a HIP graph of {glen} layer calls"
    if tail:
        desc += f" + 1 replay of a graph of {tail}"
    del g, gt
    return ms, desc


def gemm_event_ms(torch, lm, step, n, eager_ms):
    """Average GEMM kernel duration from event pairs its own dispatch stamps,
    over n eager calls queued behind a spin kernel so that they run back to
    back as in the timed region (an idle GPU between calls stretches each
    kernel's events)."""
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev_b + ev_e:
        e.record()  # creates the underlying hipEvent
    torch.cuda.synchronize()
    spin_ms = 1.5 * eager_ms * n + 1.0
    torch.cuda._sleep(int(spin_ms * 1e-3 * 2.4e9))
    for i in range(n):
        step(i, lm.LinearOpts(gemm_begin_event=ev_b[i].cuda_event,
                              gemm_end_event=ev_e[i].cuda_event))
    torch.cuda.synchronize()
    return sum(ev_b[i].elapsed_time(ev_e[i]) for i in range(n)) / n


def eager_ms(torch, step, n):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def quantize_passes(torch, lm, Xs, Ws, threshold, calls=20):
    """Standalone time and algorithmic bandwidth of the three public quantize
    passes, each replayed from a HIP graph of `calls` calls cycling through the
    given activations (weights), against the 8 TB/s peak. The callers pass
    weight copies that together exceed the 256 MB Infinity Cache, so the column
    pass reads W from HBM."""
    M, K = Xs[0].shape
    N = Ws[0].shape[1]
    nb = pass_bytes(M, K, N)
    dev = Xs[0].device
    ws = torch.empty((max(lm.llmint8_find_outliers_workspace_size(M, K), 1),),
                     dtype=torch.uint8, device=dev)
    found = [lm.llmint8_find_outliers(X, threshold, workspace=ws) for X in Xs]
    torch.cuda.synchronize()
    runs = {
        "find_outliers": lambda i: lm.llmint8_find_outliers(Xs[i % len(Xs)], threshold,
                                                            workspace=ws),
        "quantize_rowwise": lambda i: lm.llmint8_quantize_rowwise(Xs[i % len(Xs)],
                                                                  *found[i % len(Xs)]),
        "quantize_colwise": lambda i: lm.llmint8_quantize_colwise(Ws[i % len(Ws)]),
    }
    out = {}
    for name, fn in runs.items():
        n = calls if name != "quantize_colwise" else max(2, min(calls, 8))
        ms, _ = graph_time(torch, fn, n)
        gbs = nb[name] / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 5), "algorithmic_bytes": nb[name],
                     "GB_per_s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        torch.cuda.empty_cache()
    return out


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


def cpu_baseline(wl, X, W, threshold, budget_s, hbm_bound, n_out, fp8=False):
    """The oracle as it stands, single-threaded, on a bounded sample, with each
    step timed on its own: weight quantization (a0, load time), the outlier
    scan (a1), row quantization (a2) and the int8 product with the merge
    (a3-a5). The headline figure is the whole call's rate."""
    import numpy as np
    import oracle

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    # one core: the oracle is single-threaded; pin this thread to the first core
    # it may run on for the timing (restored below)
    allowed = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
    pinned = min(allowed) if allowed else None
    if pinned is not None:
        os.sched_setaffinity(0, {pinned})
    try:
        return _cpu_baseline_pinned(wl, X, W, threshold, budget_s, hbm_bound, n_out, fp8, timed,
                                    pinned)
    finally:
        if allowed:
            os.sched_setaffinity(0, allowed)


def _cpu_baseline_pinned(wl, X, W, threshold, budget_s, hbm_bound, n_out, fp8, timed, pinned):
    import numpy as np
    import oracle

    rows = wl.M if hbm_bound else 4
    Wsub = W if hbm_bound else W[:, :min(W.shape[1], 2048)]
    if fp8:
        (Wq, s), t_a0 = timed(lambda: oracle.quantize_colwise_fp8(Wsub))
        if Wsub is not W:
            Wq, s = oracle.quantize_colwise_fp8(W)
    else:
        (Wq, s), t_a0 = timed(lambda: oracle.quantize_colwise(Wsub))
        if Wsub is not W:
            Wq, s = oracle.quantize_colwise(W)
    Xs = np.ascontiguousarray(X[:rows])
    steps = {"a1_find_outliers": [], "a2_quantize_rowwise": [], "a3_a5_gemm_and_merge": []}
    reps, elapsed = 0, 0.0
    while reps == 0 or (elapsed < budget_s and reps < 50):
        idx, t1 = timed(lambda: oracle.find_outliers(X, threshold))
        if fp8:
            (Xq, m), t2 = timed(lambda: oracle.quantize_rowwise_fp8(Xs, idx))
            _, t3 = timed(lambda: oracle.merge_fp8(oracle.gemm_fp8(Xq, Wq), m, s, Xs, W, idx))
        else:
            (Xq, m), t2 = timed(lambda: oracle.quantize_rowwise(Xs, idx))
            _, t3 = timed(lambda: oracle.merge(oracle.gemm_i8(Xq, Wq), m, s, Xs, W, idx))
        for k, t in zip(steps, (t1, t2, t3)):
            steps[k].append(t)
        elapsed += t1 + t2 + t3
        reps += 1
    med = {k: sorted(v)[len(v) // 2] for k, v in steps.items()}
    nb = pass_bytes(wl.M, wl.K, Wsub.shape[1])
    per_step = {
        "a0_quantize_colwise": {"s": round(t_a0, 4), "GB_per_s": round(
            nb["quantize_colwise"] / t_a0 / 1e9, 4), "sample": f"W [{wl.K} x {Wsub.shape[1]}]"},
        "a1_find_outliers": {"s": round(med["a1_find_outliers"], 5), "GB_per_s": round(
            nb["find_outliers"] / med["a1_find_outliers"] / 1e9, 4)},
        "a2_quantize_rowwise": {"s": round(med["a2_quantize_rowwise"], 5), "GB_per_s": round(
            pass_bytes(rows, wl.K, 1)["quantize_rowwise"] / med["a2_quantize_rowwise"] / 1e9, 4),
            "rows": rows},
        "a3_a5_gemm_and_merge": {"s": round(med["a3_a5_gemm_and_merge"], 5), "TOPS": round(
            2 * rows * wl.N * wl.K / med["a3_a5_gemm_and_merge"] / 1e12, 6), "rows": rows},
    }
    per_call = med["a1_find_outliers"] + med["a2_quantize_rowwise"] + med["a3_a5_gemm_and_merge"]
    if hbm_bound:
        call_bytes = step_work(wl.M, wl.K, wl.N, n_out, False, large_m=fp8)[0]
        value, unit = call_bytes / per_call / 1e9, "GB/s"
        sample = (f"{reps} whole layer calls on the {wl.M}x{wl.K}x{wl.N} workload "
                  f"(median per step)")
    else:
        work = 2 * rows * wl.N * wl.K
        value, unit = work / per_call / 1e12, "TOPS"
        sample = (f"outlier scan over all {wl.M} rows + rows 0..{rows - 1} of the "
                  f"{wl.M}x{wl.K}x{wl.N} workload, {reps} repetitions (median per step)")
    facts = host_facts()
    return {"value": round(value, 6), "unit": unit, "cores": 1, "kind": "oracle",
            "sample": sample, "seconds": round(elapsed + t_a0, 2), "per_step": per_step,
            "threads_used": 1, "pinned_cpu": pinned, "cpu_model": facts["cpu_model"],
            "nproc": facts["nproc"]}


class Layer:
    """Device inputs of one workload and one call of the layer on them."""

    def __init__(self, torch, lm, wl, threshold, dev, variant="int8", outlier_weights="fp16",
                 rotate_weights=True, x_pool=4):
        import workloads
        self.torch, self.lm, self.wl, self.threshold = torch, lm, wl, threshold
        self.fp8 = variant == "fp8"
        self.int8w = outlier_weights == "int8"
        self.outlier_weights = outlier_weights
        self.W_host = workloads.make_w(wl)
        W0 = torch.from_numpy(self.W_host).to(dev)
        self.X_host = ([workloads.make_x(wl, c) for c in range(x_pool)] if wl.per_call
                       else [workloads.make_x(wl)])
        self.Xs = [torch.from_numpy(self.X_host[c % len(self.X_host)]).to(dev)
                   for c in range(x_pool)]
        quantize = lm.llmint8_quantize_colwise_fp8 if self.fp8 else lm.llmint8_quantize_colwise
        Wq0, s0 = quantize(W0)
        self.W0 = W0
        self.n_sets = max(2, min(32, math.ceil(600e6 / (wl.N * wl.K)))) if rotate_weights else 1
        self.sets = [(Wq0, s0, None if self.int8w else W0)] + [
            (Wq0.clone(), s0.clone(), None if self.int8w else W0.clone())
            for _ in range(self.n_sets - 1)]
        self.Y = torch.empty((wl.M, wl.N), dtype=torch.float16, device=dev)
        ws_size = (lm.llmint8_linear_fp8_workspace_size if self.fp8
                   else lm.llmint8_workspace_size)
        self.ws = torch.empty((ws_size(wl.M, wl.K, wl.N),), dtype=torch.uint8, device=dev)
        self.cnt = torch.zeros((1,), dtype=torch.int32, device=dev)
        torch.cuda.synchronize()

    def step(self, i, opts=None):
        Wq, s, W = self.sets[i % self.n_sets]
        X = self.Xs[i % len(self.Xs)]
        if self.fp8:
            self.lm.llmint8_linear_fp8(X, Wq, s, W, self.threshold, Y=self.Y, workspace=self.ws,
                                       outlier_count=self.cnt, opts=opts)
        else:
            self.lm.llmint8_linear(X, Wq, s, W, self.threshold, Y=self.Y, workspace=self.ws,
                                   outlier_count=self.cnt, opts=opts,
                                   outlier_weights=self.outlier_weights)

    def work(self):
        wl = self.wl
        n_out = int(self.cnt.item())
        compacted = uses_compaction(wl.M, wl.K, n_out, any_m=self.fp8)
        return (n_out, compacted) + step_work(wl.M, wl.K, wl.N, n_out, compacted, self.int8w,
                                              large_m=self.fp8)


def rooflines(hbm_bound, ms_per_step, gemm_ms, call_bytes, gemm_bytes, int8_ops, fp16_flops):
    """The dominant kernel's roofline (the GEMM: HBM for small M, int8 MFMA for
    large M; fp16 flops weigh double against the int8 peak) and the whole
    call's: algorithmic bytes over the step time against 8 TB/s, or the ideal
    time int8_ops / 5 POPS + fp16_flops / 2.5 PFLOPS over the step time."""
    if hbm_bound:
        achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        kern = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        call_gbs = call_bytes / (ms_per_step * 1e-3) / 1e9
        call = {"bound": "hbm", "achieved": round(call_gbs, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(call_gbs / HBM_PEAK_GBS, 4)}
    else:
        achieved = (int8_ops + 2 * fp16_flops) / (gemm_ms * 1e-3) / 1e12
        kern = {"bound": "mfma", "achieved": round(achieved, 2), "peak": INT8_PEAK_TOPS,
                "unit": "TFLOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4)}
        t_ideal_ms = (int8_ops / (INT8_PEAK_TOPS * 1e12) + fp16_flops / (FP16_PEAK_TFLOPS * 1e12)) * 1e3
        call = {"bound": "mfma", "ideal_ms": round(t_ideal_ms, 5),
                "frac": round(t_ideal_ms / ms_per_step, 4)}
    return kern, call


def sweep_workload(torch, lm, name, thresholds, dev, steps=10):
    """One larger workload at each of its thresholds: graph-timed steps, the
    GEMM kernel's event time, rooflines and the standalone quantize passes."""
    import workloads
    wl = workloads.WORKLOADS[name]
    L = Layer(torch, lm, wl, thresholds[0], dev, rotate_weights=False,
              x_pool=2 if wl.per_call else 1)
    # copies of W beyond the 256 MB Infinity Cache, so that the column pass
    # reads W from HBM as it would at load time
    Wc = [L.W0] + [L.W0.clone() for _ in range(math.ceil(600e6 / (2 * wl.K * wl.N)) - 1)]
    outs = []
    for threshold in thresholds:
        print(f"# measuring {name} at threshold {threshold}", file=sys.stderr, flush=True)
        L.threshold = threshold
        for i in range(3):
            L.step(i)
        torch.cuda.synchronize()
        ms, _ = graph_time(torch, L.step, steps)
        e_ms = eager_ms(torch, L.step, steps)
        g_ms = gemm_event_ms(torch, lm, L.step, steps, e_ms)
        n_out, compacted, call_bytes, gemm_bytes, int8_ops, fp16_flops = L.work()
        kern, call = rooflines(False, ms, g_ms, call_bytes, gemm_bytes, int8_ops, fp16_flops)
        passes = quantize_passes(torch, lm, L.Xs, Wc, threshold, calls=10)
        outs.append({"workload": wl.description, "M": wl.M, "K": wl.K, "N": wl.N,
                     "threshold": threshold, "outlier_columns": n_out,
                     "k_compacted": compacted, "steps": steps, "ms_per_step": round(ms, 5),
                     "TOPS": round((int8_ops + fp16_flops) / (ms * 1e-3) / 1e12, 2),
                     "gemm_kernel_ms": round(g_ms, 5), "roofline": kern, "call_roofline": call,
                     "quantize_passes": passes})
        torch.cuda.empty_cache()
    del L
    torch.cuda.empty_cache()
    return outs


def summarize_profile(path: str, min_calls: int = 1) -> str:
    """Text summary of a rocprofv3 CSV output directory: per kernel, the call
    count and durations (kernel_stats.csv), or per kernel and counter the
    average value per dispatch (counter_collection.csv)."""
    import csv
    import glob

    lines = []
    stats = sorted(glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True))
    for f in stats:
        rows = list(csv.DictReader(open(f)))
        total = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
        lines.append("# columns: calls, total ns, average ns, min ns, max ns, share of GPU "
                     "time, kernel")
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            if int(r["Calls"]) < min_calls:
                continue
            lines.append(f"{int(r['Calls']):6d} {float(r['TotalDurationNs']):12.0f} "
                         f"{float(r['AverageNs']):12.1f} {float(r['MinNs']):10.0f} "
                         f"{float(r['MaxNs']):10.0f} "
                         f"{100 * float(r['TotalDurationNs']) / total:6.2f}%  {r['Name'][:160]}")
    counters = sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"),
                                recursive=True))
    for f in counters:
        acc = {}
        for r in csv.DictReader(open(f)):
            key = (r["Kernel_Name"], r["Counter_Name"])
            d = acc.setdefault(key, {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        lines.append("# columns: dispatches, average value per dispatch, counter, kernel")
        for (kern, ctr), d in sorted(acc.items(), key=lambda kv: (kv[0][0], kv[0][1])):
            if len(d) < min_calls:
                continue
            lines.append(f"{len(d):6d} {sum(d.values()) / len(d):18.1f}  {ctr:32s} {kern[:160]}")
    return "\n".join(lines)


def main():
    import workloads

    if len(sys.argv) >= 3 and sys.argv[1] == "--summarize-profile":
        print(summarize_profile(sys.argv[2], int(sys.argv[3]) if len(sys.argv) > 3 else 1))
        return

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
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the prefill, 13b and 70b measurements next to the headline")
    ap.add_argument("--variant", default="int8", choices=("int8", "fp8"),
                    help="int8: the LLM.int8() layer; fp8: its E4M3 variant")
    ap.add_argument("--outlier-weights", default="fp16", choices=("fp16", "int8"),
                    help="fp16: outlier rows of the fp16 weight; int8: from Wq (no fp16 W kept)")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed region and the GEMM-event calls (for profiler runs): "
                         "no sustained rate, quantize passes, ceiling, accuracy, sweep or "
                         "CPU baseline")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the layer on one GPU; a run on several GPUs is not "
              "provided (how the layer would shard is described, not measured). "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_quantized_matmul_col_amd as lm

    lm.lib()
    wl = workloads.WORKLOADS[args.workload]
    threshold = wl.threshold if args.threshold is None else args.threshold
    hbm_bound = args.workload in HBM_BOUND
    steps = args.steps if args.steps is not None else (1000 if hbm_bound else 20)
    warmup = args.warmup if args.warmup is not None else max(10, steps // 10)
    if steps < 1 or warmup < 0:
        sys.exit("--steps must be at least 1 and --warmup at least 0")
    dev = torch.device("cuda:0")
    fp8 = args.variant == "fp8"
    if fp8 and args.outlier_weights != "fp16":
        sys.exit("the FP8 layer takes its outlier rows from the fp16 weight")

    L = Layer(torch, lm, wl, threshold, dev, variant=args.variant,
              outlier_weights=args.outlier_weights, rotate_weights=True)
    for i in range(warmup):
        L.step(i)
    torch.cuda.synchronize()

    # Timed region: exactly `steps` layer calls, replayed from HIP graphs.
    ms_per_step, timed_desc = graph_time(torch, L.step, steps)
    # Sustained rate over at least 1000 calls (more weight sets than the cache holds).
    sus_calls = max(1000, steps) if not args.no_extras else steps
    sus_ms, sus_desc = ((ms_per_step, timed_desc) if args.no_extras
                        else graph_time(torch, L.step, sus_calls))
    e_steps = min(max(steps, 100), 1000) if not args.no_extras else steps
    e_ms = eager_ms(torch, L.step, e_steps)
    kt_steps = min(max(steps, 100), 500) if not args.no_extras else steps
    gemm_ms = gemm_event_ms(torch, lm, L.step, kt_steps, e_ms)

    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        a = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    n_out, compacted, call_bytes, gemm_bytes, int8_ops, fp16_flops = L.work()
    kern, call = rooflines(hbm_bound, ms_per_step, gemm_ms, call_bytes, gemm_bytes, int8_ops,
                           fp16_flops)
    kern["traffic"] = read_traffic(args.workload, args.variant)
    if hbm_bound:
        value, unit = call_bytes / (ms_per_step * 1e-3) / 1e9, "GB/s"
    else:
        value, unit = (int8_ops + fp16_flops) / (ms_per_step * 1e-3) / 1e12, "TOPS"

    facts = device_facts(torch, dev) if not args.no_extras else {}
    ceiling = copy_ceiling(torch, dev) if not args.no_extras else {}
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
                   "k_compacted": compacted, "weight_sets_cycled": L.n_sets,
                   "activation_pool": len(L.Xs), "parallelism": "single GPU"},
        "roofline": kern,
        "call_roofline": call,
        "gemm_kernel_ms": round(gemm_ms, 6),
        "timing": {"timed_region": timed_desc, "timed_region_ms": round(ms_per_step * steps, 4),
                   "sustained": {"calls": sus_calls, "region": sus_desc,
                                 "ms_per_step": round(sus_ms, 6),
                                 "value": round(call_bytes / (sus_ms * 1e-3) / 1e9 if hbm_bound
                                                else (int8_ops + fp16_flops) / (sus_ms * 1e-3)
                                                / 1e12, 3)},
                   "eager_ms_per_step": round(e_ms, 6),
                   "gemm_kernel_timing": f"dispatch-stamped events around the GEMM kernel "
                                         f"of {kt_steps} eager calls queued behind a spin "
                                         f"kernel (run back to back)"},
        "whole_step": {"algorithmic_bytes": call_bytes, "gemm_algorithmic_bytes": gemm_bytes,
                       "int8_ops": int8_ops, "fp16_flops": fp16_flops,
                       "GB_per_s": round(call_bytes / (ms_per_step * 1e-3) / 1e9, 2),
                       "TOPS": round((int8_ops + fp16_flops) / (ms_per_step * 1e-3) / 1e12, 3)},
        "build": {"source_digest": lm.build_record.get("source_digest", "")[:16],
                  "compiler": lm.build_record.get("compiler", ""),
                  "built_at": lm.build_record.get("built_at", "")},
        "peaks": {"hbm_published_GB_per_s": HBM_PEAK_GBS,
                  "int8_published_TOPS": INT8_PEAK_TOPS,
                  "fp16_published_TFLOPS": FP16_PEAK_TFLOPS, "device": facts,
                  "measured_copy_ceiling": ceiling},
    }
    if not args.no_extras:
        out["quantize_passes"] = quantize_passes(
            torch, lm, L.Xs, [st[2] if st[2] is not None else L.W0 for st in L.sets], threshold)
    if args.no_extras:
        args.no_accuracy = args.no_sweep = args.no_cpu_baseline = True
    if not args.no_accuracy:
        out["accuracy"] = accuracy(torch, lm, L.X_host[0], L.W_host, L.Xs[0], L.W0, threshold)
    X0_host, W_host = L.X_host[0], L.W_host
    del L
    torch.cuda.empty_cache()
    if not args.no_sweep and args.variant == "int8" and args.outlier_weights == "fp16":
        out["workloads"] = []
        for name, thrs in SWEEP:
            thrs = [t for t in thrs if not (name == args.workload and t == threshold)]
            if thrs:
                out["workloads"] += sweep_workload(torch, lm, name, thrs, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, X0_host, W_host, threshold, args.cpu_seconds,
                                           hbm_bound, n_out, fp8)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
