"""The benchmark's host-side bookkeeping (no GPU): the algorithmic byte and op
counts it reports, its copy of the library's compaction rule, and its refusal
of a multi-GPU run."""
import glob
import math
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_call_bytes():
    # 2MK (X) + KN (Wq) + 4N (scales) + 2|O|N (fp16 outlier rows) + 2MN (Y)
    call, gemm, ops, flops = bench.step_work(32, 4096, 4096, 4, False)
    assert call == 2 * 32 * 4096 + 4096 * 4096 + 4 * 4096 + 2 * 4 * 4096 + 2 * 32 * 4096
    assert call == 17350656
    # the small-M GEMM kernel must read Wq and the fp16 X; its int32 split sums
    # are its own intermediate and are not counted
    assert gemm == 4096 * 4096 + 2 * 32 * 4096 == 17039360
    assert ops == 2 * 32 * 4096 * (4096 - 4) and flops == 2 * 32 * 4096 * 4
    # int8-only weights: the outlier rows come out of Wq, already counted
    assert bench.step_work(32, 4096, 4096, 4, False, int8w=True)[0] == call - 2 * 4 * 4096


def test_large_m_work():
    M, K, N, n = 2048, 4096, 11008, 20
    call, gemm, ops, flops = bench.step_work(M, K, N, n, False)
    assert ops == 2 * M * N * (K - n) and flops == 2 * M * N * n
    assert gemm == N * K + 4 * N + M * K + 4 * M + 2 * M * n + 2 * n * N + 2 * M * N
    # compaction: the 8-bit operands shrink to the K - |O| kept columns
    gemm_c = bench.step_work(M, K, N, n, True)[1]
    assert gemm - gemm_c == (N + M) * n


def test_compaction_rule_matches_the_library():
    # M * |O| * 16 > 5000 * (2K - |O|), K <= 32768, and never on the small-M path
    assert bench.uses_compaction(400, 1024, 1000)
    # no M of the small-M path reaches the rule: M <= 64 < 5000 / 16
    assert not bench.uses_compaction(64, 1024, 1024, any_m=True)
    assert bench.uses_compaction(4096, 5120, 1218)  # the 13b workload
    assert not bench.uses_compaction(2048, 4096, 20)  # prefill
    assert not bench.uses_compaction(100000, 40000, 20000)  # K above the LDS staging cap
    for M, K, n in [(313, 1000, 1000), (312, 1000, 1000), (700, 1008, 300)]:
        assert bench.uses_compaction(M, K, n) == (M * n * 16 > 5000 * (2 * K - n))


def test_multi_gpu_run_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 2
    assert "one GPU" in out.stderr


def test_counter_digest_families(tmp_path, monkeypatch):
    # decode-sized workloads read the small-M kernels' counters, the others the
    # large-M ones; each digest covers only its own family's sources
    assert bench.kernel_family("decode") == "small_m" and bench.kernel_family("tiny") == "small_m"
    for w in ("prefill", "13b", "70b"):
        assert bench.kernel_family(w) == "large_m"
    small = set(map(os.path.basename, bench.KERNEL_SOURCES["small_m"]))
    large = set(map(os.path.basename, bench.KERNEL_SOURCES["large_m"]))
    assert "decode.hip" in small and "decode.hip" not in large
    assert "gemm_core.hpp" in large and "gemm_core.hpp" not in small
    # comments and blank space do not change a digest; code does
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; }  // one\n")
    monkeypatch.setitem(bench.KERNEL_SOURCES, "small_m", [str(src)])
    d0 = bench.kernel_source_digest("small_m")
    src.write_text("/* header */\nint f() {\n  return 1;\n}\n// two\n")
    assert bench.kernel_source_digest("small_m") == d0
    src.write_text("int f() { return 2; }\n")
    assert bench.kernel_source_digest("small_m") != d0


def test_committed_counters_match_the_sources():
    # every committed counter summary was taken on the kernels as they are
    for w in ("decode", "prefill", "13b", "70b"):
        for v in ("int8", "fp8"):
            assert bench.read_traffic(w, v) is not None, (w, v)


def test_every_counter_summary_names_the_current_gemm_sources():
    # the MFMA, LDS and memory-pipeline summaries of the large-M GEMM carry the
    # digest of the sources they were taken on; a kernel change marks them stale
    files = sorted(glob.glob(os.path.join(bench.PROFILES, "gemm_*_counters.txt")))
    assert len(files) >= 12
    for f in files:
        digests = [line.split(":", 1)[1].strip() for line in open(f)
                   if "kernel_source_digest:" in line and not line.startswith("#")]
        assert len(digests) == 1, f
        fam = "small_m" if os.path.basename(f) in ("gemm_decode_hbm_counters.txt",
                                                    "gemm_fp8_decode_hbm_counters.txt") else "large_m"
        assert digests[0] == bench.kernel_source_digest(fam), f


def test_quantize_pass_bytes():
    # each tensor read or written once
    b = bench.pass_bytes(8192, 8192, 28672)
    assert b["find_outliers"] == 2 * 8192 * 8192
    assert b["quantize_rowwise"] == 3 * 8192 * 8192 + 4 * 8192
    assert b["quantize_colwise"] == 3 * 8192 * 28672 + 4 * 28672


def test_rooflines():
    # decode: the GEMM kernel's bytes over its time, the call's over the step
    k, c = bench.rooflines(True, 0.010, 0.005, 16e6, 8e6, 0, 0)
    assert k["bound"] == "hbm" and math.isclose(k["achieved"], 1600.0)
    assert math.isclose(k["frac"], 0.2) and math.isclose(c["frac"], 0.2)
    # large M: fp16 flops weigh double against the int8 peak; the call's
    # fraction is the ideal time over the step time
    k, c = bench.rooflines(False, 0.2, 0.1, 0, 0, 250e9, 50e9)
    assert k["bound"] == "mfma" and math.isclose(k["achieved"], 3500.0)
    assert math.isclose(c["ideal_ms"], (250e9 / 5e15 + 50e9 / 2.5e15) * 1e3)
    assert math.isclose(c["frac"], c["ideal_ms"] / 0.2, rel_tol=1e-3)


def test_host_facts():
    f = bench.host_facts()
    assert f["nproc"] >= 1 and isinstance(f["cpu_model"], str)
