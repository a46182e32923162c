"""Host-side sanitizer runs (CPU only).

The CPU oracle is built with AddressSanitizer and UndefinedBehaviorSanitizer
(no recovery, float-to-int cast checks on) together with a C harness that
drives every oracle entry point over seeded shapes and the method's edge cases
(tests/sanitize/oracle_harness.c). The HIP library is built with the same
sanitizers on its host side and a C harness calls every entry point with
arguments that must be rejected before any HIP call, plus the size queries at
extreme shapes (tests/sanitize/abi_harness.c); that run hides every GPU.
Both harnesses exit non-zero, or the sanitizer aborts them, on any finding.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "bit_quantized_matmul_col_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def run(cmd, **kw):
    out = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert out.returncode == 0, f"{cmd[0]} failed ({out.returncode}):\n{out.stdout}\n{out.stderr}"
    return out


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_harness")
    run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", *SAN,
         "-fsanitize=float-cast-overflow", os.path.join(ROOT, "oracle", "llmint8_oracle.c"),
         os.path.join(HERE, "oracle_harness.c"), "-o", exe, "-lm"])
    out = run([exe], timeout=300)
    assert "cases clean" in out.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="ROCm compilers not installed")
def test_abi_argument_checks_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libllmint8_san.so")
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    host_san = []
    for flag in SAN:  # every sanitizer flag applies to the host pass only
        host_san += ["-Xarch_host", flag]
    run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", lib], timeout=900)
    rt = run([CLANG, "--print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    exe = str(tmp_path / "abi_harness")
    run([CLANG, "-O1", "-g", "-std=c11", *SAN, "-shared-libsan",
         "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "abi_harness.c"),
         "-L", str(tmp_path), "-lllmint8_san", f"-Wl,-rpath,{tmp_path}",
         f"-Wl,-rpath,{os.path.dirname(rt)}", "-o", exe])
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1", ASAN_OPTIONS="detect_leaks=0")
    out = run([exe], env=env, timeout=120)
    assert "abi harness: clean" in out.stdout
