"""The C-ABI library on the CPU: it loads, exports what include/llmint8.h
declares, and rejects bad arguments with the documented status before making
any HIP call. The rejection checks run in a child process with every GPU
hidden, so even a wrongly accepted call could not reach a device."""
import ctypes as C
import json
import math
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llmint8.h")
LIB = os.path.join(ROOT, "bit_quantized_matmul_col_amd", "libllmint8.so")



@pytest.fixture(autouse=True)
def _library(built_library):
    return built_library


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(llmint8_\w+)\s*\(", text)))


def test_header_is_plain_c():
    subprocess.run(["gcc", "-fsyntax-only", "-Wall", "-Werror", "-x", "c", HEADER], check=True)
    subprocess.run(["g++", "-fsyntax-only", "-Wall", "-Werror", "-x", "c++", HEADER], check=True)


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"llmint8_quantize_rowwise", "llmint8_quantize_colwise", "llmint8_find_outliers",
            "llmint8_linear"} <= set(names)
    lib = C.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = sorted(set(re.findall(r"\bT (llmint8_\w+)", out)))
    assert exported == names


CHILD = r"""
import ctypes as C, json, math, sys
L = C.CDLL(sys.argv[1])
p, i64, f32, sz = C.c_void_p, C.c_int64, C.c_float, C.c_size_t
L.llmint8_quantize_colwise.argtypes = [p, i64, i64, i64, p, p, p]
L.llmint8_find_outliers.argtypes = [p, i64, i64, i64, f32, p, p, p, sz, p]
L.llmint8_quantize_rowwise.argtypes = [p, i64, i64, i64, p, p, p, p, p]
L.llmint8_linear.argtypes = [p, i64, i64, i64, p, p, p, i64, i64, f32, p, i64, p, p, p, sz, p]
L.llmint8_linear_ex.argtypes = L.llmint8_linear.argtypes + [p]
L.llmint8_linear_noalloc.argtypes = [p, i64, i64, i64, p, p, p, i64, i64, f32, p, i64, p, p, p]
class Opts(C.Structure):
    _fields_ = [("struct_size", sz), ("b", p), ("e", p), ("outlier_weights", C.c_int),
                ("bias", p), ("y_col_absmax", p), ("x_col_absmax", p)]
L.llmint8_workspace_size.argtypes = [i64, i64, i64]
L.llmint8_workspace_size.restype = sz
L.llmint8_quantize_tensorwise.argtypes = [p, i64, i64, i64, p, p, p, sz, p]
L.llmint8_quantize_tensorwise_workspace_size.argtypes = [i64, i64]
L.llmint8_quantize_tensorwise_workspace_size.restype = sz
L.llmint8_linear_tensorwise.argtypes = [p, i64, i64, i64, p, p, i64, p, p, i64, p, p, p, sz, p]
L.llmint8_linear_tensorwise_workspace_size.argtypes = [i64, i64, i64]
L.llmint8_linear_tensorwise_workspace_size.restype = sz
L.llmint8_quantize_colwise_fp8.argtypes = [p, i64, i64, i64, p, p, p]
L.llmint8_quantize_rowwise_fp8.argtypes = [p, i64, i64, i64, p, p, p, p, p]
L.llmint8_linear_fp8.argtypes = L.llmint8_linear_ex.argtypes
L.llmint8_linear_fp8_workspace_size.argtypes = [i64, i64, i64]
L.llmint8_linear_fp8_workspace_size.restype = sz
L.llmint8_find_outliers_workspace_size.argtypes = [i64, i64]
L.llmint8_find_outliers_workspace_size.restype = sz
A, B, MIS = 0x100000, 0x200000, 0x300008   # 16-byte aligned fakes and a misaligned one
N0 = None
inf = math.inf
res = {}
def colwise(name, W=A, K=64, N=32, ldw=32, Wq=B, s=A):
    res[name] = L.llmint8_quantize_colwise(W, K, N, ldw, Wq, s, None)
def find(name, X=A, M=4, K=64, ldx=64, t=6.0, idx=B, cnt=B, ws=A, wsb=0):
    res[name] = L.llmint8_find_outliers(X, M, K, ldx, t, idx, cnt, ws, wsb, None)
def rowq(name, X=A, M=4, K=64, ldx=64, idx=N0, cnt=N0, Xq=B, m=A):
    res[name] = L.llmint8_quantize_rowwise(X, M, K, ldx, idx, cnt, Xq, m, None)
def linear(name, X=A, M=4, K=64, ldx=64, Wq=B, s=A, W=A, ldw=32, N=32, t=6.0, Y=B, ldy=32,
           cnt=N0, cdbg=N0, ws=A, wsb=0):
    res[name] = L.llmint8_linear(X, M, K, ldx, Wq, s, W, ldw, N, t, Y, ldy, cnt, cdbg, ws, wsb, None)
def linear_ex(name, size=C.sizeof(Opts), ow=0, bias=N0, ycm=N0, xcm=N0, W=A, t=6.0, wsb=0):
    o = Opts(size, None, None, ow, bias, ycm, xcm)
    res[name] = L.llmint8_linear_ex(A, 4, 64, 64, B, A, W, 32, 32, t, B, 32, None, None, A, wsb,
                                    None, C.byref(o))
def qtw(name, W=A, K=64, N=32, ldw=32, Wq=B, sw=A, ws=A, wsb=1 << 20):
    res[name] = L.llmint8_quantize_tensorwise(W, K, N, ldw, Wq, sw, ws, wsb, None)
def ltw(name, X=A, M=4, K=64, ldx=64, Wq=B, sw=A, N=32, bias=N0, Y=B, ldy=32, xa=N0, cdbg=N0,
        ws=A, wsb=0):
    res[name] = L.llmint8_linear_tensorwise(X, M, K, ldx, Wq, sw, N, bias, Y, ldy, xa, cdbg, ws,
                                            wsb, None)
def lfp8(name, size=C.sizeof(Opts), ow=0, W=A, t=6.0, M=4, cdbg=N0, wsb=0, opts=True):
    o = Opts(size, None, None, ow, None, None, None)
    res[name] = L.llmint8_linear_fp8(A, M, 64, 64, B, A, W, 32, 32, t, B, 32, None, cdbg, A, wsb,
                                     None, C.byref(o) if opts else None)
def noalloc(name, X=A, M=4, K=64, ldx=64, W=A, N=32, t=6.0, Y=B, ldy=32, cdbg=N0):
    res[name] = L.llmint8_linear_noalloc(X, M, K, ldx, B, A, W, 32 if N == 32 else N, N, t, Y,
                                         ldy, None, cdbg, None)
noalloc("noalloc_null_X", X=N0)
noalloc("noalloc_nan_threshold", t=math.nan)
noalloc("noalloc_null_W_finite_threshold", W=N0)
noalloc("noalloc_ldy_short", ldy=16)
noalloc("noalloc_misaligned_cdbg", cdbg=MIS)
noalloc("noalloc_K_too_big", K=133152, ldx=133152)
# a workspace beyond the 32 MiB scratch is refused before any HIP call
noalloc("noalloc_beyond_scratch", M=2048, K=4096, ldx=4096, N=11008, ldy=11008)
colwise("colwise_null_W", W=N0)
colwise("colwise_K0", K=0)
colwise("colwise_ld_short", ldw=16)
colwise("colwise_ld_not_mult8", ldw=36)
colwise("colwise_misaligned_W", W=MIS)
colwise("colwise_K_not_mult16", K=72)
colwise("colwise_N_not_mult8", N=30, ldw=32)
colwise("colwise_K_too_big", K=133152)
colwise("colwise_null_Wq", Wq=N0)
find("find_nan_threshold", t=math.nan)
find("find_null_idx", idx=N0)
find("find_no_workspace", ws=N0, wsb=1 << 20)
find("find_workspace_small", wsb=16)
find("find_neg_M", M=-1)
rowq("rowq_idx_without_count", idx=A)
rowq("rowq_null_Xq", Xq=N0)
rowq("rowq_misaligned_m", m=MIS)
rowq("rowq_K_too_big", K=200000, ldx=200000)
linear("linear_null_W_finite_threshold", W=N0)
linear("linear_null_W_inf_threshold_small_ws", W=N0, t=inf)
linear("linear_null_Y", Y=N0)
linear("linear_ldy_short", ldy=8)
linear("linear_nan_threshold", t=math.nan)
linear("linear_misaligned_cdbg", cdbg=MIS, wsb=1 << 40)
linear("linear_workspace_small", wsb=100)
linear("linear_K_not_mult16", K=40, ldx=48)
linear("linear_N0", N=0)
linear("linear_M0", M=0)
rowq("rowq_M0", M=0)
find("find_M0", M=0)
ltw("ltw_M0", M=0)
lfp8("lfp8_M0", M=0, wsb=1 << 40)
noalloc("noalloc_M0", M=0)
linear_ex("ex_struct_size_old", size=24)
linear_ex("ex_bad_outlier_weights", ow=2)
linear_ex("ex_misaligned_bias", bias=MIS)
linear_ex("ex_misaligned_y_col_absmax", ycm=MIS)
linear_ex("ex_misaligned_x_col_absmax", xcm=MIS)
linear_ex("ex_int8_weights_null_W_small_ws", ow=1, W=N0)
linear_ex("ex_fp16_weights_null_W", ow=0, W=N0)
qtw("qtw_null_sw", sw=N0)
qtw("qtw_misaligned_Wq", Wq=MIS)
qtw("qtw_K_not_mult16", K=40)
qtw("qtw_workspace_small", wsb=16)
qtw("qtw_no_workspace", ws=N0)
qtw("qtw_K_too_big", K=133152)
ltw("ltw_null_Wq", Wq=N0)
ltw("ltw_null_X", X=N0)
ltw("ltw_ldy_short", ldy=16)
ltw("ltw_misaligned_bias", bias=MIS)
ltw("ltw_misaligned_x_absmax", xa=MIS)
ltw("ltw_N_not_mult8", N=36, ldy=40)
ltw("ltw_workspace_small", wsb=64)
res["cfp8_null_Wq8"] = L.llmint8_quantize_colwise_fp8(A, 64, 32, 32, None, A, None)
res["cfp8_N_not_mult8"] = L.llmint8_quantize_colwise_fp8(A, 64, 30, 32, B, A, None)
res["rfp8_idx_without_count"] = L.llmint8_quantize_rowwise_fp8(A, 4, 64, 64, A, None, B, A, None)
res["rfp8_misaligned_Xq8"] = L.llmint8_quantize_rowwise_fp8(A, 4, 64, 64, None, None, MIS, A, None)
lfp8("lfp8_int8_weights_rejected", ow=1, wsb=1 << 40)
lfp8("lfp8_struct_size_old", size=24)
lfp8("lfp8_null_W_finite_threshold", W=N0)
lfp8("lfp8_null_W_inf_small_ws", W=N0, t=math.inf)
lfp8("lfp8_no_opts_small_ws", opts=False)
lfp8("lfp8_misaligned_cdbg", cdbg=MIS, wsb=1 << 40)
res["ws_fp8_small_m"] = L.llmint8_linear_fp8_workspace_size(8, 4096, 4096)
res["ws_int8_small_m"] = L.llmint8_workspace_size(8, 4096, 4096)
res["ws_size_ok"] = L.llmint8_workspace_size(32, 4096, 4096)
res["qtw_ws"] = L.llmint8_quantize_tensorwise_workspace_size(4096, 11008)
res["qtw_ws_bad"] = L.llmint8_quantize_tensorwise_workspace_size(4096, 0)
res["ltw_ws"] = L.llmint8_linear_tensorwise_workspace_size(2048, 4096, 11008)
res["ltw_ws_bad"] = L.llmint8_linear_tensorwise_workspace_size(2048, 133160, 64)
res["ws_size_prefill"] = L.llmint8_workspace_size(2048, 4096, 11008)
res["ws_fp8_prefill"] = L.llmint8_linear_fp8_workspace_size(2048, 4096, 11008)
res["ws_size_13b"] = L.llmint8_workspace_size(4096, 5120, 13824)
res["ws_fp8_13b"] = L.llmint8_linear_fp8_workspace_size(4096, 5120, 13824)
res["ws_size_70b"] = L.llmint8_workspace_size(8192, 8192, 28672)
res["ws_fp8_70b"] = L.llmint8_linear_fp8_workspace_size(8192, 8192, 28672)
res["ws_size_6tiles"] = L.llmint8_workspace_size(300, 8192, 520)
res["ws_fp8_6tiles"] = L.llmint8_linear_fp8_workspace_size(300, 8192, 520)
res["ws_size_768"] = L.llmint8_workspace_size(768, 8192, 8192)
res["ws_fp8_768"] = L.llmint8_linear_fp8_workspace_size(768, 8192, 8192)
res["ws_size_short_k"] = L.llmint8_workspace_size(300, 2048, 2048)
res["ws_fp8_short_k"] = L.llmint8_linear_fp8_workspace_size(300, 2048, 2048)
res["ws_size_short_k_many"] = L.llmint8_workspace_size(1024, 1024, 4096)
res["ws_fp8_short_k_many"] = L.llmint8_linear_fp8_workspace_size(1024, 1024, 4096)
res["ws_size_short_k_wide"] = L.llmint8_workspace_size(400, 2048, 8192)
res["ws_fp8_short_k_wide"] = L.llmint8_linear_fp8_workspace_size(400, 2048, 8192)
res["ws_size_bad"] = L.llmint8_workspace_size(0, 4096, 4096)
res["find_ws_ok"] = L.llmint8_find_outliers_workspace_size(8192, 8192)
res["find_ws_bad"] = L.llmint8_find_outliers_workspace_size(8, 133160)
print(json.dumps(res))
"""

EXPECTED = {
    "noalloc_null_X": 1, "noalloc_nan_threshold": 1, "noalloc_null_W_finite_threshold": 1,
    "noalloc_ldy_short": 1, "noalloc_misaligned_cdbg": 2, "noalloc_K_too_big": 3,
    "noalloc_beyond_scratch": 4,
    "colwise_null_W": 1, "colwise_K0": 1, "colwise_ld_short": 1, "colwise_ld_not_mult8": 2,
    "colwise_misaligned_W": 2, "colwise_K_not_mult16": 2, "colwise_N_not_mult8": 2,
    "colwise_K_too_big": 3, "colwise_null_Wq": 1,
    "find_nan_threshold": 1, "find_null_idx": 1, "find_no_workspace": 4,
    "find_workspace_small": 4, "find_neg_M": 1,
    "rowq_idx_without_count": 1, "rowq_null_Xq": 1, "rowq_misaligned_m": 2, "rowq_K_too_big": 3,
    "linear_null_W_finite_threshold": 1, "linear_null_W_inf_threshold_small_ws": 4,
    "linear_null_Y": 1, "linear_ldy_short": 1, "linear_nan_threshold": 1,
    "linear_misaligned_cdbg": 2, "linear_workspace_small": 4, "linear_K_not_mult16": 2,
    "linear_N0": 1, "linear_M0": 1, "rowq_M0": 1, "find_M0": 1, "ltw_M0": 1, "lfp8_M0": 1,
    "noalloc_M0": 1,
    "ex_struct_size_old": 1, "ex_bad_outlier_weights": 1, "ex_misaligned_bias": 2,
    "ex_misaligned_y_col_absmax": 2, "ex_misaligned_x_col_absmax": 2,
    # int8 outlier weights need no fp16 W at any threshold: the call reaches the
    # workspace check
    "ex_int8_weights_null_W_small_ws": 4, "ex_fp16_weights_null_W": 1,
    "qtw_null_sw": 1, "qtw_misaligned_Wq": 2, "qtw_K_not_mult16": 2, "qtw_workspace_small": 4,
    "qtw_no_workspace": 4, "qtw_K_too_big": 3,
    "ltw_null_Wq": 1, "ltw_null_X": 1, "ltw_ldy_short": 1, "ltw_misaligned_bias": 2,
    "ltw_misaligned_x_absmax": 2, "ltw_N_not_mult8": 2, "ltw_workspace_small": 4,
    "cfp8_null_Wq8": 1, "cfp8_N_not_mult8": 2, "rfp8_idx_without_count": 1,
    "rfp8_misaligned_Xq8": 2,
    "lfp8_int8_weights_rejected": 1, "lfp8_struct_size_old": 1,
    "lfp8_null_W_finite_threshold": 1, "lfp8_null_W_inf_small_ws": 4,
    "lfp8_no_opts_small_ws": 4, "lfp8_misaligned_cdbg": 2,
}


def test_invalid_arguments_are_rejected_before_any_hip_call():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    out = subprocess.run([sys.executable, "-c", CHILD, LIB], capture_output=True, text=True,
                         env=env, timeout=120)
    assert out.returncode == 0, out.stderr
    res = json.loads(out.stdout.strip().splitlines()[-1])
    for name, code in EXPECTED.items():
        assert res[name] == code, (name, res[name], code)
    # small M: int8 + fp16 copies of X and the split-K partial sums
    assert res["ws_size_ok"] >= 32 * 4096 * 3 + 32 * 4096 * 4
    # large M: int8 + fp16 copies of X and room for a compacted Wq
    assert res["ws_size_prefill"] >= 2048 * 4096 * 3 + 11008 * 4096
    assert res["ws_size_bad"] == 0
    assert res["find_ws_ok"] > 0 and res["find_ws_bad"] == 0
    # per-tensor layer: the column maxima for W; the int8 copy of X and the scales
    assert res["qtw_ws"] >= 11008 * 4 and res["qtw_ws_bad"] == 0
    assert res["ltw_ws"] >= 2048 * 4096 + 2048 * 4 + 11008 * 4 and res["ltw_ws_bad"] == 0
    # FP8 layer: the same layouts as the int8 layer
    assert res["ws_fp8_small_m"] == res["ws_int8_small_m"] > 0
    # Large M: when a launch has fewer tiles than the 256 CUs, the int8 layer
    # also holds the split-K GEMM's arrival counters (256-byte aligned) and one
    # slot of int32 sums per part of each tile (bm x 256 x 4 bytes).
    # 300 x 8192 x 520: 3 x 3 tiles of 128 x 256 in 4 parts of 16 stages of 128
    # bytes of k. The 7B prefill, 13b and 70b shapes have no split.
    def split_room(tiles, parts, bm=128):
        return (tiles * 4 + 255) // 256 * 256 + tiles * parts * bm * 256 * 4
    assert res["ws_size_prefill"] == res["ws_fp8_prefill"]
    assert res["ws_size_13b"] == res["ws_fp8_13b"]
    assert res["ws_size_70b"] == res["ws_fp8_70b"]
    assert res["ws_size_6tiles"] - res["ws_fp8_6tiles"] == split_room(9, 4)
    # 768 x 8192 x 8192: 192 tiles of 128 x 256 do not split, 96 of 256 x 256 do (2 parts)
    assert res["ws_size_768"] - res["ws_fp8_768"] == split_room(96, 2, 256)
    # short k ranges (K <= 2048, at most 16 stages): 128 x 256 tiles only, parts of
    # at least 4 stages up to 96 tiles, else of at least 8
    assert res["ws_size_short_k"] - res["ws_fp8_short_k"] == split_room(24, 4)
    assert res["ws_size_short_k_many"] == res["ws_fp8_short_k_many"]  # 128 tiles of 8 stages
    assert res["ws_size_short_k_wide"] - res["ws_fp8_short_k_wide"] == split_room(128, 2)


def test_status_strings():
    lib = C.CDLL(LIB)
    lib.llmint8_status_string.restype = C.c_char_p
    for code in range(6):
        assert lib.llmint8_status_string(code).decode().startswith("LLMINT8_")
    assert b"unknown" in lib.llmint8_status_string(99)


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import bit_quantized_matmul_col_amd as b
    monkeypatch.setattr(b, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(b, "_lib", None)
    with pytest.raises(ImportError):
        b.lib()


def test_library_matches_its_build_record(monkeypatch):
    # the binding loads the in-tree library only if it is the recorded build of
    # the sources as they are now
    import bit_quantized_matmul_col_amd as b
    from bit_quantized_matmul_col_amd import build
    rec = build.check_record()
    assert rec["source_digest"] == build.source_digest()
    assert "--offload-arch=gfx950" in rec["flags"] and "-packed-fp32-ops" in rec["flags"]
    monkeypatch.setattr(b, "_lib", None)
    monkeypatch.setattr(build, "source_digest", lambda: "0" * 64)
    with pytest.raises(ImportError, match="different sources"):
        b.lib()
