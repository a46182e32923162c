"""ctypes wrapper around the plain-C oracle (test infrastructure only).

Each function calls one step of llmint8_oracle.c on numpy arrays. fp16 inputs
are passed as their IEEE binary16 bit patterns (numpy float16 or uint16).
`linear` composes the steps in the order the pages give them: outlier columns,
row-wise quantization of X, int8 matmul, 16-bit outlier product, merge.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        lib = C.CDLL(_build.LIB)
        p = C.c_void_p
        i64 = C.c_int64
        lib.ora_half_to_float.argtypes = [p, i64, p]
        lib.ora_half_to_float.restype = None
        lib.ora_quantize_colwise.argtypes = [p, i64, i64, i64, p, p]
        lib.ora_quantize_colwise.restype = None
        lib.ora_find_outliers.argtypes = [p, i64, i64, i64, C.c_float, p]
        lib.ora_find_outliers.restype = C.c_int32
        lib.ora_quantize_rowwise.argtypes = [p, i64, i64, i64, p, C.c_int32, p, p]
        lib.ora_quantize_rowwise.restype = None
        lib.ora_gemm_i8.argtypes = [p, p, i64, i64, i64, p]
        lib.ora_gemm_i8.restype = C.c_int
        lib.ora_merge.argtypes = [p, p, p, p, i64, p, i64, p, C.c_int32, i64, i64, p]
        lib.ora_merge.restype = None
        lib.ora_merge_int8w.argtypes = [p, p, p, p, i64, p, i64, p, C.c_int32, i64, i64, p]
        lib.ora_merge_int8w.restype = None
        lib.ora_quantize_tensorwise.argtypes = [p, i64, i64, i64, p]
        lib.ora_quantize_tensorwise.restype = C.c_float
        lib.ora_linear_tensorwise.argtypes = [p, i64, i64, i64, p, C.c_float, i64, p, p, p]
        lib.ora_linear_tensorwise.restype = C.c_float
        lib.ora_add_bias.argtypes = [p, i64, i64, p]
        lib.ora_add_bias.restype = None
        lib.ora_e4m3_encode_array.argtypes = [p, i64, p]
        lib.ora_e4m3_encode_array.restype = None
        lib.ora_e4m3_value_array.argtypes = [p, i64, p]
        lib.ora_e4m3_value_array.restype = None
        lib.ora_quantize_colwise_fp8.argtypes = [p, i64, i64, i64, p, p]
        lib.ora_quantize_colwise_fp8.restype = None
        lib.ora_quantize_rowwise_fp8.argtypes = [p, i64, i64, i64, p, C.c_int32, p, p]
        lib.ora_quantize_rowwise_fp8.restype = None
        lib.ora_gemm_fp8.argtypes = [p, p, i64, i64, i64, p]
        lib.ora_gemm_fp8.restype = None
        lib.ora_merge_fp8.argtypes = [p, p, p, p, i64, p, i64, p, C.c_int32, i64, i64, p]
        lib.ora_merge_fp8.restype = None
        _lib = lib
    return _lib


def _bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("fp16 input must be float16 or uint16 bit patterns")
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def half_to_float(h: np.ndarray) -> np.ndarray:
    h = _bits(h)
    out = np.empty(h.shape, np.float32)
    _load().ora_half_to_float(_ptr(h), h.size, _ptr(out))
    return out


def quantize_colwise(W: np.ndarray):
    """W fp16 [K, N] -> (Wq int8 [N, K], s float32 [N])."""
    W = _bits(W)
    K, N = W.shape
    Wq = np.empty((N, K), np.int8)
    s = np.empty(N, np.float32)
    _load().ora_quantize_colwise(_ptr(W), K, N, N, _ptr(Wq), _ptr(s))
    return Wq, s


def find_outliers(X: np.ndarray, threshold: float) -> np.ndarray:
    """X fp16 [M, K] -> ascending int32 outlier column indices."""
    X = _bits(X)
    M, K = X.shape
    idx = np.empty(max(K, 1), np.int32)
    n = _load().ora_find_outliers(_ptr(X), M, K, K, float(threshold), _ptr(idx))
    return idx[:n].copy()


def quantize_rowwise(X: np.ndarray, idx: np.ndarray | None = None):
    """X fp16 [M, K], outlier columns -> (Xq int8 [M, K], m float32 [M])."""
    X = _bits(X)
    M, K = X.shape
    idx = np.ascontiguousarray(np.zeros(0, np.int32) if idx is None else idx, dtype=np.int32)
    Xq = np.empty((M, K), np.int8)
    m = np.empty(M, np.float32)
    _load().ora_quantize_rowwise(_ptr(X), M, K, K, _ptr(idx), int(idx.size), _ptr(Xq), _ptr(m))
    return Xq, m


def gemm_i8(Xq: np.ndarray, Wq: np.ndarray) -> np.ndarray:
    """Xq int8 [M, K], Wq int8 [N, K] -> C int32 [M, N] = Xq . Wq^T."""
    Xq = np.ascontiguousarray(Xq, dtype=np.int8)
    Wq = np.ascontiguousarray(Wq, dtype=np.int8)
    M, K = Xq.shape
    N, K2 = Wq.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    Cm = np.empty((M, N), np.int32)
    if _load().ora_gemm_i8(_ptr(Xq), _ptr(Wq), M, N, K, _ptr(Cm)):
        raise OverflowError("int32 accumulator overflow")
    return Cm


def merge(Cm: np.ndarray, m: np.ndarray, s: np.ndarray, X: np.ndarray, W: np.ndarray,
          idx: np.ndarray) -> np.ndarray:
    """Dequantize C and add the fp16 outlier product -> Y float64 [M, N]."""
    X = _bits(X)
    W = _bits(W)
    Cm = np.ascontiguousarray(Cm, dtype=np.int32)
    m = np.ascontiguousarray(m, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    M, N = Cm.shape
    Y = np.empty((M, N), np.float64)
    _load().ora_merge(_ptr(Cm), _ptr(m), _ptr(s), _ptr(X), X.shape[1], _ptr(W), W.shape[1],
                      _ptr(idx), int(idx.size), M, N, _ptr(Y))
    return Y


def merge_int8w(Cm: np.ndarray, m: np.ndarray, s: np.ndarray, X: np.ndarray, Wq: np.ndarray,
                idx: np.ndarray) -> np.ndarray:
    """Dequantize C and add the outlier product with W_O = Wq . s / 127 -> Y float64."""
    X = _bits(X)
    Cm = np.ascontiguousarray(Cm, dtype=np.int32)
    m = np.ascontiguousarray(m, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    Wq = np.ascontiguousarray(Wq, dtype=np.int8)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    M, N = Cm.shape
    Y = np.empty((M, N), np.float64)
    _load().ora_merge_int8w(_ptr(Cm), _ptr(m), _ptr(s), _ptr(X), X.shape[1], _ptr(Wq),
                            Wq.shape[1], _ptr(idx), int(idx.size), M, N, _ptr(Y))
    return Y


def add_bias(Y: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """Y float64 [M, N] + fp16 bias [N] (a new array)."""
    Y = np.array(Y, dtype=np.float64, order="C")
    b = _bits(bias)
    _load().ora_add_bias(_ptr(Y), Y.shape[0], Y.shape[1], _ptr(b))
    return Y


def quantize_tensorwise(W: np.ndarray):
    """W fp16 [K, N] -> (Wq int8 [N, K], absmax float32 over all of W)."""
    W = _bits(W)
    K, N = W.shape
    Wq = np.empty((N, K), np.int8)
    sw = _load().ora_quantize_tensorwise(_ptr(W), K, N, N, _ptr(Wq))
    return Wq, np.float32(sw)


def linear_tensorwise(X: np.ndarray, Wq: np.ndarray, sw, bias=None) -> dict:
    """The traditional per-tensor int8 layer (no outlier decomposition)."""
    X = _bits(X)
    Wq = np.ascontiguousarray(Wq, dtype=np.int8)
    M, K = X.shape
    N = Wq.shape[0]
    Xq = np.empty((M, K), np.int8)
    Cm = np.empty((M, N), np.int32)
    Y = np.empty((M, N), np.float64)
    sx = _load().ora_linear_tensorwise(_ptr(X), M, K, K, _ptr(Wq), float(sw), N, _ptr(Xq),
                                       _ptr(Cm), _ptr(Y))
    if bias is not None:
        Y = add_bias(Y, bias)
    return dict(Xq=Xq, sx=np.float32(sx), C=Cm, Y=Y)


def _merge_mode(Cm, m, s, X, W, Wq, idx, outlier_weights):
    if outlier_weights == "fp16":
        return merge(Cm, m, s, X, W, idx)
    if outlier_weights == "int8":
        return merge_int8w(Cm, m, s, X, Wq, idx)
    raise ValueError("outlier_weights is 'fp16' or 'int8'")


def linear(X: np.ndarray, W: np.ndarray, threshold: float, Wq=None, s=None, *,
           outlier_weights: str = "fp16", bias=None) -> dict:
    """The whole layer. Returns every intermediate the GPU path also exposes.

    outlier_weights "fp16" takes the outlier rows of W as given; "int8" takes
    them from the dequantized codes Wq * s / 127 (W is then only needed to
    quantize, if Wq and s are not passed). bias, if given, is added last."""
    if Wq is None or s is None:
        Wq, s = quantize_colwise(W)
    idx = find_outliers(X, threshold)
    Xq, m = quantize_rowwise(X, idx)
    Cm = gemm_i8(Xq, Wq)
    Y = _merge_mode(Cm, m, s, X, W, Wq, idx, outlier_weights)
    if bias is not None:
        Y = add_bias(Y, bias)
    return dict(idx=idx, Xq=Xq, m=m, Wq=Wq, s=s, C=Cm, Y=Y)


def linear_rows(X: np.ndarray, W: np.ndarray, threshold: float, rows, Wq=None, s=None, *,
                outlier_weights: str = "fp16", bias=None) -> dict:
    """The layer's results for selected rows of X only.

    The outlier set is a property of the whole X, so it is found on all rows;
    every later step is independent per row and runs on the selected rows.
    """
    if Wq is None or s is None:
        Wq, s = quantize_colwise(W)
    rows = np.asarray(rows, dtype=np.int64)
    idx = find_outliers(X, threshold)
    Xs = np.ascontiguousarray(_bits(X)[rows])
    Xq, m = quantize_rowwise(Xs, idx)
    Cm = gemm_i8(Xq, Wq)
    Y = _merge_mode(Cm, m, s, Xs, W, Wq, idx, outlier_weights)
    if bias is not None:
        Y = add_bias(Y, bias)
    return dict(rows=rows, idx=idx, Xq=Xq, m=m, Wq=Wq, s=s, C=Cm, Y=Y)


# ---- FP8 (E4M3) variant --------------------------------------------------------------

def e4m3_encode(t: np.ndarray) -> np.ndarray:
    """fp32 values -> nearest E4M3 codes (uint8), ties to even, |t| > 448 -> 448."""
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, np.uint8)
    _load().ora_e4m3_encode_array(_ptr(t), t.size, _ptr(out))
    return out


def e4m3_value(c: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) -> their values (float64; NaN for 0x7f / 0xff)."""
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().ora_e4m3_value_array(_ptr(c), c.size, _ptr(out))
    return out


def quantize_colwise_fp8(W: np.ndarray):
    """W fp16 [K, N] -> (Wq8 uint8 E4M3 codes [N, K], s float32 [N])."""
    W = _bits(W)
    K, N = W.shape
    Wq = np.empty((N, K), np.uint8)
    s = np.empty(N, np.float32)
    _load().ora_quantize_colwise_fp8(_ptr(W), K, N, N, _ptr(Wq), _ptr(s))
    return Wq, s


def quantize_rowwise_fp8(X: np.ndarray, idx: np.ndarray | None = None):
    """X fp16 [M, K], outlier columns -> (Xq8 uint8 E4M3 codes [M, K], m float32 [M])."""
    X = _bits(X)
    M, K = X.shape
    idx = np.ascontiguousarray(np.zeros(0, np.int32) if idx is None else idx, dtype=np.int32)
    Xq = np.empty((M, K), np.uint8)
    m = np.empty(M, np.float32)
    _load().ora_quantize_rowwise_fp8(_ptr(X), M, K, K, _ptr(idx), int(idx.size), _ptr(Xq),
                                     _ptr(m))
    return Xq, m


def gemm_fp8(Xq8: np.ndarray, Wq8: np.ndarray) -> np.ndarray:
    """E4M3 codes Xq8 [M, K] and Wq8 [N, K] -> C float64 [M, N] (exact products)."""
    Xq8 = np.ascontiguousarray(Xq8, dtype=np.uint8)
    Wq8 = np.ascontiguousarray(Wq8, dtype=np.uint8)
    M, K = Xq8.shape
    N, K2 = Wq8.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    Cm = np.empty((M, N), np.float64)
    _load().ora_gemm_fp8(_ptr(Xq8), _ptr(Wq8), M, N, K, _ptr(Cm))
    return Cm


def merge_fp8(Cm, m, s, X, W, idx) -> np.ndarray:
    """Y = C m s / 448^2 + the fp16 outlier product -> float64 [M, N]."""
    X = _bits(X)
    W = _bits(W)
    Cm = np.ascontiguousarray(Cm, dtype=np.float64)
    m = np.ascontiguousarray(m, dtype=np.float32)
    s = np.ascontiguousarray(s, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    M, N = Cm.shape
    Y = np.empty((M, N), np.float64)
    _load().ora_merge_fp8(_ptr(Cm), _ptr(m), _ptr(s), _ptr(X), X.shape[1], _ptr(W), W.shape[1],
                          _ptr(idx), int(idx.size), M, N, _ptr(Y))
    return Y


def linear_fp8(X: np.ndarray, W: np.ndarray, threshold: float, Wq8=None, s=None,
               rows=None) -> dict:
    """The FP8 variant of the layer: the same outlier split, E4M3 codes with
    absmax scaling to 448 for the rest. With `rows`, results for those rows of X
    only (the outlier set is still found on all of X)."""
    if Wq8 is None or s is None:
        Wq8, s = quantize_colwise_fp8(W)
    idx = find_outliers(X, threshold)
    Xs = _bits(X) if rows is None else np.ascontiguousarray(_bits(X)[np.asarray(rows)])
    Xq8, m = quantize_rowwise_fp8(Xs, idx)
    Cm = gemm_fp8(Xq8, Wq8)
    Y = merge_fp8(Cm, m, s, Xs, W, idx)
    return dict(idx=idx, Xq=Xq8, m=m, Wq=Wq8, s=s, C=Cm, Y=Y)
