"""MI355X (gfx950) LLM.int8() mixed-precision linear layer.

Thin ctypes binding over libllmint8.so (include/llmint8.h). The Python
functions carry the C entry points' names and do argument marshalling only:
they check dtypes/devices, allocate outputs as torch tensors (PyTorch supplies
device memory and the current HIP stream) and call the library, which runs
every step of the layer in its own HIP kernels. There is no CPU fallback: if
the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libllmint8.so")
_DEFAULT_LIB = LIB_PATH
# filled when the library is loaded: source digest, compiler and flags it was built with
build_record: dict = {}

LLMINT8_OK = 0
LLMINT8_ERR_INVALID_ARG = 1
LLMINT8_ERR_UNSUPPORTED = 2
LLMINT8_ERR_OVERFLOW = 3
LLMINT8_ERR_WORKSPACE = 4
LLMINT8_ERR_HIP = 5
LLMINT8_MAX_K = 133144
LLMINT8_NOALLOC_SCRATCH_BYTES = 32 << 20

_lib = None


LLMINT8_OUTLIER_W_FP16 = 0
LLMINT8_OUTLIER_W_INT8 = 1


class LinearOpts(C.Structure):
    """Mirror of llmint8_linear_opts."""
    _fields_ = [("struct_size", C.c_size_t), ("gemm_begin_event", C.c_void_p),
                ("gemm_end_event", C.c_void_p), ("outlier_weights", C.c_int),
                ("bias", C.c_void_p), ("y_col_absmax", C.c_void_p),
                ("x_col_absmax", C.c_void_p)]

    def __init__(self, **kw):
        super().__init__(struct_size=C.sizeof(LinearOpts), **kw)


class Llmint8Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def lib() -> C.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        if LIB_PATH == _DEFAULT_LIB:
            # the in-tree library must be the recorded build of the current sources
            from . import build as _build
            build_record.update(_build.check_record())
        L = C.CDLL(LIB_PATH)
        p, i64, f32, sz = C.c_void_p, C.c_int64, C.c_float, C.c_size_t
        L.llmint8_quantize_colwise.argtypes = [p, i64, i64, i64, p, p, p]
        L.llmint8_find_outliers_workspace_size.argtypes = [i64, i64]
        L.llmint8_find_outliers_workspace_size.restype = sz
        L.llmint8_find_outliers.argtypes = [p, i64, i64, i64, f32, p, p, p, sz, p]
        L.llmint8_quantize_rowwise.argtypes = [p, i64, i64, i64, p, p, p, p, p]
        L.llmint8_workspace_size.argtypes = [i64, i64, i64]
        L.llmint8_workspace_size.restype = sz
        L.llmint8_linear.argtypes = [p, i64, i64, i64, p, p, p, i64, i64, f32, p, i64, p, p, p,
                                     sz, p]
        L.llmint8_linear_ex.argtypes = L.llmint8_linear.argtypes + [p]
        L.llmint8_linear_noalloc.argtypes = [p, i64, i64, i64, p, p, p, i64, i64, f32, p, i64,
                                             p, p, p]
        L.llmint8_quantize_tensorwise_workspace_size.argtypes = [i64, i64]
        L.llmint8_quantize_tensorwise_workspace_size.restype = sz
        L.llmint8_quantize_tensorwise.argtypes = [p, i64, i64, i64, p, p, p, sz, p]
        L.llmint8_linear_tensorwise_workspace_size.argtypes = [i64, i64, i64]
        L.llmint8_linear_tensorwise_workspace_size.restype = sz
        L.llmint8_linear_tensorwise.argtypes = [p, i64, i64, i64, p, p, i64, p, p, i64, p, p, p,
                                                sz, p]
        L.llmint8_quantize_colwise_fp8.argtypes = [p, i64, i64, i64, p, p, p]
        L.llmint8_quantize_rowwise_fp8.argtypes = [p, i64, i64, i64, p, p, p, p, p]
        L.llmint8_linear_fp8_workspace_size.argtypes = [i64, i64, i64]
        L.llmint8_linear_fp8_workspace_size.restype = sz
        L.llmint8_linear_fp8.argtypes = L.llmint8_linear_ex.argtypes
        L.llmint8_status_string.argtypes = [C.c_int]
        L.llmint8_status_string.restype = C.c_char_p
        for name in ("llmint8_quantize_colwise", "llmint8_find_outliers",
                     "llmint8_quantize_rowwise", "llmint8_linear", "llmint8_linear_ex",
                     "llmint8_linear_noalloc",
                     "llmint8_quantize_tensorwise", "llmint8_linear_tensorwise",
                     "llmint8_quantize_colwise_fp8", "llmint8_quantize_rowwise_fp8",
                     "llmint8_linear_fp8"):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def llmint8_status_string(status: int) -> str:
    return lib().llmint8_status_string(int(status)).decode()


def _check(status: int):
    if status != LLMINT8_OK:
        raise Llmint8Error(status, llmint8_status_string(status))


def _stream(t: torch.Tensor):
    return C.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(None)


def _need(t: torch.Tensor, name: str, dtype, ndim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    if ndim == 2 and t.numel() == 0:
        # the C calls take M, K, N >= 1 (LLMINT8_ERR_INVALID_ARG otherwise)
        raise ValueError(f"{name} is empty ({tuple(t.shape)}); every dimension must be >= 1")


def _need_shape(t: torch.Tensor, name: str, shape: tuple, contiguous: bool = False):
    """Reject a buffer whose shape differs from the one the kernels write (or
    read) with the pitches the call passes: they would run past its end."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_vec(t: torch.Tensor, name: str, dtype, n: int, exact: bool = True):
    """A contiguous vector of n elements (at least n when exact is False)."""
    _need(t, name, dtype)
    if not t.is_contiguous() or (t.numel() != n if exact else t.numel() < n):
        raise ValueError(f"{name} must be a contiguous vector of {'' if exact else 'at least '}"
                         f"{n} elements, got {tuple(t.shape)}")


def _ws(workspace: torch.Tensor):
    """(pointer, size in bytes) of a caller-supplied device workspace."""
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise ValueError("workspace must be a GPU tensor")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def _ld(t: torch.Tensor, name: str) -> int:
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")
    # a single row has no meaningful row stride (numpy and torch may report 0)
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def llmint8_quantize_colwise(W: torch.Tensor):
    """fp16 W [K, N] -> (Wq int8 [N, K], col_absmax fp32 [N])."""
    _need(W, "W", torch.float16, 2)
    K, N = W.shape
    Wq = torch.empty((N, K), dtype=torch.int8, device=W.device)
    s = torch.empty((N,), dtype=torch.float32, device=W.device)
    _check(lib().llmint8_quantize_colwise(_ptr(W), K, N, _ld(W, "W"), _ptr(Wq), _ptr(s),
                                          _stream(W)))
    return Wq, s


def llmint8_find_outliers_workspace_size(M: int, K: int) -> int:
    return int(lib().llmint8_find_outliers_workspace_size(M, K))


def llmint8_find_outliers(X: torch.Tensor, threshold: float = 6.0, workspace=None):
    """fp16 X [M, K] -> (idx int32 [K] ascending in idx[:count], count int32 [1]) on device."""
    _need(X, "X", torch.float16, 2)
    M, K = X.shape
    idx = torch.empty((K,), dtype=torch.int32, device=X.device)
    count = torch.empty((1,), dtype=torch.int32, device=X.device)
    need = llmint8_find_outliers_workspace_size(M, K)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=X.device)
    _check(lib().llmint8_find_outliers(_ptr(X), M, K, _ld(X, "X"), float(threshold), _ptr(idx),
                                       _ptr(count), *_ws(workspace),
                                       _stream(X)))
    return idx, count


def llmint8_quantize_rowwise(X: torch.Tensor, idx: torch.Tensor | None = None,
                             count: torch.Tensor | None = None):
    """fp16 X [M, K] (+ outlier idx/count on device) -> (Xq int8 [M, K], row_absmax fp32 [M])."""
    _need(X, "X", torch.float16, 2)
    if (idx is None) != (count is None):
        raise ValueError("idx and count go together")
    M, K = X.shape
    if idx is not None:
        _need_vec(idx, "idx", torch.int32, K, exact=False)
        _need_vec(count, "count", torch.int32, 1, exact=False)
    Xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    m = torch.empty((M,), dtype=torch.float32, device=X.device)
    _check(lib().llmint8_quantize_rowwise(_ptr(X), M, K, _ld(X, "X"), _ptr(idx), _ptr(count),
                                          _ptr(Xq), _ptr(m), _stream(X)))
    return Xq, m


def llmint8_workspace_size(M: int, K: int, N: int) -> int:
    return int(lib().llmint8_workspace_size(M, K, N))


def llmint8_linear(X: torch.Tensor, Wq: torch.Tensor, col_absmax: torch.Tensor,
                   W: torch.Tensor | None, threshold: float = 6.0, *, Y=None, workspace=None,
                   outlier_count: torch.Tensor | None = None,
                   C_debug: torch.Tensor | None = None,
                   opts: LinearOpts | None = None, outlier_weights: str = "fp16",
                   bias: torch.Tensor | None = None,
                   y_col_absmax: torch.Tensor | None = None,
                   x_col_absmax: torch.Tensor | None = None) -> torch.Tensor:
    """The whole LLM.int8() layer: fp16 X [M, K] with Wq [N, K], col_absmax [N] and the
    fp16 weight W [K, N] (rows in the outlier set feed the 16-bit product) -> fp16 Y [M, N].

    outlier_weights "int8" takes the outlier rows from the codes Wq * col_absmax / 127
    instead (W may then be None); bias [N] fp16 is added to Y; y_col_absmax [N] fp32
    receives max_i |Y[i, n]|; x_col_absmax [K] fp32, if given, is taken as X's column
    absmax and decides the outlier columns without a scan of X."""
    _need(X, "X", torch.float16, 2)
    _need(Wq, "Wq", torch.int8, 2)
    M, K = X.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or not Wq.is_contiguous():
        raise ValueError("Wq must be contiguous [N, K]")
    _need_vec(col_absmax, "col_absmax", torch.float32, N)
    if outlier_weights not in ("fp16", "int8"):
        raise ValueError("outlier_weights is 'fp16' or 'int8'")
    if W is not None:
        _need(W, "W", torch.float16, 2)
        if tuple(W.shape) != (K, N):
            raise ValueError("W must be [K, N]")
    elif outlier_weights == "fp16" and not (math.isinf(threshold) and threshold > 0):
        raise ValueError("W may be omitted only with threshold=+inf or int8 outlier weights")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _need(Y, "Y", torch.float16, 2)
    _need_shape(Y, "Y", (M, N))
    if outlier_count is not None:
        _need_vec(outlier_count, "outlier_count", torch.int32, 1, exact=False)
    if C_debug is not None:
        _need(C_debug, "C_debug", torch.int32)
        _need_shape(C_debug, "C_debug", (M, N), contiguous=True)
    for name, t, dt, n in (("bias", bias, torch.float16, N),
                           ("y_col_absmax", y_col_absmax, torch.float32, N),
                           ("x_col_absmax", x_col_absmax, torch.float32, K)):
        if t is not None:
            _need(t, name, dt, 1)
            if t.numel() != n or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous vector of {n}")
    if workspace is None:
        workspace = torch.empty((llmint8_workspace_size(M, K, N),), dtype=torch.uint8,
                                device=X.device)
    extra = (outlier_weights != "fp16" or bias is not None or y_col_absmax is not None
             or x_col_absmax is not None)
    if extra:
        o = LinearOpts(gemm_begin_event=opts.gemm_begin_event if opts else None,
                       gemm_end_event=opts.gemm_end_event if opts else None,
                       outlier_weights=(LLMINT8_OUTLIER_W_INT8 if outlier_weights == "int8"
                                        else LLMINT8_OUTLIER_W_FP16),
                       bias=bias.data_ptr() if bias is not None else None,
                       y_col_absmax=y_col_absmax.data_ptr() if y_col_absmax is not None else None,
                       x_col_absmax=x_col_absmax.data_ptr() if x_col_absmax is not None else None)
        opts = o
    args = (_ptr(X), M, K, _ld(X, "X"), _ptr(Wq), _ptr(col_absmax), _ptr(W),
            _ld(W, "W") if W is not None else N, N, float(threshold), _ptr(Y), _ld(Y, "Y"),
            _ptr(outlier_count), _ptr(C_debug), *_ws(workspace), _stream(X))
    if opts is None:
        _check(lib().llmint8_linear(*args))
    else:
        _check(lib().llmint8_linear_ex(*args, C.byref(opts)))
    return Y


def llmint8_linear_noalloc(X: torch.Tensor, Wq: torch.Tensor, col_absmax: torch.Tensor,
                           W: torch.Tensor | None, threshold: float = 6.0, *, Y=None,
                           outlier_count: torch.Tensor | None = None,
                           C_debug: torch.Tensor | None = None) -> torch.Tensor:
    """llmint8_linear without a workspace: the library's per-GPU scratch array
    (LLMINT8_NOALLOC_SCRATCH_BYTES) takes its place, so the C call allocates
    nothing (pass Y to allocate nothing here either). Shapes whose workspace
    would exceed the scratch raise Llmint8Error (LLMINT8_ERR_WORKSPACE); calls
    that may overlap on one GPU race on the shared scratch."""
    _need(X, "X", torch.float16, 2)
    _need(Wq, "Wq", torch.int8, 2)
    M, K = X.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or not Wq.is_contiguous():
        raise ValueError("Wq must be contiguous [N, K]")
    _need_vec(col_absmax, "col_absmax", torch.float32, N)
    if W is not None:
        _need(W, "W", torch.float16, 2)
        if tuple(W.shape) != (K, N):
            raise ValueError("W must be [K, N]")
    elif not (math.isinf(threshold) and threshold > 0):
        raise ValueError("W may be omitted only with threshold=+inf")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _need(Y, "Y", torch.float16, 2)
    _need_shape(Y, "Y", (M, N))
    if outlier_count is not None:
        _need_vec(outlier_count, "outlier_count", torch.int32, 1, exact=False)
    if C_debug is not None:
        _need(C_debug, "C_debug", torch.int32)
        _need_shape(C_debug, "C_debug", (M, N), contiguous=True)
    _check(lib().llmint8_linear_noalloc(
        _ptr(X), M, K, _ld(X, "X"), _ptr(Wq), _ptr(col_absmax), _ptr(W),
        _ld(W, "W") if W is not None else N, N, float(threshold), _ptr(Y), _ld(Y, "Y"),
        _ptr(outlier_count), _ptr(C_debug), _stream(X)))
    return Y


def llmint8_quantize_tensorwise_workspace_size(K: int, N: int) -> int:
    return int(lib().llmint8_quantize_tensorwise_workspace_size(K, N))


def llmint8_quantize_tensorwise(W: torch.Tensor, workspace=None):
    """fp16 W [K, N] -> (Wq int8 [N, K], w_absmax fp32 [1]): one scale for all of W."""
    _need(W, "W", torch.float16, 2)
    K, N = W.shape
    Wq = torch.empty((N, K), dtype=torch.int8, device=W.device)
    sw = torch.empty((1,), dtype=torch.float32, device=W.device)
    if workspace is None:
        workspace = torch.empty((max(llmint8_quantize_tensorwise_workspace_size(K, N), 1),),
                                dtype=torch.uint8, device=W.device)
    _check(lib().llmint8_quantize_tensorwise(_ptr(W), K, N, _ld(W, "W"), _ptr(Wq), _ptr(sw),
                                             *_ws(workspace), _stream(W)))
    return Wq, sw


def llmint8_linear_tensorwise_workspace_size(M: int, K: int, N: int) -> int:
    return int(lib().llmint8_linear_tensorwise_workspace_size(M, K, N))


def llmint8_linear_tensorwise(X: torch.Tensor, Wq: torch.Tensor, w_absmax: torch.Tensor, *,
                              bias: torch.Tensor | None = None, Y=None, workspace=None,
                              x_absmax: torch.Tensor | None = None,
                              C_debug: torch.Tensor | None = None) -> torch.Tensor:
    """The traditional per-tensor int8 layer: fp16 X [M, K], Wq [N, K] and w_absmax [1]
    from llmint8_quantize_tensorwise -> fp16 Y [M, N] (no outlier decomposition)."""
    _need(X, "X", torch.float16, 2)
    _need(Wq, "Wq", torch.int8, 2)
    _need_vec(w_absmax, "w_absmax", torch.float32, 1, exact=False)
    M, K = X.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or not Wq.is_contiguous():
        raise ValueError("Wq must be contiguous [N, K]")
    if bias is not None:
        _need_vec(bias, "bias", torch.float16, N)
    if x_absmax is not None:
        _need_vec(x_absmax, "x_absmax", torch.float32, 1, exact=False)
    if C_debug is not None:
        _need(C_debug, "C_debug", torch.int32)
        _need_shape(C_debug, "C_debug", (M, N), contiguous=True)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _need(Y, "Y", torch.float16, 2)
    _need_shape(Y, "Y", (M, N))
    if workspace is None:
        workspace = torch.empty((llmint8_linear_tensorwise_workspace_size(M, K, N),),
                                dtype=torch.uint8, device=X.device)
    _check(lib().llmint8_linear_tensorwise(
        _ptr(X), M, K, _ld(X, "X"), _ptr(Wq), _ptr(w_absmax), N, _ptr(bias), _ptr(Y),
        _ld(Y, "Y"), _ptr(x_absmax), _ptr(C_debug), *_ws(workspace),
        _stream(X)))
    return Y


# ---- FP8 (E4M3) variant --------------------------------------------------------------

def llmint8_quantize_colwise_fp8(W: torch.Tensor):
    """fp16 W [K, N] -> (Wq8 uint8 E4M3 codes [N, K], col_absmax fp32 [N])."""
    _need(W, "W", torch.float16, 2)
    K, N = W.shape
    Wq = torch.empty((N, K), dtype=torch.uint8, device=W.device)
    s = torch.empty((N,), dtype=torch.float32, device=W.device)
    _check(lib().llmint8_quantize_colwise_fp8(_ptr(W), K, N, _ld(W, "W"), _ptr(Wq), _ptr(s),
                                              _stream(W)))
    return Wq, s


def llmint8_quantize_rowwise_fp8(X: torch.Tensor, idx: torch.Tensor | None = None,
                                 count: torch.Tensor | None = None):
    """fp16 X [M, K] (+ outlier idx/count) -> (Xq8 uint8 E4M3 codes [M, K], row_absmax [M])."""
    _need(X, "X", torch.float16, 2)
    if (idx is None) != (count is None):
        raise ValueError("idx and count go together")
    M, K = X.shape
    if idx is not None:
        _need_vec(idx, "idx", torch.int32, K, exact=False)
        _need_vec(count, "count", torch.int32, 1, exact=False)
    Xq = torch.empty((M, K), dtype=torch.uint8, device=X.device)
    m = torch.empty((M,), dtype=torch.float32, device=X.device)
    _check(lib().llmint8_quantize_rowwise_fp8(_ptr(X), M, K, _ld(X, "X"), _ptr(idx), _ptr(count),
                                              _ptr(Xq), _ptr(m), _stream(X)))
    return Xq, m


def llmint8_linear_fp8_workspace_size(M: int, K: int, N: int) -> int:
    return int(lib().llmint8_linear_fp8_workspace_size(M, K, N))


def llmint8_linear_fp8(X: torch.Tensor, Wq8: torch.Tensor, col_absmax: torch.Tensor,
                       W: torch.Tensor | None, threshold: float = 6.0, *, Y=None, workspace=None,
                       outlier_count: torch.Tensor | None = None,
                       C_debug: torch.Tensor | None = None, opts: LinearOpts | None = None,
                       bias: torch.Tensor | None = None,
                       y_col_absmax: torch.Tensor | None = None,
                       x_col_absmax: torch.Tensor | None = None) -> torch.Tensor:
    """The FP8 (E4M3) variant of the layer: fp16 X [M, K] with Wq8 [N, K] and col_absmax
    from llmint8_quantize_colwise_fp8 and the fp16 weight W [K, N] -> fp16 Y [M, N].
    C_debug, if given, is an fp32 [M, N] tensor receiving the 8-bit product."""
    _need(X, "X", torch.float16, 2)
    _need(Wq8, "Wq8", torch.uint8, 2)
    M, K = X.shape
    N = Wq8.shape[0]
    if Wq8.shape[1] != K or not Wq8.is_contiguous():
        raise ValueError("Wq8 must be contiguous [N, K]")
    _need_vec(col_absmax, "col_absmax", torch.float32, N)
    if W is not None:
        _need(W, "W", torch.float16, 2)
        if tuple(W.shape) != (K, N):
            raise ValueError("W must be [K, N]")
    elif not (math.isinf(threshold) and threshold > 0):
        raise ValueError("W may be omitted only with threshold=+inf")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device=X.device)
    _need(Y, "Y", torch.float16, 2)
    _need_shape(Y, "Y", (M, N))
    if outlier_count is not None:
        _need_vec(outlier_count, "outlier_count", torch.int32, 1, exact=False)
    if C_debug is not None:
        _need(C_debug, "C_debug", torch.float32)
        _need_shape(C_debug, "C_debug", (M, N), contiguous=True)
    for name, t, dt, n in (("bias", bias, torch.float16, N),
                           ("y_col_absmax", y_col_absmax, torch.float32, N),
                           ("x_col_absmax", x_col_absmax, torch.float32, K)):
        if t is not None:
            _need(t, name, dt, 1)
            if t.numel() != n or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous vector of {n}")
    if workspace is None:
        workspace = torch.empty((llmint8_linear_fp8_workspace_size(M, K, N),), dtype=torch.uint8,
                                device=X.device)
    o = LinearOpts(gemm_begin_event=opts.gemm_begin_event if opts else None,
                   gemm_end_event=opts.gemm_end_event if opts else None,
                   outlier_weights=LLMINT8_OUTLIER_W_FP16,
                   bias=bias.data_ptr() if bias is not None else None,
                   y_col_absmax=y_col_absmax.data_ptr() if y_col_absmax is not None else None,
                   x_col_absmax=x_col_absmax.data_ptr() if x_col_absmax is not None else None)
    _check(lib().llmint8_linear_fp8(
        _ptr(X), M, K, _ld(X, "X"), _ptr(Wq8), _ptr(col_absmax), _ptr(W),
        _ld(W, "W") if W is not None else N, N, float(threshold), _ptr(Y), _ld(Y, "Y"),
        _ptr(outlier_count), _ptr(C_debug), *_ws(workspace), _stream(X),
        C.byref(o)))
    return Y
