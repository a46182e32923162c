"""Guard bands around every output of every entry point (GPU).

Each output buffer (and each workspace) is carved out of a larger device
allocation whose bytes before and after it hold a canary pattern. The call
goes straight through the C ABI with those pointers, and afterwards every
canary byte must be unchanged: no kernel writes outside what it was handed.
The shapes take each kernel path: the single small-M kernel, the split-K
small-M kernels, the large-M kernels with ragged tiles, the one-read column
pass (a half-empty last stripe, 16 rows per thread) and the two-pass one.
"""
import ctypes as C
import math

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

CANARY = 0xA5
BAND = 4096


@pytest.fixture(scope="module")
def dev():
    import torch
    import bit_quantized_matmul_col_amd as lm
    lm.lib()
    return torch, lm


class Banded:
    """Device regions of the given byte sizes, each between two canary bands."""

    def __init__(self, torch, *sizes):
        self.torch = torch
        self.sizes = [max(int(n), 1) for n in sizes]
        self.bufs = [torch.full((n + 2 * BAND,), CANARY, dtype=torch.uint8, device="cuda")
                     for n in self.sizes]

    def ptr(self, i):
        return C.c_void_p(self.bufs[i].data_ptr() + BAND)

    def view(self, i, dtype, shape):
        n = self.sizes[i]
        return self.bufs[i][BAND:BAND + n].view(dtype).view(shape)

    def check(self, what):
        self.torch.cuda.synchronize()
        for i, (b, n) in enumerate(zip(self.bufs, self.sizes)):
            head, tail = b[:BAND], b[BAND + n:]
            assert bool((head == CANARY).all()), f"{what}: bytes before output {i} changed"
            assert bool((tail == CANARY).all()), f"{what}: bytes after output {i} changed"


def _stream(torch):
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _gpu(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("K,N", [(1024, 24), (4112, 136), (8208, 40)])
@pytest.mark.parametrize("fp8", [False, True])
def test_column_pass(dev, K, N, fp8):
    torch, lm = dev
    _, W, _ = workloads.random_case(2, K, N, seed=K + N, n_out=0)
    Wd = _gpu(torch, W)
    b = Banded(torch, N * K, 4 * N)
    fn = lm.lib().llmint8_quantize_colwise_fp8 if fp8 else lm.lib().llmint8_quantize_colwise
    assert fn(C.c_void_p(Wd.data_ptr()), K, N, N, b.ptr(0), b.ptr(1), _stream(torch)) == 0
    b.check(f"colwise K={K} N={N} fp8={fp8}")


@pytest.mark.parametrize("M,K", [(5, 1024), (300, 2064), (33, 4096)])
@pytest.mark.parametrize("fp8", [False, True])
def test_outliers_and_row_pass(dev, M, K, fp8):
    torch, lm = dev
    L = lm.lib()
    X, _, _ = workloads.random_case(M, K, 8, seed=M + K, n_out=3)
    Xd = _gpu(torch, X)
    ws = L.llmint8_find_outliers_workspace_size(M, K)
    b = Banded(torch, 4 * K, 4, ws)
    assert L.llmint8_find_outliers(C.c_void_p(Xd.data_ptr()), M, K, K, 6.0, b.ptr(0), b.ptr(1),
                                   b.ptr(2), ws, _stream(torch)) == 0
    b.check(f"find_outliers M={M} K={K}")
    r = Banded(torch, M * K, 4 * M)
    fn = L.llmint8_quantize_rowwise_fp8 if fp8 else L.llmint8_quantize_rowwise
    assert fn(C.c_void_p(Xd.data_ptr()), M, K, K, b.ptr(0), b.ptr(1), r.ptr(0), r.ptr(1),
              _stream(torch)) == 0
    r.check(f"rowwise M={M} K={K} fp8={fp8}")


# the single small-M kernel, the split-K small-M kernels, large M with ragged
# tiles, and large M with K-compaction (threshold 0: every column an outlier)
LAYER = [(8, 1024, 136, 6.0), (33, 1024, 264, 6.0), (300, 1040, 520, 6.0),
         (400, 1024, 264, 0.0), (48, 2048, 72, math.inf),
         # split-K tiles of the large-M GEMM (int8): 9 and 8 tiles of 128 rows in 2 parts
         (300, 4096, 520, 6.0), (400, 4096, 264, 0.0)]


@pytest.mark.parametrize("M,K,N,threshold", LAYER)
@pytest.mark.parametrize("variant", ["int8", "fp8", "noalloc"])
def test_layer(dev, M, K, N, threshold, variant):
    torch, lm = dev
    L = lm.lib()
    X, W, _ = workloads.random_case(M, K, N, seed=M * 7 + N, n_out=2)
    Xd, Wd = _gpu(torch, X), _gpu(torch, W)
    st = _stream(torch)
    if variant == "fp8":
        Wq, s = lm.llmint8_quantize_colwise_fp8(Wd)
        ws = L.llmint8_linear_fp8_workspace_size(M, K, N)
    else:
        Wq, s = lm.llmint8_quantize_colwise(Wd)
        ws = L.llmint8_workspace_size(M, K, N)
    b = Banded(torch, 2 * M * N, 4, 4 * M * N, ws)
    args = [C.c_void_p(Xd.data_ptr()), M, K, K, C.c_void_p(Wq.data_ptr()),
            C.c_void_p(s.data_ptr()), C.c_void_p(Wd.data_ptr()), N, N, threshold,
            b.ptr(0), N, b.ptr(1), b.ptr(2)]
    if variant == "fp8":
        rc = L.llmint8_linear_fp8(*args, b.ptr(3), ws, st, None)
    elif variant == "noalloc":
        rc = L.llmint8_linear_noalloc(*args, st)
    else:
        rc = L.llmint8_linear(*args, b.ptr(3), ws, st)
    assert rc == 0, lm.llmint8_status_string(rc)
    b.check(f"linear {variant} M={M} K={K} N={N} threshold={threshold}")
    y = b.view(0, torch.float16, (M, N))
    assert bool(torch.isfinite(y).all())


@pytest.mark.parametrize("M,K,N", [(8, 1024, 136), (300, 1040, 520)])
def test_tensorwise(dev, M, K, N):
    torch, lm = dev
    L = lm.lib()
    X, W, _ = workloads.random_case(M, K, N, seed=M + 3 * N, n_out=2)
    Xd, Wd = _gpu(torch, X), _gpu(torch, W)
    st = _stream(torch)
    wq_ws = L.llmint8_quantize_tensorwise_workspace_size(K, N)
    q = Banded(torch, N * K, 4, wq_ws)
    assert L.llmint8_quantize_tensorwise(C.c_void_p(Wd.data_ptr()), K, N, N, q.ptr(0), q.ptr(1),
                                         q.ptr(2), wq_ws, st) == 0
    q.check(f"quantize_tensorwise K={K} N={N}")
    ws = L.llmint8_linear_tensorwise_workspace_size(M, K, N)
    b = Banded(torch, 2 * M * N, 4, 4 * M * N, ws)  # Y, X's absmax, C, workspace
    rc = L.llmint8_linear_tensorwise(C.c_void_p(Xd.data_ptr()), M, K, K, q.ptr(0), q.ptr(1), N,
                                     None, b.ptr(0), N, b.ptr(1), b.ptr(2), b.ptr(3), ws, st)
    assert rc == 0, lm.llmint8_status_string(rc)
    b.check(f"linear_tensorwise M={M} K={K} N={N}")
