"""The row-parallel oracle helper of the full-size parity tests (CPU only):
its row samples cover every 256-row output tile, and its chunked, threaded
evaluation gives exactly the single-threaded oracle's results."""
import math

import numpy as np
import pytest

import oracle
import oracle_rows
import workloads


@pytest.mark.parametrize("M", [300, 2048, 4096, 8192, 8191])
def test_tile_rows_cover_every_output_tile(M):
    rows = oracle_rows.tile_rows(M)
    assert rows.size >= min(M, 256) and rows[0] == 0 and rows[-1] == M - 1
    assert np.all(np.diff(rows) > 0)
    assert set(range(-(-M // 256))) <= set((rows // 256).tolist())


def test_tile_rows_small_m_is_every_row():
    assert np.array_equal(oracle_rows.tile_rows(200), np.arange(200))


@pytest.mark.parametrize("M,K,N,threshold", [(37, 272, 72, 6.0), (130, 256, 40, 2.0),
                                             (64, 96, 24, math.inf), (9, 48, 16, 0.0)])
@pytest.mark.parametrize("mode", ["fp16", "int8"])
def test_chunked_rows_equal_the_whole_oracle(M, K, N, threshold, mode):
    X, W, _ = workloads.random_case(M, K, N, seed=M + K, n_out=3)
    Wq, s = oracle.quantize_colwise(W)
    b = (np.random.default_rng(N).standard_normal(N) * 0.5).astype(np.float16)
    whole = oracle.linear(X, W, threshold, Wq, s, outlier_weights=mode, bias=b)
    rows = np.arange(M)
    part = oracle_rows.linear_rows(X, W, threshold, rows, Wq, s, outlier_weights=mode, bias=b)
    for key in ("idx", "Xq", "m", "C"):
        assert np.array_equal(part[key], whole[key]), key
    assert np.array_equal(part["Y"], whole["Y"])
    sub = rows[::3]
    p2 = oracle_rows.linear_rows(X, W, threshold, sub, Wq, s, outlier_weights=mode, bias=b)
    assert np.array_equal(p2["C"], whole["C"][sub]) and np.array_equal(p2["Y"], whole["Y"][sub])


@pytest.mark.parametrize("threshold", [6.0, 3.0, math.inf])
def test_chunked_fp8_rows_equal_the_whole_oracle(threshold):
    X, W, _ = workloads.random_case(70, 256, 40, seed=5, n_out=3)
    Wq8, s = oracle.quantize_colwise_fp8(W)
    whole = oracle.linear_fp8(X, W, threshold, Wq8=Wq8, s=s)
    rows = np.arange(0, 70, 2)
    part = oracle_rows.linear_fp8_rows(X, W, threshold, rows, Wq8, s)
    assert np.array_equal(part["Xq"], whole["Xq"][rows])
    assert np.array_equal(part["C"], whole["C"][rows])
    assert np.array_equal(part["Y"], whole["Y"][rows])
