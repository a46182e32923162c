"""Row-parallel use of the CPU oracle for the full-size parity tests.

Once the outlier set O of X is known, every later step of the layer is
independent per row of X: the row absmax and codes of row i, row i of the int8
product and row i of the merge read nothing of the other rows ("LLM.int8()"
walkthrough, section 2.1: one scale per row of X; section 2.3: the product of
the outlier columns). The helpers here find O once on the whole X with the
oracle, then run the oracle's own per-row steps on chunks of rows in a thread
pool (the oracle's C functions release the GIL while they run). The oracle's
arithmetic is untouched: each chunk goes through exactly the functions a
single-threaded call would use, in the same order.

Row samples for the large workloads cover every 256-row output tile of the
GEMM, the first and the last row.
"""
from __future__ import annotations

import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor, as_completed

import numpy as np

import oracle

TILE_ROWS = 256


def workers() -> int:
    """Threads for the oracle: the machine's CPU share (at most 16)."""
    return max(1, min(16, os.cpu_count() or 1))


def tile_rows(M: int, n: int = 256, tile: int = TILE_ROWS, seed: int | None = None) -> np.ndarray:
    """At least n distinct rows of an M-row output (all rows if M <= n): rows 0
    and M - 1, one row drawn inside every tile of `tile` rows, the rest drawn at
    random; ascending."""
    if M <= n:
        return np.arange(M)
    rng = np.random.default_rng(M if seed is None else seed)
    rows = {0, M - 1}
    for t0 in range(0, M, tile):
        rows.add(int(rng.integers(t0, min(M, t0 + tile))))
    while len(rows) < n:
        rows.add(int(rng.integers(0, M)))
    return np.array(sorted(rows), dtype=np.int64)


def _run(fn, chunks):
    """fn over the row chunks in a thread pool, results in chunk order. Long
    runs (the full 70b workload) report their progress on stderr every 20 s."""
    t0 = last = time.monotonic()
    out = [None] * len(chunks)
    with ThreadPoolExecutor(workers()) as ex:
        futs = {ex.submit(fn, c): i for i, c in enumerate(chunks)}
        for done, f in enumerate(as_completed(futs), 1):
            out[futs[f]] = f.result()
            now = time.monotonic()
            if now - last > 20:
                print(f"oracle rows: {done}/{len(chunks)} chunks, {now - t0:.0f} s",
                      file=sys.stderr, flush=True)
                last = now
    return out


def _chunks(rows: np.ndarray, nw: int):
    per = max(1, -(-rows.size // (4 * nw)))
    return [rows[i:i + per] for i in range(0, rows.size, per)]


def linear_rows(X, W, threshold, rows, Wq, s, *, outlier_weights="fp16", bias=None):
    """The layer's results (Xq, m, C, Y) on the given rows of X, with O found on
    all of X. Same values as oracle.linear_rows, computed chunk by chunk."""
    rows = np.asarray(rows, dtype=np.int64)
    idx = oracle.find_outliers(X, threshold)
    Xb = np.ascontiguousarray(X).view(np.uint16)

    def part(r):
        Xs = np.ascontiguousarray(Xb[r])
        Xq, m = oracle.quantize_rowwise(Xs, idx)
        C = oracle.gemm_i8(Xq, Wq)
        if outlier_weights == "fp16":
            Y = oracle.merge(C, m, s, Xs, W, idx)
        else:
            Y = oracle.merge_int8w(C, m, s, Xs, Wq, idx)
        if bias is not None:
            Y = oracle.add_bias(Y, bias)
        return Xq, m, C, Y

    parts = _run(part, _chunks(rows, workers()))
    return dict(rows=rows, idx=idx, Xq=np.concatenate([p[0] for p in parts]),
                m=np.concatenate([p[1] for p in parts]),
                C=np.concatenate([p[2] for p in parts]),
                Y=np.concatenate([p[3] for p in parts]))


def linear_fp8_rows(X, W, threshold, rows, Wq8, s):
    """FP8 (E4M3) layer results on the given rows, as oracle.linear_fp8(rows=...)."""
    rows = np.asarray(rows, dtype=np.int64)
    idx = oracle.find_outliers(X, threshold)
    Xb = np.ascontiguousarray(X).view(np.uint16)

    def part(r):
        Xs = np.ascontiguousarray(Xb[r])
        Xq, m = oracle.quantize_rowwise_fp8(Xs, idx)
        C = oracle.gemm_fp8(Xq, Wq8)
        return Xq, m, C, oracle.merge_fp8(C, m, s, Xs, W, idx)

    parts = _run(part, _chunks(rows, workers()))
    return dict(rows=rows, idx=idx, Wq=Wq8, s=s, Xq=np.concatenate([p[0] for p in parts]),
                m=np.concatenate([p[1] for p in parts]),
                C=np.concatenate([p[2] for p in parts]),
                Y=np.concatenate([p[3] for p in parts]))
