"""Seeded synthetic inputs for the LLM.int8() mixed-precision linear layer.

This module only draws random fp16 tensors. It holds none of the method's
arithmetic (no absmax, no threshold test, no quantization, no matmul), so it can
feed both the HIP path and the CPU oracle without coupling them.

The workload shapes follow the layer shapes the pages discuss: an activation
X of shape [seq_len, hidden_dim] and a weight W of shape [hidden_dim,
output_dim] (LLM.int8() walkthrough page, section 2.3 "mixed decomposition"),
with a few feature columns of X carrying large values that are stable across
tokens (same page, section 2.2 "outlier features": 20-100x larger than the rest
and present in every token).

Recipe, per workload:
  * X ~ N(0, x_sigma) drawn in fp32 with PCG64, then cast to fp16 (RNE).
  * `n_out` planted outlier columns. Each column draws one sign and fills every
    row with sign * U[lo, hi] (stable across tokens, same sign).
  * W ~ N(0, w_sigma), fp32 -> fp16.
  * The 70B-scale workload re-draws its outlier columns for every call: call c
    uses its own seed and a column count drawn uniformly from 0.1%..1% of K.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

INF = float("inf")


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    x_sigma: float
    w_sigma: float
    out_lo: float
    out_hi: float
    thresholds: tuple
    seed: int
    n_out: int = 0                 # planted outlier columns (fixed count)
    fixed_cols: tuple = ()         # explicit planted columns (overrides a random choice)
    per_call: bool = False         # outlier set re-drawn on every call
    per_call_frac: tuple = (0.001, 0.01)
    description: str = field(default="", compare=False)

    @property
    def threshold(self) -> float:
        return self.thresholds[0]


WORKLOADS = {
    "tiny": Workload(
        "tiny", 16, 256, 128, 1.0, 0.02, 10.0, 30.0, (6.0,), 0,
        n_out=2, fixed_cols=(0, 131),
        description="16x256x128, 2 fixed outlier columns |x| in [10,30]"),
    "decode": Workload(
        "decode", 32, 4096, 4096, 1.0, 0.02, 20.0, 60.0, (6.0,), 1,
        n_out=4,
        description="decode-shaped 32x4096x4096, 4 outlier columns |x| in [20,60]"),
    "prefill": Workload(
        "prefill", 2048, 4096, 11008, 1.0, 0.02, 6.0, 60.0, (6.0,), 2,
        n_out=20,
        description="7B MLP up-projection prefill 2048x4096x11008, 20 outlier columns"),
    "13b": Workload(
        "13b", 4096, 5120, 13824, 1.5, 0.015, 6.0, 100.0, (6.0,), 3,
        n_out=51,
        description="13B-scale prefill 4096x5120x13824, X~N(0,1.5), 51 planted columns"),
    "70b": Workload(
        "70b", 8192, 8192, 28672, 1.0, 0.01, 6.0, 100.0, (6.0, 4.0, INF), 4,
        per_call=True,
        description="70B-scale layer 8192x8192x28672, outlier set re-drawn per call"),
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(list(key)))


def _normal_f16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(sigma)
    return a.astype(np.float16)


def planted_columns(wl: Workload, call: int = 0) -> np.ndarray:
    """Column indices that carry planted outliers for this call (ascending)."""
    if wl.fixed_cols:
        return np.array(sorted(wl.fixed_cols), dtype=np.int64)
    if wl.per_call:
        rng = _rng(wl.seed, 3, call)
        lo = max(1, int(math.ceil(wl.per_call_frac[0] * wl.K)))
        hi = max(lo, int(math.floor(wl.per_call_frac[1] * wl.K)))
        n = int(rng.integers(lo, hi + 1))
    else:
        rng = _rng(wl.seed, 3, 0)
        n = wl.n_out
    return np.sort(rng.choice(wl.K, size=n, replace=False)).astype(np.int64)


def make_x(wl: Workload, call: int = 0, rows: slice | None = None) -> np.ndarray:
    """fp16 activation X [M, K] for `call` (rows of it if `rows` is given)."""
    rng = _rng(wl.seed, 1, call if wl.per_call else 0)
    x = _normal_f16(rng, (wl.M, wl.K), wl.x_sigma)
    cols = planted_columns(wl, call)
    if cols.size:
        prng = _rng(wl.seed, 4, call if wl.per_call else 0)
        sign = np.where(prng.random(cols.size) < 0.5, -1.0, 1.0).astype(np.float32)
        mag = prng.uniform(wl.out_lo, wl.out_hi, size=(wl.M, cols.size)).astype(np.float32)
        x[:, cols] = (mag * sign[None, :]).astype(np.float16)
    if rows is not None:
        x = np.ascontiguousarray(x[rows])
    return x


def make_w(wl: Workload) -> np.ndarray:
    """fp16 weight W [K, N] (row-major, output channels along N)."""
    return _normal_f16(_rng(wl.seed, 2), (wl.K, wl.N), wl.w_sigma)


def random_case(M: int, K: int, N: int, seed: int, n_out: int = 0,
                out_lo: float = 6.0, out_hi: float = 60.0,
                x_sigma: float = 1.0, w_sigma: float = 0.05):
    """Small seeded (X, W, planted columns) triple for parity tests."""
    wl = Workload("case", M, K, N, x_sigma, w_sigma, out_lo, out_hi, (6.0,),
                  seed, n_out=min(n_out, K))
    return make_x(wl), make_w(wl), planted_columns(wl)
