"""Whole-layer brute force: an independent numpy implementation of the
LLM.int8() layer, written from the definitions ("LLM.int8()" walkthrough,
sections 2.1 and 2.3; "LLM.int8() pitfalls", sections 1 and 3.3; INT8-to-QLoRA
tutorial, sections 3.2 and 3.3), against the C oracle on 500 seeded tiny
shapes: M and N in 1..70, K a multiple of 16 up to 304, thresholds 0, 2, 4, 6
and inf.

numpy evaluates each scale in IEEE fp32 (one division 127 / absmax, one
multiply per entry, round half to even, clamp), the int8 product in int64 and
the merge in fp64 with a library matmul for the outlier product. Every integer
output (outlier list, Wq, s, Xq, m, C) must match bit for bit; Y, whose fp64
summation order differs, within 1e-12 relative.
"""
import math

import numpy as np
import pytest

import oracle

THRESHOLDS = (0.0, 2.0, 4.0, 6.0, math.inf)


def numpy_layer(X16, W16, tau):
    X = X16.astype(np.float32)
    W = W16.astype(np.float32)
    K = X.shape[1]
    # weights: per-column absmax over all K rows, codes [N, K]
    s = np.abs(W).max(axis=0)
    safe_s = np.where(s > 0, s, np.float32(1))
    inv_s = np.where(s > 0, np.float32(127) / safe_s, np.float32(0)).astype(np.float32)
    Wq = np.clip(np.rint(W * inv_s[None, :]), -127, 127).astype(np.int8).T.copy()
    # outlier columns: some |x| >= tau
    O = np.flatnonzero((np.abs(X) >= np.float32(tau)).any(axis=0)).astype(np.int32)
    kept = np.ones(K, bool)
    kept[O] = False
    # rows: absmax over kept columns, codes, outlier columns zero
    m = np.where(kept[None, :], np.abs(X), np.float32(0)).max(axis=1).astype(np.float32)
    safe_m = np.where(m > 0, m, np.float32(1))
    inv_m = np.where(m > 0, np.float32(127) / safe_m, np.float32(0)).astype(np.float32)
    Xq = np.clip(np.rint(X * inv_m[:, None]), -127, 127).astype(np.int8)
    Xq[:, ~kept] = 0
    C = Xq.astype(np.int64) @ Wq.astype(np.int64).T
    Y = (C.astype(np.float64) * m.astype(np.float64)[:, None] * s.astype(np.float64)[None, :]
         / 16129.0)
    Y += X[:, O].astype(np.float64) @ W[O, :].astype(np.float64)
    return dict(idx=O, Wq=Wq, s=s, Xq=Xq, m=m, C=C, Y=Y)


def cases(n=500, seed=8):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, N = int(rng.integers(1, 71)), int(rng.integers(1, 71))
        K = 16 * int(rng.integers(1, 20))
        out.append((M, K, N, THRESHOLDS[i % len(THRESHOLDS)], int(rng.integers(1 << 30))))
    return out


def draw(M, K, N, seed):
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((M, K)) * 1.5).astype(np.float32)
    for k in rng.choice(K, size=min(K, int(rng.integers(0, 4))), replace=False):
        X[:, k] = np.sign(rng.standard_normal()) * rng.uniform(6, 60, M)
    if M > 2 and rng.random() < 0.3:
        X[int(rng.integers(M))] = 0                    # a zero row
    W = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    if N > 2 and rng.random() < 0.3:
        W[:, int(rng.integers(N))] = 0                 # a zero column
    return X.astype(np.float16), W.astype(np.float16)


@pytest.mark.parametrize("M,K,N,tau,seed", cases())
def test_layer_matches_numpy_brute_force(M, K, N, tau, seed):
    X, W = draw(M, K, N, seed)
    ref = numpy_layer(X, W, tau)
    got = oracle.linear(X, W, tau)
    for key in ("idx", "Wq", "Xq", "C"):
        assert np.array_equal(got[key], ref[key]), key
    for key in ("s", "m"):
        assert np.array_equal(got[key].view(np.uint32), ref[key].view(np.uint32)), key
    scale = max(1.0, float(np.abs(ref["Y"]).max()))
    assert np.allclose(got["Y"], ref["Y"], rtol=1e-12, atol=1e-12 * scale)
