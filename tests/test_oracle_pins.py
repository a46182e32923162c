"""Pins of the CPU oracle against facts the pages and the mathematics fix.

None of these tests retypes the oracle's formulas: they check it against the
pages' worked example and hand-derived fixtures (tests/golden/), library
routines on special cases that reduce to them (numpy matmul, numpy's fp16
decoding), brute-force searches on tiny inputs, closed forms and invariants.
"""
import math

import numpy as np
import pytest

import oracle
import workloads
from golden_io import floats, ints, load


def f16(rows):
    return np.array(rows, dtype=np.float16)


# --- fp16 decoding -------------------------------------------------------------

def test_half_decode_every_pattern():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.half_to_float(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    # bitwise, so signed zeros and subnormals are pinned too
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# --- the quantizer: page values and hand-derived values --------------------------

def test_worked_example_codearts_section2():
    g = load("p5_worked_example.txt")
    X = f16([floats(g["x"])])
    idx = oracle.find_outliers(X, float(g["threshold"][0]))
    assert idx.size == 0
    Xq, m = oracle.quantize_rowwise(X, idx)
    assert Xq[0].tolist() == ints(g["q"])
    assert round(127.0 / float(m[0]), 2) == float(g["scale_printed"][0])
    deq = Xq[0].astype(np.float64) * float(m[0]) / 127.0
    assert [round(float(v), 2) for v in deq] == floats(g["dequantized_printed"])


def test_derived_row_with_outlier_column():
    g = load("derived_tau6.txt")
    X = f16([floats(g["x"])])
    idx = oracle.find_outliers(X, float(g["threshold"][0]))
    assert idx.tolist() == ints(g["outliers"])
    Xq, m = oracle.quantize_rowwise(X, idx)
    assert float(m[0]) == float(g["absmax"][0])
    assert Xq[0].tolist() == ints(g["q"])


def test_round_half_to_even_ties():
    g = load("rne_ties.txt")
    X = f16([floats(g["x"])])
    Xq, _ = oracle.quantize_rowwise(X, oracle.find_outliers(X, math.inf))
    assert Xq[0].tolist() == ints(g["q"])


def test_resolution_loss_closed_form_walkthrough_section_2_2():
    # A column max of 60 next to values of 3 leaves 3/60*127 ~ 6 levels for them
    # (2kiu.com walkthrough, section 2.2); isolating the 60 restores all 127.
    X = f16([[60.0, 3.0, -3.0, 1.5]])
    Xq, m = oracle.quantize_rowwise(X, oracle.find_outliers(X, math.inf))
    assert m[0] == 60.0 and Xq[0].tolist() == [127, 6, -6, 3]
    assert abs(3.0 / 60.0 * 127.0 - 6.35) < 1e-12
    idx = oracle.find_outliers(X, 6.0)
    Xq, m = oracle.quantize_rowwise(X, idx)
    assert idx.tolist() == [0] and m[0] == 3.0 and Xq[0].tolist() == [0, 127, -127, 64]


def _nearest_even_search(v: float) -> int:
    """The integer of [-127, 127] closest to v; ties go to the even one."""
    best, best_d = None, None
    for q in range(-127, 128):
        d = abs(v - q)
        if best is None or d < best_d or (d == best_d and q % 2 == 0):
            best, best_d = q, d
    return best


def test_quantizer_brute_force_rounding_and_clamp():
    rng = np.random.default_rng(11)
    for trial in range(40):
        K = int(rng.integers(1, 24))
        x = (rng.standard_normal(K) * rng.choice([0.01, 1.0, 50.0])).astype(np.float16)
        if trial % 5 == 0:
            x[rng.integers(K)] = np.float16(0.5) * np.float16(rng.integers(-9, 9))
        X = x[None, :]
        Xq, m = oracle.quantize_rowwise(X, np.zeros(0, np.int32))
        amax = np.float32(np.max(np.abs(x.astype(np.float32))))
        assert m[0] == amax
        if amax == 0:
            assert not Xq.any()
            continue
        inv = np.float32(127.0) / amax
        for k in range(K):
            v = float(np.float32(x[k]) * inv)
            assert Xq[0, k] == _nearest_even_search(v)


def test_reconstruction_error_bound():
    # |x - q*m/127| <= m/254 + m*2^-23 for every non-outlier entry (half a
    # quantization step, plus the two fp32 roundings inside x * fl(127/m)).
    X, _, planted = workloads.random_case(64, 512, 8, seed=5, n_out=6)
    idx = oracle.find_outliers(X, 6.0)
    Xq, m = oracle.quantize_rowwise(X, idx)
    xf = X.astype(np.float64)
    keep = np.ones(X.shape[1], bool)
    keep[idx] = False
    err = np.abs(xf - Xq.astype(np.float64) * m[:, None].astype(np.float64) / 127.0)[:, keep]
    bound = (m.astype(np.float64) / 254.0 + m.astype(np.float64) * 2.0 ** -23)[:, None]
    assert np.all(err <= bound)


# --- outlier detection -------------------------------------------------------------

def test_threshold_is_inclusive():
    X = np.full((5, 16), 0.25, np.float16)
    X[3, 7] = 6.0
    assert oracle.find_outliers(X, 6.0).tolist() == [7]
    just_above = float(np.nextafter(np.float32(6.0), np.float32(np.inf)))
    assert oracle.find_outliers(X, just_above).size == 0


def test_threshold_edges():
    X, _, _ = workloads.random_case(9, 48, 4, seed=2, n_out=3)
    assert oracle.find_outliers(X, math.inf).size == 0
    assert oracle.find_outliers(X, 0.0).tolist() == list(range(48))
    assert oracle.find_outliers(X, -1.0).tolist() == list(range(48))


def test_outliers_match_brute_force_and_plants():
    wl = workloads.WORKLOADS["tiny"]
    X = workloads.make_x(wl)
    idx = oracle.find_outliers(X, wl.threshold)
    brute = [k for k in range(wl.K)
             if any(abs(float(X[i, k])) >= wl.threshold for i in range(wl.M))]
    assert idx.tolist() == brute == list(wl.fixed_cols)


def test_nan_entries_are_never_outliers_and_never_set_a_row_scale():
    # the reading taken for non-finite inputs: every comparison with NaN is
    # false, so a NaN passes no threshold and no absmax; +-inf passes both
    X = f16([[1.0, np.nan, -2.0, 0.5], [np.nan, 3.0, 0.25, -np.inf], [0.5, 0.5, 8.0, 0.0]])
    assert oracle.find_outliers(X, 6.0).tolist() == [2, 3]
    assert oracle.find_outliers(X, 0.0).tolist() == [0, 1, 2, 3]
    idx = oracle.find_outliers(X, 6.0)
    Xq, m = oracle.quantize_rowwise(X, idx)
    assert m.tolist() == [1.0, 3.0, 0.5]
    assert Xq[0].tolist() == [127, 0, 0, 0]   # NaN codes as 0, column 2 is an outlier
    assert Xq[1].tolist() == [0, 127, 0, 0]
    # the columns without NaN give the same codes as the same rows without it
    Xc = X.copy()
    Xc[0, 1] = Xc[1, 0] = 0
    Xq2, m2 = oracle.quantize_rowwise(Xc, idx)
    assert np.array_equal(Xq2, Xq) and np.array_equal(m2, m)


def test_outlier_set_shrinks_as_threshold_grows():
    X, _, _ = workloads.random_case(40, 256, 4, seed=3, n_out=5)
    prev = None
    for tau in [0.0, 1.0, 2.0, 3.0, 4.0, 6.0, 20.0, math.inf]:
        cur = set(oracle.find_outliers(X, tau).tolist())
        if prev is not None:
            assert cur <= prev
        prev = cur


# --- special cases that reduce to a library matmul -------------------------------

def _exact_integer_case(rng, M, K, N):
    """Integer-valued X, W (|v| <= 127) with a +-127 in every row of X and every
    column of W, so both scales are exactly 1 and quantization is exact."""
    X = rng.integers(-127, 128, size=(M, K)).astype(np.float64)
    X[np.arange(M), rng.integers(0, K, M)] = 127.0 * rng.choice([-1, 1], M)
    W = rng.integers(-127, 128, size=(K, N)).astype(np.float64)
    W[rng.integers(0, K, N), np.arange(N)] = 127.0 * rng.choice([-1, 1], N)
    return X, W


def test_threshold_inf_is_plain_vectorwise_int8():
    # With threshold +inf nothing is an outlier and the layer is the pure
    # vector-wise int8 product (Lightning Fabric page, section 2.2). On exact
    # integer data with unit scales it must equal X @ W exactly.
    rng = np.random.default_rng(7)
    X, W = _exact_integer_case(rng, 13, 37, 11)
    r = oracle.linear(X.astype(np.float16), W.astype(np.float16), math.inf)
    assert r["idx"].size == 0
    ref = X @ W
    assert np.array_equal(r["C"].astype(np.float64), ref)
    assert np.array_equal(r["Y"], ref)
    # power-of-two scaling of rows of X and columns of W: the int8 operands do
    # not change, the scales absorb the powers exactly, Y scales exactly.
    rs = 2.0 ** rng.integers(-6, 3, size=(13, 1))
    cs = 2.0 ** rng.integers(-6, 3, size=(1, 11))
    r2 = oracle.linear((X * rs).astype(np.float16), (W * cs).astype(np.float16), math.inf)
    assert np.array_equal(r2["Xq"], r["Xq"]) and np.array_equal(r2["Wq"], r["Wq"])
    assert np.array_equal(r2["m"].astype(np.float64), 127.0 * rs[:, 0])
    assert np.array_equal(r2["s"].astype(np.float64), 127.0 * cs[0])
    assert np.array_equal(r2["Y"], ref * rs * cs)


def test_all_outlier_columns_reduce_to_fp16_matmul():
    # threshold 0: every column is an outlier, the int8 part is empty and the
    # layer is the 16-bit matmul of X and W.
    X, W, _ = workloads.random_case(21, 96, 17, seed=4, n_out=2)
    r = oracle.linear(X, W, 0.0)
    assert r["idx"].tolist() == list(range(96))
    assert not r["Xq"].any() and not r["m"].any() and not r["C"].any()
    ref = X.astype(np.float64) @ W.astype(np.float64)
    np.testing.assert_allclose(r["Y"], ref, rtol=1e-12, atol=1e-12)


def test_int8_matmul_matches_numpy():
    rng = np.random.default_rng(8)
    for M, K, N in [(1, 1, 1), (3, 70, 5), (17, 300, 9), (40, 64, 33)]:
        Xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
        Wq = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
        ref = Xq.astype(np.int64) @ Wq.astype(np.int64).T
        assert np.array_equal(oracle.gemm_i8(Xq, Wq), ref)
    big = np.full((2, 133144), 127, np.int8)
    assert oracle.gemm_i8(big, big)[0, 0] == 127 * 127 * 133144


def test_hand_worked_layer_call():
    g = load("hand_linear.txt")
    X = f16([floats(g["X"])])
    W = f16([floats(r) for r in g["W_rows"]])
    r = oracle.linear(X, W, float(g["threshold"][0]))
    assert r["idx"].tolist() == ints(g["outliers"])
    assert r["m"].tolist() == floats(g["absmax_x"])
    assert r["Xq"][0].tolist() == ints(g["Xq"])
    assert r["s"].tolist() == floats(g["absmax_w"])
    assert r["Wq"].tolist() == [ints(row) for row in g["Wq_rows"]]
    assert r["C"][0].tolist() == ints(g["C"])
    np.testing.assert_allclose(r["Y"][0], floats(g["Y"]), rtol=1e-15, atol=0)


# --- invariants ------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_layer_invariants(seed):
    X, W, planted = workloads.random_case(33, 160, 24, seed=seed, n_out=4)
    r = oracle.linear(X, W, 6.0)
    idx, Xq, m, C = r["idx"], r["Xq"], r["m"], r["C"]
    assert set(planted.tolist()) <= set(idx.tolist())
    assert np.all(np.abs(Xq.astype(np.int32)) <= 127)
    assert not Xq[:, idx].any()
    rows = np.nonzero(m > 0)[0]
    assert np.all(np.abs(Xq[rows].astype(np.int32)).max(axis=1) == 127)
    assert np.all(np.abs(r["Wq"].astype(np.int32)).max(axis=1)[r["s"] > 0] == 127)
    assert np.all(np.abs(C.astype(np.int64)) <= 127 * 127 * (160 - idx.size))
    # sign flips negate the integer results exactly (round-half-even is odd-symmetric)
    rn = oracle.linear(-X, W, 6.0)
    assert np.array_equal(rn["idx"], idx) and np.array_equal(rn["m"], m)
    assert np.array_equal(rn["Xq"], -Xq) and np.array_equal(rn["C"], -C)
    rw = oracle.linear(X, -W, 6.0)
    assert np.array_equal(rw["Wq"], -r["Wq"]) and np.array_equal(rw["C"], -C)
    np.testing.assert_allclose(rw["Y"], -r["Y"], rtol=0, atol=0)


def test_joint_permutation_of_inner_dimension():
    X, W, _ = workloads.random_case(12, 128, 20, seed=9, n_out=5)
    perm = np.random.default_rng(1).permutation(128)
    r = oracle.linear(X, W, 6.0)
    rp = oracle.linear(np.ascontiguousarray(X[:, perm]), np.ascontiguousarray(W[perm]), 6.0)
    assert sorted(perm[rp["idx"]].tolist()) == r["idx"].tolist()
    assert np.array_equal(rp["m"], r["m"])
    assert np.array_equal(rp["C"], r["C"])
    np.testing.assert_allclose(rp["Y"], r["Y"], rtol=1e-12, atol=1e-12)


def test_rows_are_independent_given_the_outlier_set():
    X, W, _ = workloads.random_case(30, 96, 16, seed=12, n_out=3)
    full = oracle.linear(X, W, 6.0)
    rows = [0, 7, 29]
    part = oracle.linear_rows(X, W, 6.0, rows)
    assert np.array_equal(part["idx"], full["idx"])
    assert np.array_equal(part["Xq"], full["Xq"][rows])
    assert np.array_equal(part["C"], full["C"][rows])
    assert np.array_equal(part["Y"], full["Y"][rows])


def test_outlier_isolation_beats_per_tensor_int8():
    # Qualitative (2kiu.com walkthrough section 2.2; codearts page sections 2
    # and 4): one scale for the whole tensor loses the small values next to an
    # outlier; the decomposition keeps them. Compared against exact X @ W.
    wl = workloads.WORKLOADS["tiny"]
    X, W = workloads.make_x(wl), workloads.make_w(wl)
    exact = X.astype(np.float64) @ W.astype(np.float64)
    y = oracle.linear(X, W, 6.0)["Y"]
    xf, wf = X.astype(np.float64), W.astype(np.float64)
    sx, sw = np.abs(xf).max() / 127, np.abs(wf).max() / 127
    per_tensor = np.rint(xf / sx) @ np.rint(wf / sw) * sx * sw
    e_mixed = np.linalg.norm(y - exact)
    e_tensor = np.linalg.norm(per_tensor - exact)
    assert e_mixed * 5 < e_tensor


# --- int8-only weight residency (walkthrough sections 2.4 and 6) --------------------

def exact_code_weight(K, N, seed):
    """fp16 W whose columns are integer codes times a power of two, with one code
    of magnitude 127 per column: quantize_colwise recovers the codes exactly and
    Wq * s / 127 reproduces W exactly."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, size=(K, N))
    q[rng.integers(0, K, size=N), np.arange(N)] = 127 * rng.choice([-1, 1], size=N)
    e = rng.integers(-12, -4, size=N).astype(np.float64)
    return (q * np.exp2(e)).astype(np.float16), q, e


def test_int8_weights_equal_fp16_weights_when_codes_are_exact():
    X, _, _ = workloads.random_case(9, 96, 8, seed=3, n_out=4)
    W, q, e = exact_code_weight(96, 20, seed=4)
    a = oracle.linear(X, W, 6.0)
    assert np.array_equal(a["Wq"].T.astype(np.int64), q)
    assert np.array_equal(a["s"].astype(np.float64), 127 * np.exp2(e))
    b = oracle.linear(X, W, 6.0, outlier_weights="int8")
    assert a["idx"].size >= 4
    assert np.array_equal(a["Y"], b["Y"])


def test_int8_weights_all_outlier_is_matmul_with_dequantized_codes():
    # threshold 0: every column is an outlier, so Y = X . (Wq^T * s / 127) exactly
    X, W, _ = workloads.random_case(7, 64, 24, seed=5, n_out=2)
    r = oracle.linear(X, W, 0.0, outlier_weights="int8")
    assert r["idx"].size == 64 and not r["C"].any()
    deq = r["Wq"].T.astype(np.float64) * r["s"].astype(np.float64) / 127.0
    np.testing.assert_allclose(r["Y"], X.astype(np.float64) @ deq, rtol=1e-12, atol=1e-12)


def test_int8_weights_without_outliers_change_nothing():
    X, W, _ = workloads.random_case(11, 80, 16, seed=6, n_out=3)
    a = oracle.linear(X, W, math.inf)
    b = oracle.linear(X, W, math.inf, outlier_weights="int8")
    assert a["idx"].size == 0 and np.array_equal(a["Y"], b["Y"])


def test_int8_weights_brute_force():
    X, W, _ = workloads.random_case(3, 32, 5, seed=7, n_out=2)
    r = oracle.linear(X, W, 5.0, outlier_weights="int8")
    xf = X.astype(np.float64)
    Wq, s = r["Wq"], r["s"].astype(np.float64)
    for i in range(3):
        for n in range(5):
            acc = sum(float(r["Xq"][i, k]) * float(Wq[n, k]) for k in range(32))
            y = acc * float(r["m"][i]) * s[n] / 16129.0
            for k in r["idx"]:
                y += xf[i, k] * (float(Wq[n, k]) * s[n] / 127.0)
            assert abs(y - r["Y"][i, n]) <= 1e-12 * max(1.0, abs(y))


# --- the traditional per-tensor int8 layer (codearts page sections 1 and 2) -----------

def test_per_tensor_worked_example_codearts_section2():
    # the page's example is one scale for the whole (1 x 4) tensor
    g = load("p5_worked_example.txt")
    X = f16([floats(g["x"])])
    W = np.eye(4, dtype=np.float16)
    Wq, sw = oracle.quantize_tensorwise(W)
    r = oracle.linear_tensorwise(X, Wq, sw)
    assert r["Xq"][0].tolist() == ints(g["q"])
    assert round(127.0 / float(r["sx"]), 2) == float(g["scale_printed"][0])


def test_per_tensor_exact_integers_reduce_to_integer_matmul():
    rng = np.random.default_rng(8)
    X = rng.integers(-100, 101, size=(6, 40)).astype(np.float16)
    W = rng.integers(-100, 101, size=(40, 12)).astype(np.float16)
    # both absmax 127, reached only in the last row and column: scale 1, codes = values
    X[5, 39], W[39, 11] = 127, -127
    Wq, sw = oracle.quantize_tensorwise(W)
    r = oracle.linear_tensorwise(X, Wq, sw)
    assert float(sw) == 127.0 and float(r["sx"]) == 127.0
    exact = X.astype(np.int64) @ W.astype(np.int64)
    assert np.array_equal(r["C"].astype(np.int64), exact)
    assert np.array_equal(r["Y"], exact.astype(np.float64))


def test_per_tensor_weights_equal_per_column_when_columns_share_the_absmax():
    X, W, _ = workloads.random_case(1, 48, 10, seed=9)
    W = W.astype(np.float32)
    W[5, :] = 0.75  # every column reaches the same absmax 0.75 (larger than the rest)
    W = W.astype(np.float16)
    Wq_t, sw = oracle.quantize_tensorwise(W)
    Wq_c, s = oracle.quantize_colwise(W)
    assert np.all(s == sw) and np.array_equal(Wq_t, Wq_c)


def test_bias_is_added_after_the_rescale():
    X, W, _ = workloads.random_case(5, 64, 12, seed=10, n_out=2)
    b = (np.arange(12) * 0.125 - 0.5).astype(np.float16)
    for mode in ("fp16", "int8"):
        a = oracle.linear(X, W, 6.0, outlier_weights=mode)
        c = oracle.linear(X, W, 6.0, outlier_weights=mode, bias=b)
        assert np.array_equal(c["Y"], a["Y"] + b.astype(np.float64)[None, :])
    Wq, sw = oracle.quantize_tensorwise(W)
    a = oracle.linear_tensorwise(X, Wq, sw)
    c = oracle.linear_tensorwise(X, Wq, sw, bias=b)
    assert np.array_equal(c["Y"], a["Y"] + b.astype(np.float64)[None, :])


# --- FP8 (E4M3) variant ------------------------------------------------------------
# The "INT8 vs FP8 vs GPTQ" page (mlqm.cn, sections 2 and 4): E4M3 has 4
# exponent bits and 3 mantissa bits, its largest value is about 448, and
# wide-ranged activations need a scale before the cast.

def test_e4m3_format_facts():
    codes = np.arange(256, dtype=np.uint8)
    v = oracle.e4m3_value(codes)
    assert v[0x7E] == 448.0 and np.nanmax(v) == 448.0  # largest finite value
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2  # no infinities
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x38] == 1.0
    assert v[0x00] == 0.0 and math.copysign(1.0, v[0x80]) == -1.0
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)  # codes 0x00..0x7e ascend with their value
    assert np.array_equal(v[0x80:0xFF], -pos)  # the sign bit negates
    # 3 mantissa bits: 8 values per binade above the subnormals
    assert np.sum((pos >= 1.0) & (pos < 2.0)) == 8


def _torch_e4m3(t):
    import torch
    return torch.from_numpy(np.ascontiguousarray(t, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encoding_matches_torch_cast():
    # in range the encoder must agree bit for bit with PyTorch's own cast to
    # float8_e4m3fn (round to nearest, ties to even), including every exact
    # midpoint between neighbouring codes
    rng = np.random.default_rng(3)
    mag = np.exp2(rng.uniform(-13.0, np.log2(448.0), 200000)).astype(np.float32)
    t = mag * rng.choice(np.float32([-1.0, 1.0]), mag.size)
    pos = oracle.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[1:] + pos[:-1]) / 2)  # exact in fp32
    t = np.concatenate([t, mids, -mids, pos.astype(np.float32), np.float32([0.0, -0.0])])
    assert np.array_equal(oracle.e4m3_encode(t), _torch_e4m3(t))


def test_e4m3_saturates_above_448():
    t = np.float32([448.0, 449.0, 463.9, 464.0, 480.0, 1e6, -500.0])
    assert oracle.e4m3_encode(t).tolist() == [0x7E] * 6 + [0xFE]


def test_fp8_quantizer_brute_force():
    pos = oracle.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    rng = np.random.default_rng(12)
    for trial in range(30):
        K = int(rng.integers(1, 20))
        x = (rng.standard_normal(K) * rng.choice([0.001, 1.0, 30.0])).astype(np.float16)
        Xq, m = oracle.quantize_rowwise_fp8(x[None, :], None)
        amax = np.float32(np.abs(x.astype(np.float32)).max())
        assert m[0] == amax
        if amax == 0:
            assert not Xq.any()
            continue
        inv = np.float32(448.0) / amax
        for k in range(K):
            t = float(np.float32(x[k]) * inv)
            d = np.abs(pos - abs(t))
            best = np.flatnonzero(d == d.min())
            code = int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])
            assert Xq[0, k] == (code | (0x80 if np.signbit(np.float32(t)) else 0))


def _exact_fp8_case(rng, M, K, N):
    """X, W whose every non-outlier entry is an E4M3 value times a power of two
    set by its row (X) or column (W) absmax of 448 * 2^-r, so both quantizations
    are exact."""
    vals = oracle.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    vals = vals[vals >= 2.0 ** -6]  # normal values (exact in fp16 after the shift)

    def draw(rows, cols, axis):
        a = rng.choice(vals, size=(rows, cols)) * rng.choice([-1.0, 1.0], size=(rows, cols))
        if axis == 1:
            a[np.arange(rows), rng.integers(cols, size=rows)] = 448.0
            return a * np.exp2(-rng.integers(0, 6, size=(rows, 1)))
        a[rng.integers(rows, size=cols), np.arange(cols)] = -448.0
        return a * np.exp2(-rng.integers(4, 10, size=(1, cols)))

    Xd, Wd = draw(M, K, 1), draw(K, N, 0)
    X, W = Xd.astype(np.float16), Wd.astype(np.float16)
    assert np.array_equal(X.astype(np.float64), Xd) and np.array_equal(W.astype(np.float64), Wd)
    return X, W


def test_fp8_exact_codes_reduce_to_matmul():
    rng = np.random.default_rng(21)
    X, W = _exact_fp8_case(rng, 9, 40, 12)
    ref = oracle.linear_fp8(X, W, math.inf)
    exact = X.astype(np.float64) @ W.astype(np.float64)
    assert np.allclose(ref["Y"], exact, rtol=1e-12, atol=1e-12)
    # and the codes decode to the scaled inputs exactly
    deq = oracle.e4m3_value(ref["Xq"]) * ref["m"][:, None] / 448.0
    assert np.array_equal(deq, X.astype(np.float64))


def test_fp8_all_outlier_columns_reduce_to_fp16_matmul():
    X, W, _ = workloads.random_case(11, 64, 24, seed=8, n_out=2)
    ref = oracle.linear_fp8(X, W, 0.0)
    assert ref["idx"].size == 64 and not ref["Xq"].any() and not ref["m"].any()
    assert np.allclose(ref["Y"], X.astype(np.float64) @ W.astype(np.float64), rtol=1e-12,
                       atol=1e-12)


def test_fp8_reconstruction_error_bound():
    # |t - e4m3(t)| <= max(|t| 2^-4, 2^-10) for t = x * 448 / m (half a step of
    # 3 mantissa bits; subnormal steps are 2^-9), back in x units times m / 448,
    # plus the fp32 roundings inside x * fl(448 / m)
    X, _, _ = workloads.random_case(64, 512, 8, seed=15, n_out=5)
    idx = oracle.find_outliers(X, 6.0)
    Xq, m = oracle.quantize_rowwise_fp8(X, idx)
    keep = np.ones(X.shape[1], bool)
    keep[idx] = False
    xf = X.astype(np.float64)
    md = m.astype(np.float64)[:, None]
    err = np.abs(xf - oracle.e4m3_value(Xq) * md / 448.0)[:, keep]
    bound = (np.maximum(np.abs(xf) * 2.0 ** -4, md / 448.0 * 2.0 ** -10) * (1 + 2.0 ** -20)
             + np.abs(xf) * 2.0 ** -22)[:, keep]
    assert np.all(err <= bound)
    assert np.all(Xq[:, idx] == 0)


def test_fp8_layer_brute_force_against_torch_encoding():
    # an independent implementation of the FP8 layer: numpy arithmetic with
    # PyTorch's float8_e4m3fn cast as the encoder
    import torch
    X, W, _ = workloads.random_case(13, 48, 20, seed=31, n_out=3)
    thr = 6.0
    xf, wf = X.astype(np.float32), W.astype(np.float32)
    out = np.flatnonzero((np.abs(xf) >= thr).any(axis=0))
    keep = np.setdiff1d(np.arange(48), out)
    m = np.abs(xf[:, keep]).max(axis=1)
    s = np.abs(wf).max(axis=0)
    xs = (xf * (np.float32(448.0) / m)[:, None]).astype(np.float32)
    xs[:, out] = 0.0
    ws = (wf * (np.float32(448.0) / s)[None, :]).astype(np.float32)
    xc, wc = _torch_e4m3(xs), _torch_e4m3(ws.T)

    def dec(c):
        return torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()

    Cm = dec(xc) @ dec(wc).T
    Y = Cm * m[:, None].astype(np.float64) * s[None, :].astype(np.float64) / 448.0 ** 2 \
        + X[:, out].astype(np.float64) @ W[out].astype(np.float64)
    ref = oracle.linear_fp8(X, W, thr)
    assert ref["idx"].tolist() == out.tolist()
    assert np.array_equal(ref["Xq"], xc) and np.array_equal(ref["Wq"], wc)
    assert np.array_equal(ref["m"], m) and np.array_equal(ref["s"], s)
    assert np.allclose(ref["C"], Cm, rtol=1e-13, atol=1e-9)
    assert np.allclose(ref["Y"], Y, rtol=1e-12, atol=1e-12)
