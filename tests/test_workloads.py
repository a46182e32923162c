"""The seeded input generator: deterministic, right shapes, planted columns."""
import numpy as np

import workloads


def test_deterministic_and_shaped():
    wl = workloads.WORKLOADS["tiny"]
    a, b = workloads.make_x(wl), workloads.make_x(wl)
    assert a.dtype == np.float16 and a.shape == (16, 256)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    w = workloads.make_w(wl)
    assert w.dtype == np.float16 and w.shape == (256, 128)


def test_planted_columns_are_stable_across_tokens():
    wl = workloads.WORKLOADS["tiny"]
    x = workloads.make_x(wl).astype(np.float32)
    for c in wl.fixed_cols:
        col = x[:, c]
        assert np.all(np.abs(col) >= wl.out_lo) and np.all(np.abs(col) <= wl.out_hi)
        assert np.all(np.sign(col) == np.sign(col[0]))


def test_per_call_outlier_sets_differ():
    wl = workloads.WORKLOADS["70b"]
    sets = [workloads.planted_columns(wl, c) for c in range(4)]
    for s in sets:
        assert 8 <= s.size <= 81 and np.all(np.diff(s) > 0)
    assert len({tuple(s.tolist()) for s in sets}) == 4


def test_rows_slice_matches_full():
    wl = workloads.WORKLOADS["decode"]
    full = workloads.make_x(wl)
    part = workloads.make_x(wl, rows=slice(3, 9))
    assert np.array_equal(full[3:9].view(np.uint16), part.view(np.uint16))
