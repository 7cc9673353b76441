"""Pins of the W64 row reductions: exact results on integer data, the float64
error bound, the tie rule of MAX on signed zeros, empty rows, and the
sabotage arms that change the lane tree."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("n", [0, 1, 7, 63, 64, 65, 767, 768, 4099])
def test_integer_rows_exact(n):
    rng = np.random.default_rng(n)
    v = rng.integers(-1000, 1000, n).astype(np.float32)
    w = rng.integers(-30, 30, n).astype(np.float32)
    assert oracle.sum64(v) == np.float32(int(v.astype(np.int64).sum()))
    assert oracle.dot64(v, w) == np.float32(int((v.astype(np.int64) * w.astype(np.int64)).sum()))
    if n:
        assert oracle.max64(v) == v.max()


def test_empty_rows():
    assert np.float32(oracle.sum64(np.zeros(0))).tobytes() == np.float32(0.0).tobytes()
    assert oracle.max64(np.zeros(0)) == -np.inf


@pytest.mark.parametrize("n", [5, 64, 1000, 50257])
def test_float_error_bound(n):
    v = np.random.default_rng(n).uniform(-1, 1, n).astype(np.float32)
    exact = v.astype(np.float64).sum()
    gamma = n * 2.0 ** -24 / (1 - n * 2.0 ** -24)
    assert abs(float(oracle.sum64(v)) - exact) <= gamma * np.abs(v).astype(np.float64).sum()


def test_max_tie_keeps_earlier_operand():
    # lane 0 holds the first element, lane 1 the second; equal values keep lane 0
    assert np.float32(oracle.max64(np.float32([-0.0, 0.0]))).tobytes() == np.float32(-0.0).tobytes()
    assert np.float32(oracle.max64(np.float32([0.0, -0.0]))).tobytes() == np.float32(0.0).tobytes()


@pytest.mark.parametrize("arm", ["w64_mirror_pairing", "w32_lanes"])
def test_tree_sabotage_changes_bits(arm):
    # 32 rows of 4096 positive values: a different lane tree changes the last
    # rounding of some rows (any single row only with probability about 1/2)
    rows = np.random.default_rng(3).uniform(0, 1, (32, 4096)).astype(np.float32)
    good = [np.float32(oracle.sum64(r)).tobytes() for r in rows]
    oracle.set_sabotage(oracle.SABOTAGE[arm])
    try:
        bad = [np.float32(oracle.sum64(r)).tobytes() for r in rows]
    finally:
        oracle.set_sabotage(0)
    assert good != bad
