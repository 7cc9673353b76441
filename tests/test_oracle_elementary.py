"""Pins of the oracle's exp/log spellings and of its arithmetic environment.

exp_p and log_p are the profile's own spellings (Cody-Waite reduction with a
Taylor polynomial; atanh series), so the pins are mathematical: closeness to
binary64 exp/log, exact special values, the overflow/underflow thresholds,
monotonicity, and the absence of flush-to-zero."""
import math
import struct

import numpy as np
import pytest

import oracle


def f(u):
    return struct.unpack("<f", struct.pack("<I", u))[0]


def bits(x):
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def ulp_err(got, ref):
    got = got.astype(np.float64)
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ue = np.maximum(e - 23, -149)
    return np.abs(got - ref) / np.exp2(ue)


@pytest.fixture(scope="module")
def sample():
    u = np.arange(0, 1 << 32, 4099, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    return x[np.isfinite(x)]


def test_no_ftz_daz():
    assert oracle.lib().orc_ftz_daz_set() == 0


def test_exp_within_one_ulp_of_binary64(sample):
    x = sample[(sample > -103.9) & (sample < 88.7)]
    y = oracle.exp(x)
    ref = np.exp(x.astype(np.float64))
    assert ulp_err(y, ref).max() <= 1.0


def test_log_within_two_ulp_of_binary64(sample):
    x = sample[sample > 0]
    y = oracle.log(x)
    ref = np.log(x.astype(np.float64))
    assert ulp_err(y, ref).max() <= 2.0


def test_special_values():
    E, L = oracle.lib().orc_exp, oracle.lib().orc_log
    assert bits(E(0.0)) == 0x3F800000 and bits(E(-0.0)) == 0x3F800000
    assert bits(L(1.0)) == 0x00000000
    assert E(float("inf")) == float("inf") and bits(E(float("-inf"))) == 0
    assert math.isnan(E(float("nan"))) and math.isnan(L(float("nan")))
    assert L(0.0) == float("-inf") and L(-0.0) == float("-inf")
    assert math.isnan(L(-1.0)) and math.isnan(L(float("-inf")))
    assert L(float("inf")) == float("inf")


def test_exp_thresholds():
    E = oracle.lib().orc_exp
    assert math.isfinite(E(f(0x42B17217))) and E(f(0x42B17218)) == float("inf")
    # exp just above ln(2^-150) rounds up to the smallest subnormal; at the threshold it is 0
    assert bits(E(f(0xC2CFF1B4))) == 0x00000001
    assert bits(E(f(0xC2CFF1B5))) == 0x00000000


def test_exp_subnormal_results_no_flush():
    x = np.float32([-90.0, -95.0, -100.0, -103.0])
    y = oracle.exp(x)
    assert np.all(y > 0)
    ref = np.exp(x.astype(np.float64))
    assert np.all(np.abs(y - ref) <= 2.0 ** -149)


def test_log_subnormal_inputs():
    x = np.array([f(1), f(2), f(0x00400000), f(0x007FFFFF)], dtype=np.float32)
    y = oracle.log(x)
    ref = np.log(x.astype(np.float64))
    assert ulp_err(y, ref).max() <= 2.0


def test_monotone(sample):
    x = np.sort(sample[(sample > -110) & (sample < 88.7)])
    assert np.all(np.diff(oracle.exp(x).astype(np.float64)) >= 0)
    x = np.sort(sample[sample > 0])
    assert np.all(np.diff(oracle.log(x).astype(np.float64)) >= 0)


def test_fma_single_rounding():
    a = b = np.float32(1 + 2 ** -12)
    c = np.float32(-1.0)
    fused = oracle.fma(a, b, c)[()]
    assert fused == np.float32(2 ** -11 + 2 ** -24)      # exact product kept
    assert np.float32(a * b) + c == np.float32(2 ** -11)  # the unfused value differs


def test_sabotaged_exp_differs():
    x = oracle.f32a(np.linspace(-20, 20, 4001))
    good = oracle.exp(x)
    oracle.set_sabotage(oracle.SABOTAGE["libm_exp"])
    try:
        bad = oracle.exp(x)
    finally:
        oracle.set_sabotage(0)
    assert np.any(good.view(np.uint32) != bad.view(np.uint32))


def test_ftz_arm_flushes_subnormals():
    x = np.float32([-100.0])
    good = oracle.exp(x)
    oracle.set_threads(1)
    oracle.set_sabotage(oracle.SABOTAGE["ftz_daz"])
    try:
        bad = oracle.exp(x)
        assert oracle.lib().orc_ftz_daz_set() == 1
    finally:
        oracle.set_sabotage(0)
    assert good[0] > 0 and bad[0] == 0
    assert oracle.lib().orc_ftz_daz_set() == 0
