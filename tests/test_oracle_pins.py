"""Pins of the oracle's order rules that no closed form fixes.

The pages name the categories a frozen profile has to fix (mojolearn PyPI page,
"What bitwise identity means": reduction order and partitioning, FMA policy,
transcendental spellings, tie rules) but print none of the concrete choices, so
the oracle's rules are a reading. Each rule is pinned here two ways: a literal
evaluator written in Python from the rule's statement (exact rational
arithmetic for every fused multiply-add, numpy binary32 scalars for every other
operation, each rounded once) must reproduce the oracle's bits, and a sabotage
arm of the oracle that changes only that rule must move them.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from bitwise_reproducible_fp32_amd import inputs as I

F32 = np.float32


def rn32(q: Fraction) -> np.float32:
    """The binary32 value nearest to the exact rational q (ties to even)."""
    c = F32(float(q))                   # within one binary32 step of the answer
    best = None
    for cand in (np.nextafter(c, F32(-np.inf)), c, np.nextafter(c, F32(np.inf))):
        if not np.isfinite(cand):
            continue
        err = abs(Fraction(float(cand)) - q)
        if best is None or err < best[0] or (err == best[0] and (int(cand.view(np.uint32)) & 1) == 0):
            best = (err, cand)
    return F32(best[1])


def fma_exact(a, b, c) -> np.float32:
    """RN(a*b + c) from the exact value (a, b, c binary32). An exact zero is
    +0, except that a zero product of negative sign plus -0 stays -0 (IEEE
    754 sign rule for sums of zeros)."""
    q = Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c))
    if q == 0:
        prod_is_neg_zero = (float(a) == 0 or float(b) == 0) and (np.signbit(a) != np.signbit(b))
        if prod_is_neg_zero and float(c) == 0 and np.signbit(c):
            return F32(-0.0)
        return F32(0.0)
    return rn32(q)


def bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).view(np.uint32)


# ------------------------------------------------------------------- W64
def w64_literal(vals, op, init):
    """Element i goes to lane i mod 64 in ascending i; then lane l takes
    op(lane l, lane l+s) for s = 32, 16, 8, 4, 2, 1; the result is lane 0."""
    acc = [init] * 64
    for i, v in enumerate(vals):
        acc[i % 64] = op(acc[i % 64], v)
    s = 32
    while s >= 1:
        for l in range(s):
            acc[l] = op(acc[l], acc[l + s])
        s //= 2
    return F32(acc[0])


def add32(a, b):
    return F32(F32(a) + F32(b))


def max_keep(a, b):
    return b if b > a else a     # ties keep the earlier operand


W64_SIZES = [1, 63, 64, 65, 767, 50257]


@pytest.mark.parametrize("n", W64_SIZES)
def test_sum64_and_max64_follow_the_lane_rule(n):
    rng = np.random.default_rng(100 + n)
    v = (rng.standard_normal(n) * np.exp(rng.uniform(-8, 8, n))).astype(np.float32)
    assert bits(oracle.sum64(v)) == bits(w64_literal(v, add32, F32(0.0)))
    assert bits(oracle.max64(v)) == bits(w64_literal(v, max_keep, F32(-np.inf)))


@pytest.mark.parametrize("n", [1, 63, 65, 767, 4099])
def test_dot64_follows_the_lane_rule(n):
    rng = np.random.default_rng(200 + n)
    a = rng.standard_normal(n).astype(np.float32)
    b = rng.standard_normal(n).astype(np.float32)
    acc = [F32(0.0)] * 64
    for i in range(n):
        acc[i % 64] = fma_exact(a[i], b[i], acc[i % 64])
    s = 32
    while s >= 1:
        for l in range(s):
            acc[l] = add32(acc[l], acc[l + s])
        s //= 2
    assert bits(oracle.dot64(a, b)) == bits(acc[0])


def test_w64_lane_rule_separates_block_assignment():
    """Dealing contiguous blocks to the lanes (a plausible misreading) gives
    other bits on ordinary rows, so the literal check above can tell them apart."""
    moved = 0
    for n in (767, 50257):
        v = np.random.default_rng(300 + n).standard_normal(n).astype(np.float32)
        want = bits(w64_literal(v, add32, F32(0.0)))
        oracle.set_sabotage(oracle.SABOTAGE["w64_blocks"])
        try:
            got = bits(oracle.sum64(v))
        finally:
            oracle.set_sabotage(0)
        moved += int(got != want)
    assert moved >= 1


def test_max64_tie_keeps_earlier_operand():
    # -0 and +0 compare equal: the lane keeps the one it saw first, and the
    # tree keeps the lower lane's value
    v = np.zeros(130, np.float32)
    v[0] = -0.0
    assert bits(oracle.max64(v)) == bits(F32(-0.0))
    v = np.zeros(130, np.float32)
    v[1] = -0.0
    assert bits(oracle.max64(v)) == bits(F32(0.0))


# ------------------------------------------------- RMSNorm gain gradient
def test_gain_gradient_follows_the_chunk_rule():
    """dw[c] over 2,500 rows: chunks of rows [0,1024), [1024,2048),
    [2048,2500), each an fma chain from +0 of dy[n,c] * RN(x[n,c] * r[n]) in
    ascending n, then chunk 0 + chunk 1, then + chunk 2."""
    rows, d = 2500, 6
    rng = np.random.default_rng(17)
    x = rng.standard_normal((rows, d)).astype(np.float32)
    dy = rng.standard_normal((rows, d)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    _, r = oracle.rmsnorm_fwd(x, w, 1e-6)
    _, dw = oracle.rmsnorm_bwd(dy, x, w, r)
    want = np.empty(d, np.float32)
    for c in range(d):
        total = None
        for c0 in range(0, rows, 1024):
            acc = F32(0.0)
            for n in range(c0, min(rows, c0 + 1024)):
                acc = fma_exact(dy[n, c], F32(x[n, c] * r[n]), acc)
            total = acc if total is None else add32(total, acc)
        want[c] = total
    assert np.array_equal(bits(dw), bits(want))


def test_gain_gradient_chunking_moves_bits():
    rows, d = 2500, 64
    rng = np.random.default_rng(18)
    x = rng.standard_normal((rows, d)).astype(np.float32)
    dy = rng.standard_normal((rows, d)).astype(np.float32)
    w = np.ones(d, np.float32)
    _, r = oracle.rmsnorm_fwd(x, w, 1e-6)
    _, good = oracle.rmsnorm_bwd(dy, x, w, r)
    oracle.set_sabotage(oracle.SABOTAGE["rms_dw_unchunked"])
    try:
        _, bad = oracle.rmsnorm_bwd(dy, x, w, r)
    finally:
        oracle.set_sabotage(0)
    assert np.any(bits(good) != bits(bad))


# ------------------------------------------------------- SwiGLU backward
def test_swiglu_backward_spelling():
    """du = dA * (g * sig); dsilu = sig * (1 + g * (1 - sig));
    dg = (dA * u) * dsilu, one binary32 rounding per operation, with sig the
    oracle's sigmoid (itself pinned through exp)."""
    rows, F = 64, 40
    rng = np.random.default_rng(19)
    gu = (rng.standard_normal((rows, 2 * F)) * 3).astype(np.float32)
    dA = rng.standard_normal((rows, F)).astype(np.float32)
    L = oracle.lib()
    dgu = np.empty_like(gu)
    L.orc_swiglu_bwd(dA, F, gu, rows, F, 2 * F, dgu)
    g, u = gu[:, :F], gu[:, F:]
    sig = np.empty_like(g)
    L.orc_sigmoid_array(np.ascontiguousarray(g).ravel(), sig.ravel(), g.size)
    one = F32(1.0)
    silu = g * sig
    dsilu = sig * (one + (g * (one - sig)))
    assert np.array_equal(bits(dgu[:, F:]), bits(dA * silu))
    assert np.array_equal(bits(dgu[:, :F]), bits((dA * u) * dsilu))
    oracle.set_sabotage(oracle.SABOTAGE["swiglu_bwd_spelling"])
    try:
        bad = np.empty_like(gu)
        L.orc_swiglu_bwd(dA, F, gu, rows, F, 2 * F, bad)
    finally:
        oracle.set_sabotage(0)
    assert np.any(bits(bad[:, :F]) != bits(dgu[:, :F]))


def test_sigmoid_is_one_over_one_plus_exp():
    x = np.random.default_rng(20).standard_normal(4096).astype(np.float32) * 8
    s = np.empty_like(x)
    oracle.lib().orc_sigmoid_array(x, s, x.size)
    want = F32(1.0) / (F32(1.0) + oracle.exp(-x))
    assert np.array_equal(bits(s), bits(want))


# ------------------------------------------------- attention dS spelling
def test_attention_ds_spelling_through_unit_keys():
    """With k_j and v_j the unit vectors e_j (T <= hd), dP_ij = dO_i[j] and
    dq_i[j] = dS_ij exactly (one nonzero term per chain), so the oracle's dq
    exposes dS: dS_ij = (P_ij * (dP_ij - D_i)) * scale with D_i = DOT64(dO_i,
    O_i) and scale = RN(1/sqrt(hd))."""
    BH, T, hd = 2, 16, 16
    rng = np.random.default_rng(21)
    q = rng.standard_normal((BH, T, hd)).astype(np.float32)
    eye = np.broadcast_to(np.eye(T, hd, dtype=np.float32), (BH, T, hd)).copy()
    P, O = oracle.attention_fwd(q, eye, eye)
    dO = rng.standard_normal((BH, T, hd)).astype(np.float32)
    dq, _, dv = oracle.attention_bwd(q, eye, eye, P, O, dO)
    scale = F32(oracle.lib().orc_attn_scale(hd))
    assert bits(scale) == bits(F32(0.25))
    for z in range(BH):
        for i in range(T):
            acc = [F32(0.0)] * 64
            for c in range(hd):
                acc[c % 64] = fma_exact(dO[z, i, c], O[z, i, c], acc[c % 64])
            s = 32
            while s >= 1:
                for l in range(s):
                    acc[l] = add32(acc[l], acc[l + s])
                s //= 2
            D = acc[0]
            for j in range(i + 1):
                ds = F32(F32(P[z, i, j] * F32(dO[z, i, j] - D)) * scale)
                want = F32(ds + F32(0.0))          # the chain starts from +0
                assert bits(dq[z, i, j]) == bits(want), (z, i, j)
            assert np.all(bits(dq[z, i, i + 1:]) == 0)
    oracle.set_sabotage(oracle.SABOTAGE["ds_spelling"])
    try:
        bad, _, _ = oracle.attention_bwd(q, eye, eye, P, O, dO)
    finally:
        oracle.set_sabotage(0)
    assert np.any(bits(bad) != bits(dq))


# ------------------------------------------------- AdamW bias corrections
@pytest.mark.parametrize("t", [1, 2, 7, 250, 5000])
@pytest.mark.parametrize("beta_bits", [0x3F666666, 0x3F733333])
def test_bias_correction(t, beta_bits):
    """bc_t = RN(1 - beta^t) with beta^t a product of the binary32 beta in
    binary64 (t roundings), and within one binary32 step of the exact value."""
    beta = np.uint32(beta_bits).view(np.float32)
    got = F32(oracle.lib().orc_bias_correction(beta, t))
    p = 1.0
    for _ in range(t):
        p *= float(beta)
    assert bits(got) == bits(F32(1.0 - p))
    exact = rn32(1 - Fraction(float(beta)) ** t)
    assert abs(int(bits(got)) - int(bits(exact))) <= 1


# ------------------------------------------------- learning-rate table
def test_learning_rate_table():
    # warmup: lr_t = 6e-4 * t / 250 rounded once; the two steps the oracle
    # checks at full size take 0x36210FB0 and 0x36A10FB0
    assert bits(F32(I.lr_at("c4", 1))) == 0x36210FB0
    assert bits(F32(I.lr_at("c4", 2))) == 0x36A10FB0
    assert F32(I.lr_at("c4", 250)) == F32(6e-4)
    assert F32(I.lr_at("c4", 5000)) == F32(6e-5)
    assert I.lr_at("c4", 2625) == pytest.approx(0.5 * (6e-4 + 6e-5), rel=1e-6)
