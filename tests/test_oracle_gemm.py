"""Pins of the G1024 contraction: exact results on integer-valued data (which
fix indexing, strides, segments, causal ranges and masks independently of
the order), a literal element-by-element evaluation of the chunk rule on
small cases, the float64 error bound, degenerate sizes, and the sabotage
arms that change the order."""
import numpy as np
import pytest

import oracle

KC = 1024


def ints(shape, seed, lo=-8, hi=9):
    return np.random.default_rng(seed).integers(lo, hi, shape).astype(np.float32)


def ref_int(A, B, krange=0, kseg=None):
    """Exact int64 contraction with the causal ranges applied."""
    A64, B64 = A.astype(np.int64), B.astype(np.int64)
    M, K = A.shape
    if krange == 0:
        return A64 @ B64
    k = np.arange(K)[None, :]
    i = np.arange(M)[:, None]
    mask = (k <= i) if krange == 1 else (k >= i)
    return (A64 * mask) @ B64


@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (37, 767, 5), (129, 3, 257), (64, 2600, 33)])
def test_forward_form_integer_exact(M, K, N):
    X, W = ints((M, K), 1), ints((N, K), 2)
    Y = oracle.linear(X, W)
    assert np.array_equal(Y.astype(np.int64), X.astype(np.int64) @ W.astype(np.int64).T)


@pytest.mark.parametrize("layout", ["nn", "tn"])
def test_transposed_layouts_integer_exact(layout):
    M, K, N = 45, 2100, 19
    A, B = ints((M, K), 3), ints((K, N), 4)
    if layout == "nn":
        C = oracle.gemm(A, B, M, N, K, K, 1, N, 1).reshape(M, N)
    else:
        At = np.ascontiguousarray(A.T)               # stored [K, M]
        C = oracle.gemm(At, B, M, N, K, 1, M, N, 1).reshape(M, N)
    assert np.array_equal(C.astype(np.int64), ref_int(A, B))


@pytest.mark.parametrize("krange", [1, 2])
def test_causal_ranges_integer_exact(krange):
    T, hd = 2100, 7
    A, B = ints((T, T), 5, -3, 4), ints((T, hd), 6)
    C = oracle.gemm(A, B, T, hd, T, T, 1, hd, 1, krange=krange).reshape(T, hd)
    assert np.array_equal(C.astype(np.int64), ref_int(A, B, krange))


def test_segments_integer_exact():
    N, d, nseg = 9, 40, 3
    A, B = ints((N, nseg * d), 7), ints((nseg * d, d), 8)
    C = oracle.gemm(A, B, N, d, nseg * d, nseg * d, 1, d, 1, kseg=d).reshape(N, d)
    assert np.array_equal(C.astype(np.int64), A.astype(np.int64) @ B.astype(np.int64))


def test_modes_and_outmask():
    M, K = 33, 10
    A, B = ints((M, K), 9), ints((K, M), 10)
    base = np.full((M, M), 5.0, np.float32)
    C = oracle.gemm(A, B, M, M, K, K, 1, M, 1, C=base.copy().ravel(), mode=1).reshape(M, M)
    assert np.array_equal(C, (A.astype(np.int64) @ B.astype(np.int64) + 5).astype(np.float32))
    C = oracle.gemm(A, B, M, M, K, K, 1, M, 1, C=base.copy().ravel(), mode=2, scale=0.5,
                    outmask=1).reshape(M, M)
    full = (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float32) * np.float32(0.5)
    low = np.tril(np.ones((M, M), bool))
    assert np.array_equal(C[low], full[low]) and np.all(C[~low] == 5.0)


def test_empty_contraction_is_positive_zero():
    C = oracle.gemm(np.zeros(4, np.float32), np.zeros(4, np.float32), 2, 2, 0, 0, 0, 0, 0)
    assert np.all(C.view(np.uint32) == 0)


def chain_rule_literal(A, B, rows, krange=0, kseg=None):
    """The chunk rule evaluated one output at a time with the oracle's fma."""
    M, K = A.shape
    N = B.shape[1]
    kseg = kseg or K
    fma = oracle.lib().orc_fma
    out = np.zeros((len(rows), N), np.float32)
    for r, i in enumerate(rows):
        lo, hi = (0, K) if krange == 0 else ((0, min(K, i + 1)) if krange == 1 else (i, K))
        for j in range(N):
            total = None
            for s in range(K // kseg):
                for c0 in range(0, kseg, KC):
                    l0 = max(s * kseg + c0, lo)
                    l1 = min(s * kseg + min(c0 + KC, kseg), hi)
                    if l0 >= l1:
                        continue
                    acc = 0.0
                    for k in range(l0, l1):
                        acc = fma(float(A[i, k]), float(B[k, j]), acc)
                    total = np.float32(acc) if total is None else np.float32(total + np.float32(acc))
            out[r, j] = np.float32(0.0) if total is None else total
    return out


@pytest.mark.parametrize("M,K,N,krange,kseg", [(1, 1, 1, 0, None), (3, 2500, 2, 0, None),
                                               (2, 2400, 2, 0, 800), (2060, 2060, 2, 1, None),
                                               (2060, 2060, 2, 2, None)])
def test_chunk_rule_literal(M, K, N, krange, kseg):
    rng = np.random.default_rng(M * 7 + K)
    A = (rng.uniform(-1, 1, (M, K)) * np.exp2(rng.integers(-10, 10, (M, K)))).astype(np.float32)
    B = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    rows = list(range(M)) if M < 8 else [0, 1, 1023, 1024, 1500, M - 1]
    C = oracle.gemm_rows(A, B, M, N, K, K, 1, N, 1, rows, kseg=kseg or K, krange=krange)
    lit = chain_rule_literal(A, B, rows, krange, kseg)
    assert np.array_equal(C.view(np.uint32), lit.view(np.uint32))


@pytest.mark.parametrize("K", [767, 3000, 50257])
def test_float_error_bound(K):
    rng = np.random.default_rng(K)
    M, N = 3, 4
    A, B = rng.uniform(-1, 1, (M, K)).astype(np.float32), rng.uniform(-1, 1, (K, N)).astype(np.float32)
    C = oracle.gemm(A, B, M, N, K, K, 1, N, 1).reshape(M, N)
    exact = A.astype(np.float64) @ B.astype(np.float64)
    bound = (min(K, KC) + K // KC + 1) * 2.0 ** -24 * (np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64))
    assert np.all(np.abs(C - exact) <= bound)


def test_gemm_rows_matches_gemm():
    rng = np.random.default_rng(11)
    A, B = rng.uniform(-1, 1, (50, 1500)).astype(np.float32), rng.uniform(-1, 1, (1500, 9)).astype(np.float32)
    C = oracle.gemm(A, B, 50, 9, 1500, 1500, 1, 9, 1).reshape(50, 9)
    rows = np.array([0, 17, 49])
    Cr = oracle.gemm_rows(A, B, 50, 9, 1500, 1500, 1, 9, 1, rows)
    assert np.array_equal(C[rows].view(np.uint32), Cr.view(np.uint32))


@pytest.mark.parametrize("arm", ["gemm_reverse_k", "gemm_kc512", "gemm_pairwise_chunks", "gemm_mul_add"])
def test_sabotage_changes_bits(arm):
    rng = np.random.default_rng(12)
    K = 3100
    A = (rng.uniform(-1, 1, (8, K)) * np.exp2(rng.integers(-12, 12, (8, K)))).astype(np.float32)
    B = rng.uniform(-1, 1, (K, 8)).astype(np.float32)
    good = oracle.gemm(A, B, 8, 8, K, K, 1, 8, 1)
    oracle.set_sabotage(oracle.SABOTAGE[arm])
    try:
        bad = oracle.gemm(A, B, 8, 8, K, K, 1, 8, 1)
    finally:
        oracle.set_sabotage(0)
    assert np.any(good.view(np.uint32) != bad.view(np.uint32))


def test_threads_do_not_change_bits():
    rng = np.random.default_rng(13)
    A, B = rng.uniform(-1, 1, (300, 2100)).astype(np.float32), rng.uniform(-1, 1, (2100, 70)).astype(np.float32)
    oracle.set_threads(1)
    one = oracle.gemm(A, B, 300, 70, 2100, 2100, 1, 70, 1)
    oracle.set_threads(4)
    try:
        four = oracle.gemm(A, B, 300, 70, 2100, 2100, 1, 70, 1)
    finally:
        oracle.set_threads(1)
    assert np.array_equal(one.view(np.uint32), four.view(np.uint32))
