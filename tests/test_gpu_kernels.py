"""Kernel-level parity on the GPU against the oracle, called through the C ABI:
the matrix-core probe, exp/log spellings, the G1024 contraction on odd shapes,
layouts, causal ranges and segments, launch-geometry perturbation, and each row
operation of the step (RMSNorm, RoPE, attention, SwiGLU, cross-entropy,
embedding scatter, AdamW)."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_bits, bits_equal, dev, diff_report, empty, host

pytestmark = pytest.mark.gpu


@pytest.fixture()
def oracle_threads():
    """The oracle on the host's cores (at most 16) for the tests that compare
    whole full-size outputs, back to its previous thread count afterwards."""
    import os
    before = oracle.lib().orc_get_threads()
    oracle.set_threads(min(16, len(os.sched_getaffinity(0))))
    yield
    oracle.set_threads(before)


@pytest.fixture(scope="module")
def mlb():
    import bitwise_reproducible_fp32_amd as m
    return m


# ------------------------------------------------------------ matrix-core probe
PROBE = {0: (32, 1), 1: (16, 1), 2: (4, 1), 3: (16, 2), 4: (4, 4)}   # variant: (outputs per lane, K)


def rnd_operands(rng, n):
    cls = rng.integers(0, 4, n)
    mant = rng.uniform(1, 2, n) * np.where(rng.integers(0, 2, n) == 0, 1, -1)
    e = np.where(cls == 0, rng.integers(-20, 21, n), np.where(cls == 2, rng.integers(-80, -59, n),
                                                             rng.integers(-130, 121, n)))
    x = (mant * np.exp2(e.astype(np.float64))).astype(np.float32)
    spec = rng.integers(0, 8, n)
    x = np.where((cls == 3) & (spec == 0), np.float32(0.0), x)
    x = np.where((cls == 3) & (spec == 1), np.float32(-0.0), x)
    return x.astype(np.float32)


@pytest.mark.parametrize("variant", sorted(PROBE))
def test_mfma_is_an_ascending_fma_chain(mlb, variant):
    """Every FP32 MFMA output equals fma chains over its k-lanes in ascending
    order, with IEEE denormals (the fact the contraction kernels rely on)."""
    R, K = PROBE[variant]
    nw = 128 + 512
    rng = np.random.default_rng(variant)
    A = np.zeros(nw * 64, np.float32)
    B = np.zeros(nw * 64, np.float32)
    # waves 0..63: one-hot A lanes, waves 64..127: one-hot B lanes (layout discovery)
    for w in range(64):
        A[w * 64 + w] = 1.0; B[w * 64:(w + 1) * 64] = 1.0
        A[(64 + w) * 64:(65 + w) * 64] = 1.0; B[(64 + w) * 64 + w] = 1.0
    A[128 * 64:] = rnd_operands(rng, (nw - 128) * 64)
    B[128 * 64:] = rnd_operands(rng, (nw - 128) * 64)
    Cin = np.zeros(nw * 64 * R, np.float32)
    Cin[128 * 64 * R:] = rnd_operands(rng, (nw - 128) * 64 * R)
    D = empty(nw * 64 * R)
    mlb.diag_mfma(variant, dev(A), dev(B), dev(Cin), D, nw)
    out = host(D).reshape(nw, 64, R)
    SA = [[np.nonzero(out[:64, l, r])[0] for r in range(R)] for l in range(64)]
    SB = [[np.nonzero(out[64:128, l, r])[0] for r in range(R)] for l in range(64)]
    assert all(len(SA[l][r]) == K and len(SB[l][r]) == K for l in range(64) for r in range(R))
    got = out[128:]
    a = A.reshape(nw, 64)[128:]
    b = B.reshape(nw, 64)[128:]
    c = Cin.reshape(nw, 64, R)[128:]
    for l in range(64):
        for r in range(R):
            acc = c[:, l, r]
            for k in range(K):      # ascending lane order = ascending k
                acc = oracle.fma(a[:, SA[l][r][k]], b[:, SB[l][r][k]], acc)
            assert_bits(f"variant {variant} lane {l} reg {r}", got[:, l, r], acc)


# ------------------------------------------------------------------ exp / log
# signed zeros, infinities, NaNs, the exp range ends and their neighbours, the
# edges of the normal and subnormal scale ranges of exp, subnormals
SPECIAL = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00000, 0x7FA00001,
                    0x42B17217, 0x42B17218, 0x42B17219, 0xC2CFF1B4, 0xC2CFF1B5, 0xC2CFF1B6, 0x42AE0000, 0x42B00000,
                    0xC2AE0000, 0xC2B00000, 0xC2B20000, 0xC2C80000, 0x00000001, 0x007FFFFF, 0x00800000,
                    0x3F800000, 0xBF800000, 0x3F317218, 0xBF317218], dtype=np.uint32)


def test_elementary_spellings_match_oracle_on_every_input(mlb):
    """exp, log, the branch-free exp the cross-entropy uses and the sigmoid on
    all 2^32 binary32 inputs, in chunks of 2^28, against the oracle bit for
    bit (NaN payloads canonicalised)."""
    import os
    import torch
    oracle.set_threads(min(16, len(os.sched_getaffinity(0))))
    chunk = 1 << 28
    y = empty(chunk)
    names = ["exp", "log", "sigmoid", "exp (branch-free)"]
    try:
        for c in range(1 << 32 >> 28):
            x = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
            xd = dev(x)
            want_exp = oracle.exp(x)
            want = {0: want_exp, 3: want_exp, 1: oracle.log(x)}
            want[2] = np.empty_like(x)
            oracle.lib().orc_sigmoid_array(x, want[2], x.size)
            for which in (0, 3, 1, 2):
                mlb.unary(xd, y, chunk, which)
                got = host(y)
                if not bits_equal(got, want[which]):
                    raise AssertionError(f"chunk {c}: " + diff_report(names[which], got, want[which]))
            del xd
            torch.cuda.synchronize()
    finally:
        oracle.set_threads(1)


@pytest.mark.parametrize("which", [0, 1, 2, 3])
def test_elementary_spellings_special_inputs(mlb, which):
    """The special inputs on their own: signed zeros, infinities, NaNs, the
    range ends of exp and their neighbours, subnormals."""
    x = SPECIAL.view(np.float32)
    y = empty(x.size)
    mlb.unary(dev(x), y, x.size, which)
    if which == 2:
        want = np.empty_like(x)
        oracle.lib().orc_sigmoid_array(x, want, x.size)
    else:
        want = (oracle.exp, oracle.log, None, oracle.exp)[which](x)
    assert_bits(["exp", "log", "sigmoid", "exp (branch-free)"][which], host(y), want)


# --------------------------------------------------------------- contractions
def make(rng, shape):
    return rng.uniform(-1, 1, shape).astype(np.float32)


def orc_contract(A, B, M, N, K, lda, a_kc, ldb, b_kc, kseg=0, krange=0, outmask=0, mode=0, scale=1.0, C0=None):
    sam, sak = (lda, 1) if a_kc else (1, lda)
    sbk, sbn = (1, ldb) if b_kc else (ldb, 1)
    C = np.zeros(M * N, np.float32) if C0 is None else C0.copy().ravel()
    return oracle.gemm(A.ravel(), B.ravel(), M, N, K, sam, sak, sbk, sbn, C=C, kseg=kseg or K, mode=mode,
                       scale=scale, krange=krange, outmask=outmask).reshape(M, N)


SHAPES = [(1, 1, 1), (37, 767, 5), (129, 3, 257), (200, 2100, 130), (64, 64, 64), (300, 1030, 70), (200, 2100, 132),
          (136, 1500, 68)]


@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("layout", ["nt", "nn", "tn", "tt"])
def test_contraction_odd_shapes(mlb, M, K, N, layout):
    rng = np.random.default_rng(M + K + N)
    a_kc, b_kc = layout[0] == "n", layout[1] == "t"
    A = make(rng, (M, K) if a_kc else (K, M))
    B = make(rng, (N, K) if b_kc else (K, N))
    lda = K if a_kc else M
    ldb = K if b_kc else N
    want = orc_contract(A, B, M, N, K, lda, a_kc, ldb, b_kc)
    for tile in (0, 1, 2):
        C = empty(M * N)
        mlb.gemm(dev(A), dev(B), C, M, N, K, lda, a_kc, ldb, b_kc, N, tile=tile)
        assert_bits(f"{layout} tile {tile}", host(C).reshape(M, N), want)
    C = empty(M * N)
    mlb.gemm(dev(A), dev(B), C, M, N, K, lda, a_kc, ldb, b_kc, N, simple=1)
    assert_bits(f"{layout} simple", host(C).reshape(M, N), want)


@pytest.mark.parametrize("K", [2048, 3000, 8192])
def test_split_chunks_same_bits(mlb, K):
    """Per-chunk partials folded by a second kernel equal the in-kernel fold."""
    rng = np.random.default_rng(K)
    M, N = 96, 160
    A, B = make(rng, (K, M)), make(rng, (K, N))
    want = orc_contract(A, B, M, N, K, M, False, N, False)
    ws = empty((K + 1023) // 1024 * M * N)
    for split in (0, 1):
        C = empty(M * N)
        mlb.gemm(dev(A), dev(B), C, M, N, K, M, False, N, False, N, split=split, ws=ws)
        assert_bits(f"split {split}", host(C).reshape(M, N), want)


def test_segments_and_modes(mlb):
    rng = np.random.default_rng(5)
    M, d, F = 70, 96, 1056   # two segments of 1056 -> chunks 1024 + 32 each
    A, B = make(rng, (M, 2 * F)), make(rng, (2 * F, d))
    C0 = make(rng, (M, d))
    want = orc_contract(A, B, M, d, 2 * F, 2 * F, True, d, False, kseg=F, mode=1, C0=C0)
    C = dev(C0.copy())
    mlb.gemm(dev(A), dev(B), C, M, d, 2 * F, 2 * F, True, d, False, d, kseg=F, mode=1)
    assert_bits("segments accumulate", host(C), want)
    want = orc_contract(A, B, M, d, 2 * F, 2 * F, True, d, False, kseg=F, mode=2, scale=0.375)
    C = empty(M * d)
    mlb.gemm(dev(A), dev(B), C, M, d, 2 * F, 2 * F, True, d, False, d, kseg=F, mode=2, scale=0.375)
    assert_bits("segments scaled", host(C).reshape(M, d), want)


@pytest.mark.parametrize("krange", [1, 2])
@pytest.mark.parametrize("T,hd", [(64, 8), (300, 5), (1100, 64), (2300, 16)])
def test_causal_ranges(mlb, krange, T, hd):
    """Both launch forms of a causal contraction over several chunks (one
    launch per chunk, or the running total in registers) and the one-thread
    reference kernel give the oracle's bits."""
    rng = np.random.default_rng(T * krange)
    P = make(rng, (T, T))
    V = make(rng, (T, hd))
    if krange == 1:   # O[i] = sum_{j<=i} P[i,j] V[j]
        want = orc_contract(P, V, T, hd, T, T, True, hd, False, krange=1)
        a_kc = True
    else:             # dV[j] = sum_{i>=j} P[i,j] dO[i]
        want = orc_contract(P, V, T, hd, T, T, False, hd, False, krange=2)
        a_kc = False
    for simple, split in ((0, -1), (0, 0), (0, 1), (1, -1)):
        C = dev(np.full(T * hd, np.nan, np.float32))
        mlb.gemm(dev(P), dev(V), C, T, hd, T, T, a_kc, hd, False, hd, krange=krange, simple=simple, split=split)
        assert_bits(f"krange {krange} simple {simple} split {split}", host(C).reshape(T, hd), want)


@pytest.mark.parametrize("a_kc", [False, True])
def test_accumulate_rows_without_terms(mlb, a_kc):
    """k >= i with more rows than K: rows i >= K have an empty contraction
    (+0), and accumulate mode gives C + (+0) there, which turns -0 into +0, on
    every launch form."""
    rng = np.random.default_rng(31)
    M, K, N = 300, 100, 40
    A = make(rng, (M, K) if a_kc else (K, M))
    B = make(rng, (K, N))
    C0 = make(rng, (M, N))
    C0[rng.random((M, N)) < 0.3] = -0.0
    lda = K if a_kc else M
    want = orc_contract(A, B, M, N, K, lda, a_kc, N, False, krange=2, mode=1, C0=C0)
    assert np.any(np.signbit(C0[K:]) & (C0[K:] == 0)) and not np.any(np.signbit(want[K:]) & (want[K:] == 0))
    for simple, split in ((0, -1), (0, 0), (0, 1), (1, -1)):
        C = dev(C0.ravel())
        mlb.gemm(dev(A), dev(B), C, M, N, K, lda, a_kc, N, False, N, krange=2, mode=1, simple=simple, split=split)
        assert_bits(f"a_kc {a_kc} simple {simple} split {split}", host(C).reshape(M, N), want)


def test_outmask_scores(mlb):
    rng = np.random.default_rng(9)
    T, hd = 300, 64
    q, k = make(rng, (T, hd)), make(rng, (T, hd))
    sc = np.float32(0.125)
    want = orc_contract(q, k, T, T, hd, hd, True, hd, True, mode=2, scale=sc, outmask=1)
    C = dev(np.full((T, T), 7.0, np.float32))
    mlb.gemm(dev(q), dev(k), C, T, T, hd, hd, True, hd, True, T, mode=2, scale=sc, outmask=1)
    got = host(C)
    low = np.tril(np.ones((T, T), bool))
    assert_bits("lower triangle", got[low], want[low])
    assert np.all(got[~low] == 7.0)


SWEEP = [(8192, 768, 2304), (8192, 768, 2048), (8192, 2048, 768), (8192, 768, 50257)]


@pytest.mark.parametrize("M,K,N", SWEEP)
def test_sweep_forward_shapes(mlb, oracle_threads, M, K, N):
    """The 162M model's forward contractions at full size as standalone calls,
    every output against the oracle (the 50,257-wide head included)."""
    rng = np.random.default_rng(7)
    X, W = make(rng, (M, K)), make(rng, (N, K))
    C = empty(M * N)
    mlb.gemm(dev(X), dev(W), C, M, N, K, K, True, K, True, N)
    got = host(C).reshape(M, N)
    del C
    want = oracle.gemm_rows(X.ravel(), W.ravel(), M, N, K, K, 1, 1, K, np.arange(M))
    assert_bits(f"{M}x{K}x{N}", got, want)


def test_sweep_weight_gradient_shape(mlb, oracle_threads):
    """768 x 8192 x 768: dY^T X over 8192 rows (8 chunks), both fold paths,
    every output against the oracle."""
    rng = np.random.default_rng(8)
    n, o, i = 8192, 768, 768
    dY, X = make(rng, (n, o)), make(rng, (n, i))
    rows = np.arange(o)
    want = oracle.gemm_rows(dY.ravel(), X.ravel(), o, i, n, 1, o, i, 1, rows)
    ws = empty(8 * o * i)
    for split in (0, 1):
        C = empty(o * i)
        mlb.gemm(dev(dY), dev(X), C, o, i, n, o, False, i, False, i, split=split, ws=ws)
        assert_bits(f"dW split {split}", host(C).reshape(o, i)[rows], want)


@pytest.mark.parametrize("M0,N0,M1,N1,K,layout", [(2304, 768, 768, 768, 2048, "tn"), (300, 100, 129, 260, 3000, "tn"),
                                                   (200, 132, 70, 96, 700, "nn"), (130, 97, 64, 200, 1500, "nt")])
@pytest.mark.parametrize("mode", [0, 1])
def test_contraction_pair(mlb, M0, N0, M1, N1, K, layout, mode):
    """Two contractions in one launch (as the step runs the q/k/v and Wo weight
    gradients): each gets its own oracle bits, with split partials or one
    chunk, on ragged tiles and odd widths; without a workspace the two run one
    after the other with running totals, with the same bits."""
    rng = np.random.default_rng(M0 + N1 + K)
    a_kc, b_kc = layout[0] == "n", layout[1] == "t"
    probs = []
    for M, N in ((M0, N0), (M1, N1)):
        A = make(rng, (M, K) if a_kc else (K, M))
        B = make(rng, (N, K) if b_kc else (K, N))
        C0 = make(rng, (M, N))
        lda, ldb = (K if a_kc else M), (K if b_kc else N)
        want = orc_contract(A, B, M, N, K, lda, a_kc, ldb, b_kc, mode=mode, C0=C0 if mode else None)
        probs.append((A, lda, B, ldb, C0, M, N, want))
    nch = (K + 1023) // 1024
    for ws in (empty(nch * (M0 * N0 + M1 * N1)), None):
        outs = [dev(C0.copy()) for (_, _, _, _, C0, _, _, _) in probs]
        args = [(dev(A), lda, dev(B), ldb, C, N, M, N) for (A, lda, B, ldb, _, M, N, _), C in zip(probs, outs)]
        mlb.gemm_pair(args[0], args[1], K, a_kc, b_kc, mode=mode, ws=ws)
        for i, ((_, _, _, _, _, M, N, want), C) in enumerate(zip(probs, outs)):
            assert_bits(f"pair problem {i} ws {ws is not None}", host(C).reshape(M, N), want)


def test_empty_and_degenerate_sizes(mlb):
    """An empty contraction (K = 0) is +0 (mode 0) or C + (+0) (mode 1, so a
    -0 in C becomes +0); M = 0 or N = 0 writes nothing; zero rows of RMSNorm,
    SwiGLU, AdamW and the scatter leave their outputs as they were, and the
    RMSNorm gain gradient over zero rows is the empty contraction, +0."""
    L = mlb.lib()
    st = mlb._stream()
    p = mlb._ptr
    M, N = 5, 7
    C0 = np.array([-0.0, 1.5, -2.25, 0.0, 3.0, -1.0, 7.5] * M, np.float32)
    A, B = dev(np.ones(64, np.float32)), dev(np.ones(64, np.float32))
    for mode in (0, 1):
        C = dev(C0.copy())
        mlb.gemm(A, B, C, M, N, 0, 4, True, 4, True, N, mode=mode)
        want = np.zeros_like(C0) if mode == 0 else C0 + np.float32(0.0)
        assert_bits(f"K = 0 mode {mode}", host(C), want)
    for m_, n_ in ((0, N), (M, 0)):
        C = dev(C0.copy())
        mlb.gemm(A, B, C, m_, n_, 3, 4, True, 4, True, N)
        assert_bits(f"M {m_} N {n_} untouched", host(C), C0)
    sentinel = np.full(64, 7.0, np.float32)
    x, w, y, r, dx, dw, ws = (dev(sentinel.copy()) for _ in range(7))
    mlb.check(L.mlb_prim_rmsnorm_fwd(p(x), p(w), 0, 8, 1e-6, p(y), p(r), st))
    mlb.check(L.mlb_prim_rmsnorm_bwd(p(x), p(x), p(w), p(r), 0, 8, p(dx), p(dw), p(ws), 256, st))
    assert_bits("rmsnorm y", host(y), sentinel)
    assert_bits("rmsnorm r", host(r), sentinel)
    assert_bits("rmsnorm dx", host(dx), sentinel)
    assert_bits("rmsnorm dw over no rows", host(dw)[:8], np.zeros(8, np.float32))
    a = dev(sentinel.copy())
    mlb.check(L.mlb_prim_swiglu_fwd(p(x), 0, 8, p(a), st))
    assert_bits("swiglu a", host(a), sentinel)
    pp, g, m, v = (dev(sentinel.copy()) for _ in range(4))
    mlb.check(L.mlb_prim_adamw(p(pp), p(g), p(m), p(v), 0, 1e-3, 0.9, 0.95, 1e-8, 0.1, 1, st))
    for name, t in (("p", pp), ("g", g), ("m", m), ("v", v)):
        assert_bits(f"adamw {name}", host(t), sentinel)
    ids = dev(np.zeros(8, np.int32))
    dE = dev(sentinel.copy())
    mlb.embed_scatter(ids, x, 0, 8, 8, dE, empty(2 * 8192 * 2))
    assert_bits("scatter dE", host(dE), sentinel)


# ------------------------------------------------------------- row operations
@pytest.mark.parametrize("rows,d", [(8192, 767), (8192, 768), (3, 32)])
def test_rmsnorm(mlb, rows, d):
    rng = np.random.default_rng(d)
    x, w, dy = make(rng, (rows, d)), make(rng, d), make(rng, (rows, d))
    eps = np.float32(1e-6)
    y, r = empty(rows * d), empty(rows)
    xd_shape = dev(x)
    mlb.rmsnorm_fwd(xd_shape, dev(w), eps, y, r)
    yo, ro = oracle.rmsnorm_fwd(x, w, eps)
    assert_bits("y", host(y).reshape(rows, d), yo)
    assert_bits("r", host(r), ro)
    dx, dw = empty(rows * d), empty(d)
    ws = empty(((rows + 1023) // 1024) * d)
    mlb.rmsnorm_bwd(dev(dy), xd_shape, dev(w), dev(ro), dx, dw, ws)
    dxo, dwo = oracle.rmsnorm_bwd(dy, x, w, ro)
    assert_bits("dx", host(dx).reshape(rows, d), dxo)
    assert_bits("dw", host(dw), dwo)


@pytest.mark.parametrize("B,T,H,hd", [(2, 2048, 3, 64), (1, 37, 2, 8), (1, 33, 2, 6)])
def test_rope(mlb, B, T, H, hd):
    """Four pairs per thread (hd / 2 a multiple of 4) and one pair per thread."""
    rng = np.random.default_rng(2 + hd)
    ld = 3 * H * hd
    x = make(rng, (B * T, ld))
    c, s = oracle.rope_table(T, hd, 10000.0)
    for bwd in (0, 1):
        want = x.copy()
        fn = oracle.lib().orc_rope_bwd if bwd else oracle.lib().orc_rope_fwd
        fn(oracle._p(want), B, T, H, hd, ld, c, s)
        xd = dev(x)
        mlb.rope(xd, B, T, H, hd, ld, 10000.0, backward=bwd)
        assert_bits(f"rope bwd={bwd}", host(xd), want)


# hd = 64 with T a multiple of 64 and tiled P runs the paired-row-tile
# kernel (single tile, odd tile count, one and two 1024-chunks); the other
# shapes run the general contraction. T = 601 is an odd row count for the
# register-resident softmax; T = 2048 with 5-wide heads is the sweep's causal
# softmax at full length.
@pytest.mark.parametrize("BH,T,hd,tiled", [(2, 64, 8, 0), (2, 64, 8, 1), (3, 300, 5, 0), (2, 1100, 64, 0),
                                           (2, 1088, 64, 1), (3, 96, 5, 1), (1, 2080, 64, 1), (2, 64, 64, 1),
                                           (3, 192, 64, 1), (2, 1024, 64, 1), (1, 2048, 64, 1), (2, 601, 8, 0),
                                           (3, 1, 5, 0), (2, 1, 64, 0), (2, 2048, 5, 1), (1, 2048, 5, 0)])
def test_attention_fwd_bwd(mlb, BH, T, hd, tiled):
    rng = np.random.default_rng(T + hd)
    q, k, v, dO = (make(rng, (BH, T, hd)) for _ in range(4))
    P, O = empty(BH * T * T), empty(BH * T * hd)
    qd, kd, vd = dev(q), dev(k), dev(v)
    mlb.attention_fwd(BH, 1, T, hd, qd, kd, vd, hd, P, O, hd, tiled=tiled)
    Po, Oo = oracle.attention_fwd(q, k, v)
    low = np.tril(np.ones((T, T), bool))
    Pg = host(P)
    Pg = mlb.tiled_to_dense(Pg, T) if tiled else Pg.reshape(BH, T, T)
    assert_bits("P", Pg[:, low], Po[:, low])
    assert_bits("O", host(O).reshape(BH, T, hd), Oo)
    dq, dk, dv = empty(BH * T * hd), empty(BH * T * hd), empty(BH * T * hd)
    ws = empty(BH * T * T + BH * T)
    mlb.attention_bwd(BH, 1, T, hd, qd, kd, vd, hd, P, O, dev(dO), hd, dq, dk, dv, ws, tiled=tiled)
    dqo, dko, dvo = oracle.attention_bwd(q, k, v, Po, Oo, dO)
    assert_bits("dq", host(dq).reshape(BH, T, hd), dqo)
    assert_bits("dk", host(dk).reshape(BH, T, hd), dko)
    assert_bits("dv", host(dv).reshape(BH, T, hd), dvo)


def test_attention_strided_heads(mlb):
    """Heads as column slices of [B*T, 3*H*hd] (the step's layout), output
    rows of stride H*hd, every contraction routed through the paired-row-tile
    kernel; each head equals the oracle's."""
    B, H, T, hd = 2, 3, 1152, 64
    rng = np.random.default_rng(77)
    qkv = make(rng, (B * T, 3 * H * hd))
    dO = make(rng, (B * T, H * hd))
    ld, ldo = 3 * H * hd, H * hd
    qkvd = dev(qkv).reshape(-1)
    q, k, v = qkvd, qkvd[H * hd:], qkvd[2 * H * hd:]      # column offsets of the flat buffer
    P, O = empty(B * H * T * T), empty(B * T * ldo)
    mlb.attention_fwd(B, H, T, hd, q, k, v, ld, P, O, ldo, tiled=1)
    dqkv = empty(B * T * ld)
    dqkv.zero_()
    ws = empty(B * H * T * T + B * H * T)
    mlb.attention_bwd(B, H, T, hd, q, k, v, ld, P, O, dev(dO), ldo, dqkv, dqkv[H * hd:], dqkv[2 * H * hd:], ws,
                      tiled=1)
    Og, dg = host(O).reshape(B, T, H, hd), host(dqkv).reshape(B, T, 3, H, hd)
    for b in range(B):
        for h in range(H):
            x = qkv.reshape(B, T, 3, H, hd)[b, :, :, h]
            qh, kh, vh = (np.ascontiguousarray(x[:, i])[None] for i in range(3))
            Po, Oo = oracle.attention_fwd(qh, kh, vh)
            assert_bits(f"O b{b} h{h}", Og[b, :, h], Oo[0])
            dOh = np.ascontiguousarray(dO.reshape(B, T, H, hd)[b, :, h])[None]
            want = oracle.attention_bwd(qh, kh, vh, Po, Oo, dOh)
            for i, name in enumerate(("dq", "dk", "dv")):
                assert_bits(f"{name} b{b} h{h}", dg[b, :, i, h], want[i][0])


@pytest.mark.parametrize("rows,F", [(4096, 1024), (37, 1023), (5, 6)])
def test_swiglu(mlb, rows, F):
    """float4 path (F % 4 == 0) and the one-element path."""
    rng = np.random.default_rng(3 + F)
    gu = (make(rng, (rows, 2 * F)) * 8).astype(np.float32)
    dA = make(rng, (rows, F))
    a = empty(rows * F)
    gud = dev(gu)
    mlb.swiglu_fwd(gud, rows, F, a)
    ao = np.empty((rows, F), np.float32)
    oracle.lib().orc_swiglu_fwd(gu, rows, F, 2 * F, ao, F)
    assert_bits("a", host(a).reshape(rows, F), ao)
    dgu = empty(rows * 2 * F)
    mlb.swiglu_bwd(dev(dA), gud, rows, F, dgu)
    dguo = np.empty_like(gu)
    oracle.lib().orc_swiglu_bwd(dA, F, gu, rows, F, 2 * F, dguo)
    assert_bits("dgu", host(dgu).reshape(rows, 2 * F), dguo)


# (64, 256) and (3, 25344) take the three-pass kernel; the others the
# register-resident one: its smallest and largest row lengths, one where the
# later waves hold only padding, and the 50,257-token vocabulary
@pytest.mark.parametrize("N,V", [(64, 256), (3, 25344), (3, 25345), (8, 30000), (37, 50257), (5, 50688)])
def test_cross_entropy(mlb, N, V):
    rng = np.random.default_rng(V)
    logits = (make(rng, (N, V)) * 4).astype(np.float32)
    tg = rng.integers(0, V, N).astype(np.int32)
    # targets at both ends; a row whose maximum is -0 ahead of +0 (the sign of
    # a zero maximum), one with -inf entries and the maximum last, one constant
    tg[0], tg[1] = 0, V - 1
    logits[0] = -np.abs(logits[0])
    logits[0, 7], logits[0, V - 2] = np.float32(-0.0), np.float32(0.0)
    if N > 2:
        logits[2, ::3] = -np.inf
        logits[2, V - 1] = np.float32(9.0)
    if N > 3:
        logits[3] = np.float32(0.25)
    # rows outside the kernel's in-range exp path: a NaN, a +inf, entries that
    # underflow exp, and an entry exactly at exp's underflow threshold (relative
    # to a zero maximum); then one just above it, which stays on that path
    if N > 4:
        logits[4, 5] = np.float32(np.nan)
    if N > 5:
        logits[5, V // 2] = np.float32(np.inf)
    if N > 6:
        logits[6, V // 3] = np.float32(200.0)
    for r, bits in ((7, 0xC2CFF1B5), (8, 0xC2CFF1B4)):
        if N > r:
            logits[r] = -np.abs(logits[r]) * 10
            logits[r, 1] = np.float32(0.0)
            logits[r, 3] = np.array([bits], np.uint32).view(np.float32)[0]
    rows, dl, loss = empty(N), empty(N * V), empty(1)
    mlb.cross_entropy(dev(logits), dev(tg), N, V, rows, dl, loss)
    lo, ro, dlo = oracle.cross_entropy(logits, tg)
    assert_bits("rows", host(rows), ro)
    assert_bits("dl", host(dl).reshape(N, V), dlo)
    assert_bits("loss", host(loss), np.float32([lo]))


def test_cross_entropy_bad_target_refused(mlb):
    logits = np.zeros((4, 10), np.float32)
    tg = np.array([0, 1, 10, 2], np.int32)
    with pytest.raises(mlb.MlbError) as e:
        mlb.cross_entropy(dev(logits), dev(tg), 4, 10, empty(4), empty(40), empty(1))
    assert e.value.name == "MLB_E_BAD_TOKEN"


def test_embed_scatter_zipf(mlb):
    from bitwise_reproducible_fp32_amd import inputs as I
    N, V, d = 8192, 50257, 768
    ids = I.zipf_ids(N, V, 5)
    dh = make(np.random.default_rng(4), (N, d))
    base = make(np.random.default_rng(6), (V, d))
    want = oracle.embed_scatter(ids, dh, base)
    dE = dev(base)
    mlb.embed_scatter(dev(ids), dev(dh), N, d, V, dE, empty(2 * 8192 * 2))
    assert_bits("dE", host(dE), want)


@pytest.mark.parametrize("N", [8193, 20000, 65536])
def test_embed_scatter_beyond_one_sort_block(mlb, N):
    """More positions than one workgroup's LDS sort holds: blocks of 8,192
    keys sorted in LDS, then one, two and three merge passes; a ragged last
    block (8,193 and 20,000) is padded with keys that sort last."""
    from bitwise_reproducible_fp32_amd import inputs as I
    V, d = 50257, 257
    ids = I.zipf_ids(N, V, N)
    dh = make(np.random.default_rng(N + 1), (N, d))
    base = make(np.random.default_rng(N + 2), (V, d))
    want = oracle.embed_scatter(ids, dh, base)
    P = 1 << (N - 1).bit_length()
    dE = dev(base)
    mlb.embed_scatter(dev(ids), dev(dh), N, d, V, dE, empty(4 * P))
    assert_bits("dE", host(dE), want)


def test_embed_scatter_vocabulary_beyond_32_bit_keys(mlb):
    """Ids of 2^19 - 1 and more do not fit the 32-bit keys: one workgroup's
    64-bit key sort (5,000 positions) and the 64-bit segment walk."""
    from bitwise_reproducible_fp32_amd import inputs as I
    N, V, d = 5000, 600000, 20
    ids = I.zipf_ids(N, V, 9)
    ids[::7] = V - 1 - ids[::7]                        # ids above 2^19 as well
    dh = make(np.random.default_rng(10), (N, d))
    base = make(np.random.default_rng(11), (V, d))
    want = oracle.embed_scatter(ids, dh, base)
    dE = dev(base)
    mlb.embed_scatter(dev(ids), dev(dh), N, d, V, dE, empty(2 * 8192 * 2))
    assert_bits("dE", host(dE), want)


@pytest.mark.parametrize("N", [3000, 10000])
def test_embed_scatter_skips_ids_outside_the_table(mlb, N):
    """Ids below 0 or at V and beyond contribute nothing; the rest keep their
    order (compared with the oracle's scatter of the valid positions alone),
    on the 32-bit key path and the blocked 64-bit one."""
    from bitwise_reproducible_fp32_amd import inputs as I
    V, d = 50257, 33
    rng = np.random.default_rng(N)
    ids = I.zipf_ids(N, V, N + 3)
    bad = rng.random(N) < 0.05
    ids[bad] = rng.choice(np.array([-1, -7, V, V + 5, 2 ** 31 - 1], np.int32), bad.sum())
    dh = make(rng, (N, d))
    base = make(np.random.default_rng(N + 4), (V, d))
    want = oracle.embed_scatter(ids[~bad], dh[~bad], base)
    P = max(8192, 1 << (N - 1).bit_length())
    dE = dev(base)
    mlb.embed_scatter(dev(ids), dev(dh), N, d, V, dE, empty(4 * P))
    assert_bits("dE", host(dE), want)


def test_embed_scatter_limits(mlb):
    ids = dev(np.zeros(65537, np.int32))
    dh = empty(65537 * 4)
    dE = empty(8 * 4)
    with pytest.raises(mlb.MlbError) as e:               # more positions than the sort takes
        mlb.embed_scatter(ids, dh, 65537, 4, 8, dE, empty(4 * 131072))
    assert e.value.name == "MLB_E_UNSUPPORTED"
    with pytest.raises(mlb.MlbError) as e:               # 20,000 positions need 16 * 32,768 bytes
        mlb.embed_scatter(ids, dh, 20000, 4, 8, dE, empty(4 * 32768 - 1))
    assert e.value.name == "MLB_E_ARENA_TOO_SMALL"


def test_adamw(mlb):
    rng = np.random.default_rng(11)
    n = 1 << 20
    p, g = make(rng, n), (make(rng, n) * np.exp2(rng.integers(-20, 3, n))).astype(np.float32)
    m, v = make(rng, n) * 0.01, np.abs(make(rng, n)) * 1e-4
    m, v = m.astype(np.float32), v.astype(np.float32)
    b1, b2, eps, wd, lr, t = np.float32(0.9), np.float32(0.95), np.float32(1e-8), np.float32(0.1), np.float32(6e-4), 7
    pd, gd, md, vd = dev(p), dev(g), dev(m), dev(v)
    mlb.adamw(pd, gd, md, vd, n, lr, b1, b2, eps, wd, t)
    po, mo, vo = p.copy(), m.copy(), v.copy()
    oracle.lib().orc_adamw(po, g, mo, vo, n, lr, b1, b2, eps, wd, oracle.lib().orc_bias_correction(b1, t),
                           oracle.lib().orc_bias_correction(b2, t))
    assert_bits("p", host(pd), po)
    assert_bits("m", host(md), mo)
    assert_bits("v", host(vd), vo)
    assert np.all(host(gd) == 0) and not np.any(np.signbit(host(gd)))


def test_segment_split_same_bits(mlb):
    """The segment-major chunk list folded by the split path equals the in-kernel fold."""
    rng = np.random.default_rng(15)
    M, d, F = 200, 160, 1056
    A, B = make(rng, (M, 2 * F)), make(rng, (2 * F, d))
    want = orc_contract(A, B, M, d, 2 * F, 2 * F, True, d, False, kseg=F)
    ws = empty(4 * M * d)
    for split in (0, 1):
        C = empty(M * d)
        mlb.gemm(dev(A), dev(B), C, M, d, 2 * F, 2 * F, True, d, False, d, kseg=F, split=split, ws=ws)
        assert_bits(f"segments split {split}", host(C).reshape(M, d), want)


@pytest.mark.parametrize("layout", ["nt", "nn", "tn"])
def test_padded_leading_dimension(mlb, layout):
    """Vector loads over a leading dimension padded past an odd extent (the
    logits layout): the slack past K (or M) never enters a chain."""
    rng = np.random.default_rng(16)
    M, K, N = 130, 1027, 96
    a_kc, b_kc = layout[0] == "n", layout[1] == "t"
    ext_a = K if a_kc else M
    lda = (ext_a + 3) // 4 * 4
    rows_a = M if a_kc else K
    Ap = np.full((rows_a, lda), np.nan, np.float32)          # slack holds NaN on purpose
    Ap[:, :ext_a] = make(rng, (rows_a, ext_a))
    ext_b = K if b_kc else N
    ldb = (ext_b + 3) // 4 * 4
    rows_b = N if b_kc else K
    Bp = np.full((rows_b, ldb), np.nan, np.float32)
    Bp[:, :ext_b] = make(rng, (rows_b, ext_b))
    want = orc_contract(Ap, Bp, M, N, K, lda, a_kc, ldb, b_kc)
    C = empty(M * N)
    mlb.gemm(dev(Ap), dev(Bp), C, M, N, K, lda, a_kc, ldb, b_kc, N)
    assert_bits(f"padded {layout}", host(C).reshape(M, N), want)
