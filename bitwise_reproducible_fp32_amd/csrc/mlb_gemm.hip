// Fixed-order FP32 contractions on the CDNA4 matrix cores.
//
// Profile rule (G1024, the only matrix-product rule): every output is a chain
// acc = fma(a_k, b_k, acc) from +0 in ascending k inside chunks of 1024 (cut
// at multiples of 1024 of each segment's own index, intersected with the
// causal range), and the non-empty chunk results are added left to right.
//
// Why the matrix cores may run this chain: on gfx950 the FP32 MFMA
// v_mfma_f32_32x32x2_f32 computes, per output, fma(a1, b1, fma(a0, b0, c))
// with single rounding per step, IEEE denormals and the k = 0 lanes (0-31)
// applied before the k = 1 lanes (32-63). The probe that establishes this bit
// for bit against a CPU fma chain is exported as mlb_diag_mfma and is part of
// the GPU test suite. A chain of these instructions over ascending k-pairs is
// therefore exactly the profile's chain.
//
// Positions past the end of K are padded with A = -0 and B = +0: the product
// is -0 and fma(-0 * +0, c) = c for every c (including -0), so padding never
// moves a bit. Causal ranges differ per row and cannot be padded that way, so
// the one 32x32 tile that straddles the diagonal is done with per-element
// VALU fmas in the same ascending order.
//
// Tiles: a workgroup owns MT x NT outputs (64*WM x 64*WN), each wave 64x64 as
// 2x2 MFMA blocks of 32x32; K advances in LDS tiles of 32 (16 k-pairs).
// K tiles never straddle a 1024 chunk (32 divides 1024). Workgroups are
// mapped to tiles so that consecutive tiles land on the same XCD (the
// dispatcher assigns workgroup w to XCD w mod 8), grouped 8 tile-rows deep
// for L2 reuse of the B panel.
#include <cstdio>
#include <cstring>

#include "mlb_device.hpp"
#include "mlb_internal.hpp"

namespace mlb {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
constexpr int KTMIN = 32;   // K tiles are 32 or 64 wide; both divide the 1024 chunk
constexpr int64_t KC = 1024;

struct KArgs {
    int64_t M, N, K, kseg;
    const float* A; int64_t lda;
    const float* B; int64_t ldb;
    float* C; int64_t ldc;
    const float* R;
    int64_t H, sAb, sAh, sBb, sBh, sCb, sCh;
    int outmask, mode, krange, split;
    float scale;
    float* part;
    int64_t tiles_m, tiles_n, ntiles;
    // this problem's share of the grid: ntiles x nsplit x batch workgroups,
    // numbered after those of the problems before it in the same launch
    int64_t nsplit, nwg;
    // chunk >= 0: this launch runs only that 1024-chunk of a causal contraction
    // over row tiles tm_lo.. (launched in chunk order; rows whose first chunk
    // it is store, later chunks add to C)
    int64_t chunk, tm_lo;
    const float* rope_cos;   // non-null: rotary embedding of columns [0, rope_cols) in the epilogue
    const float* rope_sin;
    int64_t rope_T, rope_cols;
};

// Offset of element (r, c) of a matrix stored as 32x32 tiles, each 4 KiB
// contiguous and row-major inside, tiles row-major; ld is the logical row length
// (a multiple of 32).
__device__ __forceinline__ int64_t blk_off(int64_t ld, int64_t r, int64_t c) {
    return (((r >> 5) * (ld >> 5) + (c >> 5)) << 10) + ((r & 31) << 5) + (c & 31);
}

__device__ __forceinline__ void epilogue_store(const KArgs& a, int mode, float* C, int64_t gi, int64_t gj, float v) {
    float* p = C + gi * a.ldc + gj;
    if (mode == 0) *p = v;
    else if (mode == 1) *p = *p + v;
    else if (mode == 2) *p = v * a.scale;
    else *p = a.R[gi * a.ldc + gj] + v;
}

// Single-chunk vector-load instances fit in 168 registers, three waves per
// SIMD (the attention contractions gain most); the others keep the default so
// that their running totals do not spill.
template <bool VEC, bool MC>
constexpr int gemm_waves_per_eu() { return (VEC && !MC) ? 3 : 1; }

// One launch runs one contraction, or two independent ones of the same kind
// (a0 first, then a1; a1.nwg == 0 when there is one): the second fills the
// part-filled last wave of the first.
template <bool AKC, bool BKC, int WM, int WN, int RB, int KR, bool VEC, bool MC, int KT, bool ABLK = false>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(gemm_waves_per_eu<VEC, MC>())))
void k_gemm(KArgs a0, KArgs a1) {
    // Each wave owns RB 32-row blocks x 64 columns (two 32x32 MFMA blocks per
    // row block). MC: the contraction may span several 1024-chunks, so a
    // running total is kept beside the chunk accumulator.
    constexpr int MT = 32 * RB * WM, NT = 64 * WN, NTHR = 64 * WM * WN;
    constexpr int ALD = AKC ? KT + 1 : MT + 4;
    constexpr int BLD = BKC ? KT + 1 : NT + 4;
    constexpr int ASZ = AKC ? MT * ALD : KT * ALD;
    constexpr int BSZ = BKC ? NT * BLD : KT * BLD;
    constexpr int W = VEC ? 4 : 1;
    constexpr int EA = MT * KT / NTHR / W;     // loads per thread per tile
    constexpr int EB = NT * KT / NTHR / W;
    static_assert(EA * W * NTHR == MT * KT && EB * W * NTHR == NT * KT, "tile split");
    __shared__ float As[ASZ];
    __shared__ float Bs[BSZ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int lk = lane >> 5, li = lane & 31;

    // XCD-aware order over (tile, chunk, batch problem), batch slowest, then
    // grouped tile rows inside a problem; the launch's first contraction
    // takes the first a0.nwg logical workgroups.
    int64_t lb = xcd_logical_block();
    const bool second = lb >= a0.nwg;
    const KArgs& a = second ? a1 : a0;
    if (second) lb -= a0.nwg;
    const int64_t gy = (lb / a.ntiles) % a.nsplit, gz = lb / (a.ntiles * a.nsplit);
    const int64_t logical = lb % a.ntiles;
    constexpr int64_t GM = 8;
    const int64_t per_group = GM * a.tiles_n;
    const int64_t first_m = (logical / per_group) * GM;
    const int64_t gsize = (a.tiles_m - first_m) < GM ? (a.tiles_m - first_m) : GM;
    const int64_t tm = first_m + (logical % per_group) % gsize;
    const int64_t tn = (logical % per_group) / gsize;
    // k <= i: later row tiles hold more work, so they are dispatched first
    const int64_t tmr = (KR == 1) ? a.tiles_m - 1 - tm : tm;
    const int64_t i0 = (tmr + a.tm_lo) * MT, j0 = tn * NT;
    if (a.outmask && j0 > i0 + MT - 1) return;   // whole tile above the diagonal: nothing to write

    const int64_t z = gz, zb = z / a.H, zh = z % a.H;
    const float* __restrict__ A = a.A + zb * a.sAb + zh * a.sAh;
    const float* __restrict__ B = a.B + zb * a.sBb + zh * a.sBh;
    float* C = a.C + zb * a.sCb + zh * a.sCh;

    int64_t kbeg = 0, kend = a.K;
    if (a.split) {   // one chunk of the segment-major chunk list
        const int64_t per_seg = (a.kseg + KC - 1) / KC;
        const int64_t sg = gy / per_seg, ch = gy % per_seg;
        kbeg = sg * a.kseg + ch * KC;
        kend = sg * a.kseg + ((ch + 1) * KC < a.kseg ? (ch + 1) * KC : a.kseg);
    }
    if (a.chunk >= 0) {   // one chunk of a causal contraction (kseg == K)
        kbeg = a.chunk * KC;
        kend = (kbeg + KC < a.K) ? kbeg + KC : a.K;
    }
    // the row's first non-empty chunk applies the mode; later chunks add
    // (k <= i: chunk 0 for every row; k >= i: the chunk holding row i)
    const int64_t first_chunk = (KR == 2) ? i0 / KC : 0;
    const int emode = (a.chunk < 0 || a.chunk == first_chunk) ? a.mode : 1;
    if (KR == 1) kend = (kend < i0 + MT) ? kend : i0 + MT;
    if (KR == 2) kbeg = (kbeg > i0) ? kbeg : i0;
    const int64_t kt0 = kbeg / KT, kt1 = (kend + KT - 1) / KT;

    v16f acc00, acc01, acc10, acc11, tot00, tot01, tot10, tot11;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        acc00[e] = 0.0f; acc01[e] = 0.0f; acc10[e] = 0.0f; acc11[e] = 0.0f;
        tot00[e] = 0.0f; tot01[e] = 0.0f; tot10[e] = 0.0f; tot11[e] = 0.0f;
    }
    bool have0 = false, have1 = false, dirty0 = false, dirty1 = false;
    const int r0 = wm * 32 * RB, r1 = r0 + 32;            // row offsets of the wave's blocks in the tile
    const int64_t bi00 = i0 + r0, bi01 = i0 + r1;

    float ra[EA * W], rb[EB * W];
    // Tiles whose rows, columns and K range are all in bounds load and store
    // without per-element checks or masks (a uniform branch per K tile).
    const bool rows_in = i0 + MT <= a.M, cols_in = j0 + NT <= a.N;
    auto load_global = [&](int64_t kt) {
        const int64_t k0 = kt * KT;
        if (VEC && rows_in && cols_in && k0 + KT <= a.K) {
#pragma unroll
            for (int s = 0; s < EA; ++s) {
                const int q = tid + s * NTHR;
                int64_t gi, gk;
                if (AKC) { gi = i0 + q / (KT / W); gk = k0 + (q % (KT / W)) * W; }
                else { gk = k0 + q / (MT / W); gi = i0 + (q % (MT / W)) * W; }
                const float4 v = ABLK ? *reinterpret_cast<const float4*>(A + blk_off(a.lda, AKC ? gi : gk, AKC ? gk : gi))
                               : AKC ? *reinterpret_cast<const float4*>(A + gi * a.lda + gk)
                                     : *reinterpret_cast<const float4*>(A + gk * a.lda + gi);
                ra[s * 4 + 0] = v.x; ra[s * 4 + 1] = v.y; ra[s * 4 + 2] = v.z; ra[s * 4 + 3] = v.w;
            }
#pragma unroll
            for (int s = 0; s < EB; ++s) {
                const int q = tid + s * NTHR;
                int64_t gj, gk;
                if (BKC) { gj = j0 + q / (KT / W); gk = k0 + (q % (KT / W)) * W; }
                else { gk = k0 + q / (NT / W); gj = j0 + (q % (NT / W)) * W; }
                const float4 v = BKC ? *reinterpret_cast<const float4*>(B + gj * a.ldb + gk)
                                     : *reinterpret_cast<const float4*>(B + gk * a.ldb + gj);
                rb[s * 4 + 0] = v.x; rb[s * 4 + 1] = v.y; rb[s * 4 + 2] = v.z; rb[s * 4 + 3] = v.w;
            }
            return;
        }
#pragma unroll
        for (int s = 0; s < EA; ++s) {
            const int q = tid + s * NTHR;
            int64_t gi, gk;
            if (AKC) { gi = i0 + q / (KT / W); gk = k0 + (q % (KT / W)) * W; }
            else { gk = k0 + q / (MT / W); gi = i0 + (q % (MT / W)) * W; }
            if (VEC) {
                // the leading dimension covers the vector past the last element;
                // positions past K read as -0, rows past M as 0
                if (gk < a.K && gi < a.M) {
                    const float4 v = ABLK ? *reinterpret_cast<const float4*>(A + blk_off(a.lda, AKC ? gi : gk, AKC ? gk : gi))
                                   : AKC ? *reinterpret_cast<const float4*>(A + gi * a.lda + gk)
                                         : *reinterpret_cast<const float4*>(A + gk * a.lda + gi);
                    // positions past K inside the vector are masked at the LDS store,
                    // so that no select waits on the load here
                    ra[s * 4 + 0] = v.x; ra[s * 4 + 1] = v.y; ra[s * 4 + 2] = v.z; ra[s * 4 + 3] = v.w;
                } else {
                    const float f = (gk >= a.K) ? -0.0f : 0.0f;
                    ra[s * 4 + 0] = f; ra[s * 4 + 1] = f; ra[s * 4 + 2] = f; ra[s * 4 + 3] = f;
                }
            } else {
                if (gk >= a.K) ra[s] = -0.0f;
                else if (gi >= a.M) ra[s] = 0.0f;
                else ra[s] = ABLK ? A[blk_off(a.lda, AKC ? gi : gk, AKC ? gk : gi)]
                           : AKC ? A[gi * a.lda + gk] : A[gk * a.lda + gi];
            }
        }
#pragma unroll
        for (int s = 0; s < EB; ++s) {
            const int q = tid + s * NTHR;
            int64_t gj, gk;
            if (BKC) { gj = j0 + q / (KT / W); gk = k0 + (q % (KT / W)) * W; }
            else { gk = k0 + q / (NT / W); gj = j0 + (q % (NT / W)) * W; }
            if (VEC) {
                if (gk < a.K && gj < a.N) {
                    const float4 v = BKC ? *reinterpret_cast<const float4*>(B + gj * a.ldb + gk)
                                         : *reinterpret_cast<const float4*>(B + gk * a.ldb + gj);
                    rb[s * 4 + 0] = v.x; rb[s * 4 + 1] = v.y; rb[s * 4 + 2] = v.z; rb[s * 4 + 3] = v.w;
                } else {
                    rb[s * 4 + 0] = 0.0f; rb[s * 4 + 1] = 0.0f; rb[s * 4 + 2] = 0.0f; rb[s * 4 + 3] = 0.0f;
                }
            } else {
                if (gk >= a.K || gj >= a.N) rb[s] = 0.0f;
                else rb[s] = BKC ? B[gj * a.ldb + gk] : B[gk * a.ldb + gj];
            }
        }
    };
    auto store_lds = [&](int64_t kt) {
        const int64_t k0 = kt * KT;
        if (VEC && k0 + KT <= a.K) {   // no K tail inside this tile: plain copies
#pragma unroll
            for (int s = 0; s < EA; ++s) {
                const int q = tid + s * NTHR;
                if (AKC) {
                    const int i = q / (KT / W), k = (q % (KT / W)) * W;
#pragma unroll
                    for (int e = 0; e < W; ++e) As[i * ALD + k + e] = ra[s * W + e];
                } else {
                    const int k = q / (MT / W), i = (q % (MT / W)) * W;
#pragma unroll
                    for (int e = 0; e < W; ++e) As[k * ALD + i + e] = ra[s * W + e];
                }
            }
#pragma unroll
            for (int s = 0; s < EB; ++s) {
                const int q = tid + s * NTHR;
                if (BKC) {
                    const int j = q / (KT / W), k = (q % (KT / W)) * W;
#pragma unroll
                    for (int e = 0; e < W; ++e) Bs[j * BLD + k + e] = rb[s * W + e];
                } else {
                    const int k = q / (NT / W), j = (q % (NT / W)) * W;
#pragma unroll
                    for (int e = 0; e < W; ++e) Bs[k * BLD + j + e] = rb[s * W + e];
                }
            }
            return;
        }
#pragma unroll
        for (int s = 0; s < EA; ++s) {
            const int q = tid + s * NTHR;
            if (AKC) {
                const int i = q / (KT / W), k = (q % (KT / W)) * W;
#pragma unroll
                for (int e = 0; e < W; ++e)
                    As[i * ALD + k + e] = (VEC && e > 0 && k0 + k + e >= a.K) ? -0.0f : ra[s * W + e];
            } else {
                const int k = q / (MT / W), i = (q % (MT / W)) * W;
#pragma unroll
                for (int e = 0; e < W; ++e) As[k * ALD + i + e] = ra[s * W + e];
            }
        }
#pragma unroll
        for (int s = 0; s < EB; ++s) {
            const int q = tid + s * NTHR;
            if (BKC) {
                const int j = q / (KT / W), k = (q % (KT / W)) * W;
#pragma unroll
                for (int e = 0; e < W; ++e)
                    Bs[j * BLD + k + e] = (VEC && e > 0 && k0 + k + e >= a.K) ? 0.0f : rb[s * W + e];
            } else {
                const int k = q / (NT / W), j = (q % (NT / W)) * W;
#pragma unroll
                for (int e = 0; e < W; ++e) Bs[k * BLD + j + e] = rb[s * W + e];
            }
        }
    };
    auto a_lds = [&](int i, int k) -> float { return AKC ? As[i * ALD + k] : As[k * ALD + i]; };
    auto b_lds = [&](int k, int j) -> float { return BKC ? Bs[j * BLD + k] : Bs[k * BLD + j]; };
    auto fold_pair = [&](v16f& t0, v16f& t1, v16f& c0, v16f& c1, bool& have, bool& dirty) {
        if (!dirty) return;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            t0[e] = have ? t0[e] + c0[e] : c0[e];
            t1[e] = have ? t1[e] + c1[e] : c1[e];
            c0[e] = 0.0f;
            c1[e] = 0.0f;
        }
        have = true;
        dirty = false;
    };
    const int j0l = wn * 64 + li, j1l = j0l + 32;
    // one 32-row block against the wave's two 32-column blocks, all 16 k-pairs
    auto full_block = [&](v16f& c0, v16f& c1, int rloc, int ko) {
        // eight k-pairs per pass: the LDS reads of the next four are issued
        // while the current four's MFMAs run
#pragma unroll 8
        for (int p = 0; p < 16; ++p) {
            const int kk = ko + 2 * p + lk;
            const float av = a_lds(rloc + li, kk);
            const float b0 = b_lds(kk, j0l), b1 = b_lds(kk, j1l);
            c0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b0, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b1, c1, 0, 0, 0);
        }
    };
    // The tile on the diagonal (k0 equals the block's first row). Row il of
    // the block has its causal range boundary inside the tile. For each k-pair
    // (ka, kb) = (2p, 2p+1) the pair's MFMA result is kept for rows that take
    // both terms (k <= i: il >= kb; k >= i: il <= ka); the one row whose range
    // boundary falls between them (il == ka, resp. il == kb) takes the single
    // term with one fma; every other row keeps its value. Positions past K are
    // padded (-0 * +0) and change nothing.
    auto diag_block = [&](v16f& c0, v16f& c1, int rloc, int ko) {
#pragma unroll 1
        for (int p = 0; p < 16; ++p) {
            const int kk = ko + 2 * p + lk;
            const float av = a_lds(rloc + li, kk);
            const float b0 = b_lds(kk, j0l), b1 = b_lds(kk, j1l);
            const v16f n0 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b0, c0, 0, 0, 0);
            const v16f n1 = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b1, c1, 0, 0, 0);
            const int ka = 2 * p, kb = 2 * p + 1;              // relative to the block's first row
            const int ks = (KR == 1) ? ka : kb;               // the single term's k, also its row
            const float as = a_lds(rloc + ks, ko + ks);
            const float bs0 = b_lds(ko + ks, j0l), bs1 = b_lds(ko + ks, j1l);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int il = 8 * (e >> 2) + 4 * lk + (e & 3);
                const bool both = (KR == 1) ? (il >= kb) : (il <= ka);
                const bool single = (il == ks);
                const float s0 = __builtin_fmaf(as, bs0, c0[e]);
                const float s1 = __builtin_fmaf(as, bs1, c1[e]);
                c0[e] = both ? n0[e] : (single ? s0 : c0[e]);
                c1[e] = both ? n1[e] : (single ? s1 : c1[e]);
            }
        }
    };

    int64_t prev_chunk = -1;
    if (kt0 < kt1) load_global(kt0);
    for (int64_t kt = kt0; kt < kt1; ++kt) {
        const int64_t k0 = kt * KT;
        __syncthreads();
        store_lds(kt);
        __syncthreads();
        if (kt + 1 < kt1) load_global(kt + 1);
        if (MC) {
            const int64_t chunk = (k0 / a.kseg) * (a.kseg / KC + 1) + (k0 % a.kseg) / KC;
            if (chunk != prev_chunk) {
                if (prev_chunk >= 0) {
                    fold_pair(tot00, tot01, acc00, acc01, have0, dirty0);
                    if (RB == 2) fold_pair(tot10, tot11, acc10, acc11, have1, dirty1);
                }
                prev_chunk = chunk;
            }
        }
        // 32-wide sub-tiles of the K tile; per row block: 0 skip, 1 full, 2 diagonal
#pragma unroll
        for (int h = 0; h < KT / 32; ++h) {
            const int64_t k0h = k0 + 32 * h;
            const int ko = 32 * h;
            int st0 = 1, st1 = 1;
            if (KR == 1) {
                st0 = (k0h < bi00) ? 1 : (k0h == bi00 ? 2 : 0);
                st1 = (k0h < bi01) ? 1 : (k0h == bi01 ? 2 : 0);
            } else if (KR == 2) {
                st0 = (k0h > bi00) ? 1 : (k0h == bi00 ? 2 : 0);
                st1 = (k0h > bi01) ? 1 : (k0h == bi01 ? 2 : 0);
            }
            dirty0 = dirty0 || st0 != 0;
            dirty1 = dirty1 || st1 != 0;
            if (RB == 2 && st0 == 1 && st1 == 1) {
#pragma unroll 8
                for (int p = 0; p < 16; ++p) {
                    const int kk = ko + 2 * p + lk;
                    const float a0 = a_lds(r0 + li, kk);
                    const float a1 = a_lds(r1 + li, kk);
                    const float b0 = b_lds(kk, j0l);
                    const float b1 = b_lds(kk, j1l);
                    acc00 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc00, 0, 0, 0);
                    acc01 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc01, 0, 0, 0);
                    acc10 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc10, 0, 0, 0);
                    acc11 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc11, 0, 0, 0);
                }
            } else {
                if (st0 == 1) full_block(acc00, acc01, r0, ko);
                else if (KR != 0 && st0 == 2) diag_block(acc00, acc01, r0, ko);
                if (RB == 2) {
                    if (st1 == 1) full_block(acc10, acc11, r1, ko);
                    else if (KR != 0 && st1 == 2) diag_block(acc10, acc11, r1, ko);
                }
            }
        }
    }

    // Epilogue of one 32-row block against the wave's two 32-column blocks.
    // Interior blocks (all rows < M, all columns < N, no mask) store without a
    // per-element branch; read-modify-write modes load every operand before
    // the first store. Either way each element gets exactly the mode's one
    // operation, so the bits do not depend on the path.
    auto store_pair = [&](const v16f& v0, const v16f& v1, int64_t bi, bool valid) {
        const int mode = a.split ? 0 : emode;
        // a per-chunk launch leaves rows without a term in its chunk alone (the
        // rule skips empty chunks); a whole contraction with no term is +0,
        // so accumulate mode still stores C + (+0)
        if (!valid && mode == 1 && a.chunk >= 0) return;
        const int64_t gj0 = j0 + j0l, gj1 = j0 + j1l;
        float* out = a.split ? a.part + gy * a.M * a.N : C;
        const int64_t ld = a.split ? a.N : a.ldc;
        const bool interior = bi + 32 <= a.M && j0 + NT <= a.N && (a.split || !a.outmask);
        auto row = [&](int e) -> int64_t { return bi + 8 * (e >> 2) + 4 * lk + (e & 3); };
        auto ok0 = [&](int64_t gi) { return interior || (gi < a.M && gj0 < a.N && (a.split || !a.outmask || gj0 <= gi)); };
        auto ok1 = [&](int64_t gi) { return interior || (gi < a.M && gj1 < a.N && (a.split || !a.outmask || gj1 <= gi)); };
        float x0[16], x1[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) { x0[e] = valid ? v0[e] : 0.0f; x1[e] = valid ? v1[e] : 0.0f; }
        if (mode == 1 || mode == 3) {
            const float* src = mode == 1 ? out : a.R;
            float r0[16], r1[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t gi = row(e);
                r0[e] = ok0(gi) ? src[gi * ld + gj0] : 0.0f;
                r1[e] = ok1(gi) ? src[gi * ld + gj1] : 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) { x0[e] = r0[e] + x0[e]; x1[e] = r1[e] + x1[e]; }
        } else if (mode == 2) {
#pragma unroll
            for (int e = 0; e < 16; ++e) { x0[e] = x0[e] * a.scale; x1[e] = x1[e] * a.scale; }
        }
        // rotary embedding (128-row tiles without a causal range): this
        // wave's 64 columns (starting at a multiple of 64) are one head, and
        // the lane holds column i of it in x0 and column i + 32 in x1
        if (KR == 0 && MT == 128 && a.rope_cos && !a.split && j0 + 64 * wn < a.rope_cols) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t t = row(e) % a.rope_T;
                const float c = a.rope_cos[t * 32 + li], sn = a.rope_sin[t * 32 + li];
                const float r0 = (x0[e] * c) - (x1[e] * sn);
                const float r1 = (x1[e] * c) + (x0[e] * sn);
                x0[e] = r0;
                x1[e] = r1;
            }
        }
        if (interior && a.split) {
            // split partials are read once, by the fold: nontemporal stores
            // keep them from displacing the operand panels in the L2
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t gi = row(e);
                __builtin_nontemporal_store(x0[e], out + gi * ld + gj0);
                __builtin_nontemporal_store(x1[e], out + gi * ld + gj1);
            }
        } else if (interior) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t gi = row(e);
                out[gi * ld + gj0] = x0[e];
                out[gi * ld + gj1] = x1[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t gi = row(e);
                if (ok0(gi)) out[gi * ld + gj0] = x0[e];
                if (ok1(gi)) out[gi * ld + gj1] = x1[e];
            }
        }
    };
    if (MC && !a.split) {
        fold_pair(tot00, tot01, acc00, acc01, have0, dirty0);
        store_pair(tot00, tot01, bi00, have0);
        if (RB == 2) {
            fold_pair(tot10, tot11, acc10, acc11, have1, dirty1);
            store_pair(tot10, tot11, bi01, have1);
        }
    } else {
        store_pair(acc00, acc01, bi00, dirty0 || a.split);
        if (RB == 2) store_pair(acc10, acc11, bi01, dirty1 || a.split);
    }
}

// One thread per output, global loads, the chunk rule written out directly.
// Slow; it is the geometry-independent cross-check of the tiled kernel and the
// path for layouts the tiled kernel is not instantiated for.
__global__ __launch_bounds__(256) void k_gemm_simple(KArgs a, int a_kc, int b_kc) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= a.M * a.N) return;
    const int64_t i = idx / a.N, j = idx % a.N;
    if (a.outmask && j > i) return;
    const int64_t z = blockIdx.z, zb = z / a.H, zh = z % a.H;
    const float* A = a.A + zb * a.sAb + zh * a.sAh;
    const float* B = a.B + zb * a.sBb + zh * a.sBh;
    float* C = a.C + zb * a.sCb + zh * a.sCh;
    int64_t lo = 0, hi = a.K;
    if (a.krange == 1) hi = (i + 1 < a.K) ? i + 1 : a.K;
    if (a.krange == 2) lo = i;
    float total = 0.0f;
    bool have = false;
    const int64_t nseg = a.K > 0 ? a.K / a.kseg : 0;
    for (int64_t s = 0; s < nseg; ++s)
        for (int64_t c0 = 0; c0 < a.kseg; c0 += KC) {
            const int64_t a0 = s * a.kseg + c0;
            const int64_t a1 = s * a.kseg + ((c0 + KC < a.kseg) ? c0 + KC : a.kseg);
            const int64_t l0 = a0 > lo ? a0 : lo, l1 = a1 < hi ? a1 : hi;
            if (l0 >= l1) continue;
            float acc = 0.0f;
            for (int64_t k = l0; k < l1; ++k) {
                const float av = a_kc ? A[i * a.lda + k] : A[k * a.lda + i];
                const float bv = b_kc ? B[j * a.ldb + k] : B[k * a.ldb + j];
                acc = __builtin_fmaf(av, bv, acc);
            }
            total = have ? total + acc : acc;
            have = true;
        }
    epilogue_store(a, a.mode, C, i, j, have ? total : 0.0f);
}

// total = part[0] + part[1] + ... in chunk order, then the epilogue.
__global__ __launch_bounds__(256) void k_fold(const float* __restrict__ part, int64_t nch, int64_t M,
                                              int64_t N, KArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t MN = M * N;
    if (idx >= MN) return;
    float t = part[idx];
    for (int64_t c = 1; c < nch; ++c) t = t + part[c * MN + idx];
    epilogue_store(a, a.mode, a.C, idx / N, idx % N, t);
}

// The same fold for four adjacent outputs of a row per thread (N % 4 == 0,
// 16-byte aligned partials and rows): float4 traffic, nontemporal loads (each
// partial is read once), and the partials of up to 8 chunks loaded before the
// first addition, which is still in chunk order. Thread q takes outputs
// 4q .. 4q + 3 of problem a.
__device__ __forceinline__ void fold4_at(const KArgs& a, int64_t M, int64_t N, int64_t q) {
    const int64_t MN = M * N, idx = q * 4;
    if (idx >= MN) return;
    const int64_t MN4 = MN / 4, nch = a.nsplit;
    typedef float v4f __attribute__((ext_vector_type(4)));
    const v4f* pv = reinterpret_cast<const v4f*>(a.part);
    const v4f t0 = __builtin_nontemporal_load(pv + q);
    float4 t = make_float4(t0.x, t0.y, t0.z, t0.w);
    for (int64_t c0 = 1; c0 < nch; c0 += 8) {
        v4f x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (c0 + u < nch) x[u] = __builtin_nontemporal_load(pv + (c0 + u) * MN4 + q);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (c0 + u < nch) { t.x = t.x + x[u].x; t.y = t.y + x[u].y; t.z = t.z + x[u].z; t.w = t.w + x[u].w; }
    }
    // rows stored contiguously (ldc == N): the output offset is idx itself,
    // with no 64-bit division per thread
    const int64_t o_ij = a.ldc == N ? idx : (idx / N) * a.ldc + idx % N;
    float* c = a.C + o_ij;
    float4 r = t;
    if (a.mode == 1) {
        const float4 o = *reinterpret_cast<const float4*>(c);
        r.x = o.x + t.x; r.y = o.y + t.y; r.z = o.z + t.z; r.w = o.w + t.w;
    } else if (a.mode == 2) {
        r.x = t.x * a.scale; r.y = t.y * a.scale; r.z = t.z * a.scale; r.w = t.w * a.scale;
    } else if (a.mode == 3) {
        const float4 o = *reinterpret_cast<const float4*>(a.R + o_ij);
        r.x = o.x + t.x; r.y = o.y + t.y; r.z = o.z + t.z; r.w = o.w + t.w;
    }
    *reinterpret_cast<float4*>(c) = r;
}

__global__ __launch_bounds__(256) void k_fold4(int64_t M, int64_t N, KArgs a) {
    fold4_at(a, M, N, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// The folds of the two problems of a paired launch in one grid: blocks below
// b0 take problem 0, the others problem 1.
__global__ __launch_bounds__(256) void k_fold4_pair(int64_t M0, int64_t N0, KArgs a0, int64_t M1, int64_t N1, KArgs a1,
                                                    int64_t b0) {
    const int64_t blk = blockIdx.x;
    if (blk < b0) fold4_at(a0, M0, N0, blk * blockDim.x + threadIdx.x);
    else fold4_at(a1, M1, N1, (blk - b0) * blockDim.x + threadIdx.x);
}

struct Cfg { int wm, wn; };

thread_local char g_launched[96];

template <bool AKC, bool BKC, int WM, int WN, int RB, int KR, int KT = 32, bool ABLK = false>
void launch_t(const KArgs& a, const KArgs& b, bool vec, bool mc, dim3 grid, hipStream_t s) {
    std::snprintf(g_launched, sizeof g_launched, "k_gemm<%s, %s, %d, %d, %d, %d, %s, %s, %d, %s>",
                  AKC ? "true" : "false", BKC ? "true" : "false", WM, WN, RB, KR, vec ? "true" : "false",
                  mc ? "true" : "false", KT, ABLK ? "true" : "false");
    if (mc) {
        if (vec) k_gemm<AKC, BKC, WM, WN, RB, KR, true, true, KT, ABLK><<<grid, 64 * WM * WN, 0, s>>>(a, b);
        else k_gemm<AKC, BKC, WM, WN, RB, KR, false, true, KT, ABLK><<<grid, 64 * WM * WN, 0, s>>>(a, b);
    } else {
        if (vec) k_gemm<AKC, BKC, WM, WN, RB, KR, true, false, KT, ABLK><<<grid, 64 * WM * WN, 0, s>>>(a, b);
        else k_gemm<AKC, BKC, WM, WN, RB, KR, false, false, KT, ABLK><<<grid, 64 * WM * WN, 0, s>>>(a, b);
    }
}

// Tile configurations: 0 = 128x128 (2x2 waves of 64x64), 1 = 256x64 (4x1 waves
// of 64x64), 2 = 128x64 (4x1 waves of 32x64; the causal ranges).
// Returns false when no tiled instantiation exists for the combination.
// tm_count >= 0 restricts the launch to row tiles [tm_lo, tm_lo + tm_count).
int64_t tile_rows(int cfg) { return cfg == 1 ? 256 : 128; }

// The grid of one problem in tile configuration cfg: ntiles x nsplit x batch
// workgroups. tm_count >= 0 restricts it to row tiles [tm_lo, tm_lo + tm_count).
void set_grid(KArgs& a, const GemmDesc& d, int cfg, int64_t nsplit, int64_t tm_lo = 0, int64_t tm_count = -1) {
    const int64_t MT = tile_rows(cfg), NT = cfg == 0 ? 128 : 64;
    a.tm_lo = tm_lo;
    a.tiles_m = tm_count >= 0 ? tm_count : (d.M + MT - 1) / MT;
    a.tiles_n = (d.N + NT - 1) / NT;
    a.ntiles = a.tiles_m * a.tiles_n;
    a.nsplit = nsplit;
    a.nwg = a.ntiles * nsplit * d.batch;
}

// Launches a (gridded by set_grid), followed in the same grid by b when
// b.nwg > 0 (same layout, tile configuration and variant).
bool launch_tiled(const GemmDesc& d, const KArgs& a, const KArgs& b, int cfg, bool vec, bool mc, hipStream_t s) {
    const dim3 grid((unsigned)(a.nwg + b.nwg));
    const int key = (d.a_kc ? 1 : 0) | (d.b_kc ? 2 : 0);
    if (d.krange == 0 && cfg == 0) {
        switch (key) {
            case 3: launch_t<true, true, 2, 2, 2, 0>(a, b, vec, mc, grid, s); return true;
            case 1: launch_t<true, false, 2, 2, 2, 0>(a, b, vec, mc, grid, s); return true;
            case 0: launch_t<false, false, 2, 2, 2, 0>(a, b, vec, mc, grid, s); return true;
            case 2: launch_t<false, true, 2, 2, 2, 0>(a, b, vec, mc, grid, s); return true;
        }
    }
    if (d.krange == 0 && cfg == 1) {
        switch (key) {
            case 3: launch_t<true, true, 4, 1, 2, 0>(a, b, vec, mc, grid, s); return true;
            case 1: launch_t<true, false, 4, 1, 2, 0>(a, b, vec, mc, grid, s); return true;
            case 0: launch_t<false, false, 4, 1, 2, 0>(a, b, vec, mc, grid, s); return true;
            case 2: launch_t<false, true, 4, 1, 2, 0>(a, b, vec, mc, grid, s); return true;
        }
    }
    if (d.krange == 0 && cfg == 2) {
        switch (key) {
            case 3: launch_t<true, true, 4, 1, 1, 0>(a, b, vec, mc, grid, s); return true;
            case 1: launch_t<true, false, 4, 1, 1, 0>(a, b, vec, mc, grid, s); return true;
            case 0: launch_t<false, false, 4, 1, 1, 0>(a, b, vec, mc, grid, s); return true;
            case 2: launch_t<false, true, 4, 1, 1, 0>(a, b, vec, mc, grid, s); return true;
        }
    }
    // causal ranges; a tiled A (32x32 blocks, the attention probability layout)
    // is read as whole contiguous 4 KiB tiles
    if (d.krange == 1 && key == 1 && cfg == 2) {
        if (d.a_blk) launch_t<true, false, 4, 1, 1, 1, 32, true>(a, b, vec, mc, grid, s);
        else launch_t<true, false, 4, 1, 1, 1, 32>(a, b, vec, mc, grid, s);
        return true;
    }
    if (d.krange == 2 && key == 0 && cfg == 2) {
        if (d.a_blk) launch_t<false, false, 4, 1, 1, 2, 32, true>(a, b, vec, mc, grid, s);
        else launch_t<false, false, 4, 1, 1, 2, 32>(a, b, vec, mc, grid, s);
        return true;
    }
    return false;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Expected time, in units of one 128x128 workgroup's time at full residency,
// of a grid of `wgs` workgroups that each cost `per_wg` of that. The chip
// holds 768 of these workgroups at once (256 CUs x 3, for 128x128 and 128x64
// tiles alike), so the grid runs in full waves of 768 plus a last partial
// wave whose workgroups share their CU with fewer others and finish sooner:
// 0.45 of a wave's time when at most 256 remain (one per CU), 0.75 up to 512.
// The constants (and the 0.55 of a 128x64 tile) fit the measured times of the
// step's contraction shapes; bits never depend on the choice.
double grid_cost(int64_t wgs, double per_wg) {
    const int64_t full = wgs / 768, tail = wgs % 768;
    const double last = tail == 0 ? 0.0 : tail <= 256 ? 0.45 : tail <= 512 ? 0.75 : 1.0;
    return per_wg * ((double)full + last);
}

}  // namespace

static bool desc_ok(const GemmDesc& d) {
    if (d.M < 0 || d.N < 0 || d.K < 0 || d.batch < 1 || d.H < 1 || d.batch % d.H != 0) return false;
    if (d.krange < 0 || d.krange > 2 || d.mode < 0 || d.mode > 3) return false;
    if (d.mode == 3 && (!d.R || d.batch != 1)) return false;
    if (d.K > 0 && (d.kseg <= 0 || d.K % d.kseg != 0)) return false;
    if (d.K > 0 && d.K / d.kseg > 1 && (d.kseg % KTMIN != 0 || d.krange != 0)) return false;
    if (!d.A || !d.B || !d.C) return false;
    if (d.a_blk && (d.lda % 32 != 0 || d.krange == 0 || (d.a_kc ? d.M : d.K) > d.lda)) return false;
    return true;
}

// Number of chunks in the segment-major chunk list.
static int64_t nchunks(const GemmDesc& d) {
    if (d.K <= 0 || d.kseg <= 0) return 0;
    return (d.K / d.kseg) * ((d.kseg + KC - 1) / KC);
}

// Whether per-chunk partials are worth it: only when the output has too few
// tiles to fill the chip. Never changes bits.
// Whether per-chunk partials (folded by a second kernel) are worth it: when
// the output has too few tiles to fill the chip, or when several chunks would
// otherwise need the running-total registers. Never changes bits.
static bool split_useful(const GemmDesc& d, const GemmPlan& p) {
    if (p.split == 0 || d.krange != 0 || d.batch != 1 || d.outmask || nchunks(d) < 2) return false;
    if (p.split == 1) return true;
    return nchunks(d) <= 64;
}

static bool want_split(const GemmDesc& d, const GemmPlan& p) {
    if (!split_useful(d, p)) return false;
    if (p.split == 1) return true;
    return p.scratch && p.scratch_floats >= nchunks(d) * d.M * d.N;   // auto: only with enough scratch
}

int64_t gemm_split_scratch(const GemmDesc& d, const GemmPlan& p) {
    if (!split_useful(d, p)) return 0;
    return nchunks(d) * d.M * d.N;
}

const char* gemm_last_kernel() { return g_launched; }

double gemm_flops(const GemmDesc& d, int64_t kb, int64_t ke) {
    kb = kb > 0 ? kb : 0;
    ke = ke < d.K ? ke : d.K;
    if (kb >= ke || d.M <= 0 || d.N <= 0) return 0.0;
    double pairs = 0.0;
    if (d.krange == 0 && !d.outmask) {
        pairs = (double)d.M * (double)d.N * (double)(ke - kb);
    } else {
        for (int64_t i = 0; i < d.M; ++i) {
            int64_t lo = kb, hi = ke;
            if (d.krange == 1) hi = (i + 1 < hi) ? i + 1 : hi;
            if (d.krange == 2) lo = (i > lo) ? i : lo;
            if (lo >= hi) continue;
            const int64_t cols = d.outmask ? ((i + 1 < d.N) ? i + 1 : d.N) : d.N;
            pairs += (double)cols * (double)(hi - lo);
        }
    }
    return 2.0 * pairs * (double)d.batch;
}

namespace {
struct Traced {
    const LaunchTrace* tr;
    void begin() const { if (tr && tr->begin) tr->begin(tr->ctx); }
    void end(double flops, double bytes) const { if (tr && tr->end) tr->end(tr->ctx, g_launched, flops, bytes); }
};
}  // namespace

namespace {
KArgs make_args(const GemmDesc& d) {
    KArgs a{};
    a.M = d.M; a.N = d.N; a.K = d.K; a.kseg = d.K > 0 ? d.kseg : 1;
    a.A = d.A; a.lda = d.lda; a.B = d.B; a.ldb = d.ldb; a.C = d.C; a.ldc = d.ldc; a.R = d.R;
    a.H = d.H; a.sAb = d.sAb; a.sAh = d.sAh; a.sBb = d.sBb; a.sBh = d.sBh; a.sCb = d.sCb; a.sCh = d.sCh;
    a.outmask = d.outmask; a.mode = d.mode; a.krange = d.krange; a.scale = d.scale;
    a.split = 0; a.part = nullptr; a.chunk = -1; a.tm_lo = 0;
    a.rope_cos = d.rope_cos; a.rope_sin = d.rope_sin; a.rope_T = d.rope_T; a.rope_cols = d.rope_cols;
    return a;
}

// float4 loads need 16-byte alignment and a leading dimension that covers
// the contiguous extent rounded up to 4 (the slack is read, then masked)
bool vec_loads(const GemmDesc& d) {
    auto up4 = [](int64_t x) { return (x + 3) / 4 * 4; };
    const bool v = aligned16(d.A) && aligned16(d.B) && d.lda % 4 == 0 && d.ldb % 4 == 0 &&
                   d.sAb % 4 == 0 && d.sAh % 4 == 0 && d.sBb % 4 == 0 && d.sBh % 4 == 0;
    return v && (d.a_kc ? up4(d.K) <= d.lda : up4(d.M) <= d.lda) && (d.b_kc ? up4(d.K) <= d.ldb : up4(d.N) <= d.ldb);
}

// The split partials of a (already written) added in chunk order, then the
// epilogue mode: the second kernel of the split path.
bool fold_v4(const GemmDesc& d, const KArgs& a) {
    return d.N % 4 == 0 && d.ldc % 4 == 0 && aligned16(d.C) && aligned16(a.part) && (d.mode != 3 || aligned16(d.R));
}
int64_t fold4_blocks(const GemmDesc& d) { return (d.M * d.N / 4 + 255) / 256; }

void launch_fold(const GemmDesc& d, const KArgs& a, hipStream_t s) {
    const int64_t n = d.M * d.N;
    if (fold_v4(d, a)) k_fold4<<<(unsigned)fold4_blocks(d), 256, 0, s>>>(d.M, d.N, a);
    else k_fold<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a.part, a.nsplit, d.M, d.N, a);
}
}  // namespace

int gemm(const GemmDesc& d, const GemmPlan& p, hipStream_t s, const LaunchTrace* tr) {
    std::snprintf(g_launched, sizeof g_launched, "none");
    const Traced t{tr};
    if (!desc_ok(d)) return -1;
    if (d.M == 0 || d.N == 0) return 0;
    KArgs a = make_args(d);
    KArgs none{};   // no second problem in the launch
    // The causal attention contractions of 64-wide heads (tiled P, square,
    // one segment) have their own kernel when the plan leaves the choice open.
    if (p.tile < 0 && p.split < 0 && !p.simple && d.a_blk && d.mode == 0 && !d.outmask && !d.b_kc &&
        d.M == d.K && d.kseg == d.K && ((d.krange == 1 && d.a_kc) || (d.krange == 2 && !d.a_kc)) &&
        attn_av_fits(d.M, d.N, d.batch, d.H, d.A, d.lda, d.sAb, d.sAh, d.B, d.ldb, d.sBb, d.sBh)) {
        std::snprintf(g_launched, sizeof g_launched, "k_attn_av<%d>", d.krange);
        t.begin();
        const int r = attn_av(d.krange, d.M, d.N, d.batch, d.H, d.A, d.lda, d.sAb, d.sAh, d.B, d.ldb, d.sBb, d.sBh,
                              d.C, d.ldc, d.sCb, d.sCh, d.rope_cos, d.rope_sin, s);
        t.end(gemm_flops(d, 0, d.K), 0.0);
        return r;
    }
    if (p.simple || d.K == 0) {
        const int64_t n = d.M * d.N;
        const dim3 grid((unsigned)((n + 255) / 256), 1, (unsigned)d.batch);
        std::snprintf(g_launched, sizeof g_launched, "k_gemm_simple");
        t.begin();
        k_gemm_simple<<<grid, 256, 0, s>>>(a, d.a_kc ? 1 : 0, d.b_kc ? 1 : 0);
        t.end(gemm_flops(d, 0, d.K), 0.0);
        return hipGetLastError() == hipSuccess ? 0 : -3;
    }
    const bool vec = vec_loads(d);
    const bool rope = d.rope_cos != nullptr;
    if (rope && (!d.rope_sin || d.rope_T <= 0 || d.rope_cols % 64 != 0 || d.rope_cols > d.N || d.mode != 0 ||
                 d.krange != 0 || d.outmask || d.batch != 1 || p.simple || p.tile == 1 || p.split == 1))
        return -1;
    const bool split = !rope && want_split(d, p);
    // Tiles: 128x64 for causal ranges (their work per row tile grows along
    // the diagonal) and 256x64 for 64-wide outputs; otherwise 128x128 or
    // 128x64, whichever grid is expected to finish first (grid_cost).
    int cfg = p.tile;
    if (cfg < 0) {
        const int64_t per = (split ? nchunks(d) : 1) * d.batch;
        const int64_t wg128 = ((d.M + 127) / 128) * ((d.N + 127) / 128) * per;
        const int64_t wg64 = ((d.M + 127) / 128) * ((d.N + 63) / 64) * per;
        cfg = d.krange != 0 ? 2 : (d.N <= 64 && !rope ? 1 : (grid_cost(wg64, 0.55) < grid_cost(wg128, 1.0) ? 2 : 0));
    }
    int64_t nsplit = 1;
    if (split) {
        nsplit = nchunks(d);
        if (!p.scratch || p.scratch_floats < nsplit * d.M * d.N) return -2;
        a.split = 1;
        a.part = p.scratch;
    }
    // A causal contraction over several chunks runs one launch per chunk in
    // chunk order, each over the row tiles that chunk touches: the row's first
    // chunk stores, later ones add, which is the rule's left fold t0 + t1 + ...
    // Only for mode 0 (an existing C would be added before the fold ends) and
    // when every row's range is non-empty.
    const int64_t nch = nchunks(d);
    if (d.krange != 0 && nch > 1 && p.split != 0 && d.mode == 0 && !d.outmask &&
        (d.krange == 1 || d.M <= d.K) && cfg == 2 && KC % tile_rows(cfg) == 0) {
        const int64_t MT = tile_rows(cfg), tiles = (d.M + MT - 1) / MT;
        for (int64_t c = 0; c < nch; ++c) {
            int64_t lo, hi;   // row tiles with a non-empty range in chunk c
            if (d.krange == 1) { lo = c * KC / MT; hi = tiles; }
            else { lo = 0; const int64_t e = (c + 1) * KC < d.M ? (c + 1) * KC : d.M; hi = (e + MT - 1) / MT; }
            if (lo >= hi) continue;
            a.chunk = c;
            set_grid(a, d, cfg, 1, lo, hi - lo);
            t.begin();
            if (!launch_tiled(d, a, none, cfg, vec, false, s)) return -1;
            t.end(gemm_flops(d, c * KC, (c + 1) * KC), 0.0);
            if (hipGetLastError() != hipSuccess) return -3;
        }
        return 0;
    }
    // several chunks (or segments) per workgroup need the running total
    const bool mc = !split && nch > 1;
    set_grid(a, d, cfg, nsplit);
    t.begin();
    if (!launch_tiled(d, a, none, cfg, vec, mc, s)) {
        if (split || rope) return -1;
        const int64_t n = d.M * d.N;
        const dim3 grid((unsigned)((n + 255) / 256), 1, (unsigned)d.batch);
        std::snprintf(g_launched, sizeof g_launched, "k_gemm_simple");
        k_gemm_simple<<<grid, 256, 0, s>>>(a, d.a_kc ? 1 : 0, d.b_kc ? 1 : 0);
        t.end(gemm_flops(d, 0, d.K), 0.0);
        return hipGetLastError() == hipSuccess ? 0 : -3;
    }
    t.end(gemm_flops(d, 0, d.K), 0.0);
    if (hipGetLastError() != hipSuccess) return -3;
    if (split) {
        const int64_t n = d.M * d.N;
        char main_kernel[sizeof g_launched];
        std::memcpy(main_kernel, g_launched, sizeof g_launched);
        std::snprintf(g_launched, sizeof g_launched, "k_fold");
        t.begin();
        launch_fold(d, a, s);
        // partials read, output written (and read when accumulating)
        t.end(0.0, 4.0 * (double)n * (double)(nsplit + 1 + (d.mode == 1 || d.mode == 3 ? 1 : 0)));
        std::memcpy(g_launched, main_kernel, sizeof g_launched);
        if (hipGetLastError() != hipSuccess) return -3;
    }
    return 0;
}

int gemm_pair(const GemmDesc& d0, const GemmDesc& d1, const GemmPlan& p, hipStream_t s, const LaunchTrace* tr) {
    std::snprintf(g_launched, sizeof g_launched, "none");
    const Traced t{tr};
    if (!desc_ok(d0) || !desc_ok(d1)) return -1;
    // Only plain contractions of one layout and load width pair up, under the
    // automatic plan, both split into per-chunk partials or both one chunk.
    auto plain = [](const GemmDesc& d) {
        return d.M > 0 && d.N > 64 && d.K > 0 && d.krange == 0 && !d.outmask && d.batch == 1 && !d.rope_cos &&
               !d.a_blk;
    };
    const bool s0 = want_split(d0, p), s1 = want_split(d1, p);
    const int64_t n0 = nchunks(d0), n1 = nchunks(d1);
    const int64_t part0 = s0 ? n0 * d0.M * d0.N : 0, part1 = s1 ? n1 * d1.M * d1.N : 0;
    const bool same = plain(d0) && plain(d1) && d0.a_kc == d1.a_kc && d0.b_kc == d1.b_kc &&
                      vec_loads(d0) == vec_loads(d1) && p.tile < 0 && p.split < 0 && !p.simple &&
                      ((s0 && s1 && p.scratch && p.scratch_floats >= part0 + part1) || (n0 == 1 && n1 == 1));
    if (!same) {
        const int r = gemm(d0, p, s, tr);
        return r != 0 ? r : gemm(d1, p, s, tr);
    }
    KArgs a = make_args(d0), b = make_args(d1);
    const int64_t c0 = s0 ? n0 : 1, c1 = s1 ? n1 : 1;
    auto wg = [](const GemmDesc& d, int64_t nt, int64_t c) { return ((d.M + 127) / 128) * ((d.N + nt - 1) / nt) * c; };
    const int cfg = grid_cost(wg(d0, 64, c0) + wg(d1, 64, c1), 0.55) < grid_cost(wg(d0, 128, c0) + wg(d1, 128, c1), 1.0)
                        ? 2 : 0;
    if (s0) {
        a.split = 1; a.part = p.scratch;
        b.split = 1; b.part = p.scratch + part0;
    }
    set_grid(a, d0, cfg, c0);
    set_grid(b, d1, cfg, c1);
    t.begin();
    if (!launch_tiled(d0, a, b, cfg, vec_loads(d0), false, s)) return -1;
    t.end(gemm_flops(d0, 0, d0.K) + gemm_flops(d1, 0, d1.K), 0.0);
    if (hipGetLastError() != hipSuccess) return -3;
    if (s0) {
        char main_kernel[sizeof g_launched];
        std::memcpy(main_kernel, g_launched, sizeof g_launched);
        std::snprintf(g_launched, sizeof g_launched, "k_fold");
        auto fold_bytes = [](const GemmDesc& d, const KArgs& k) {
            return 4.0 * (double)(d.M * d.N) * (double)(k.nsplit + 1 + (d.mode == 1 || d.mode == 3 ? 1 : 0));
        };
        if (fold_v4(d0, a) && fold_v4(d1, b)) {   // both folds in one launch
            t.begin();
            const int64_t b0 = fold4_blocks(d0);
            k_fold4_pair<<<(unsigned)(b0 + fold4_blocks(d1)), 256, 0, s>>>(d0.M, d0.N, a, d1.M, d1.N, b, b0);
            t.end(0.0, fold_bytes(d0, a) + fold_bytes(d1, b));
            if (hipGetLastError() != hipSuccess) return -3;
        } else {
            for (int i = 0; i < 2; ++i) {
                const GemmDesc& d = i ? d1 : d0;
                const KArgs& k = i ? b : a;
                t.begin();
                launch_fold(d, k, s);
                t.end(0.0, fold_bytes(d, k));
                if (hipGetLastError() != hipSuccess) return -3;
            }
        }
        std::memcpy(g_launched, main_kernel, sizeof g_launched);
    }
    return 0;
}

}  // namespace mlb
