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

#include "mlb_device.hpp"
#include "mlb_internal.hpp"

namespace mlb {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
constexpr int KT = 32;
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
};

__device__ __forceinline__ void epilogue_store(const KArgs& a, float* C, int64_t gi, int64_t gj, float v) {
    float* p = C + gi * a.ldc + gj;
    if (a.mode == 0) *p = v;
    else if (a.mode == 1) *p = *p + v;
    else if (a.mode == 2) *p = v * a.scale;
    else *p = a.R[gi * a.ldc + gj] + v;
}

template <bool AKC, bool BKC, int WM, int WN, int KR, bool VEC>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm(KArgs a) {
    constexpr int MT = 64 * WM, NT = 64 * WN, NTHR = 64 * WM * WN;
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

    // XCD-aware tile order, then grouped rows.
    const int64_t w = blockIdx.x, nt = a.ntiles;
    const int64_t xcd = w & 7, idx = w >> 3, base = nt >> 3, rem = nt & 7;
    const int64_t logical = xcd * base + (xcd < rem ? xcd : rem) + idx;
    constexpr int64_t GM = 8;
    const int64_t per_group = GM * a.tiles_n;
    const int64_t first_m = (logical / per_group) * GM;
    const int64_t gsize = (a.tiles_m - first_m) < GM ? (a.tiles_m - first_m) : GM;
    const int64_t tm = first_m + (logical % per_group) % gsize;
    const int64_t tn = (logical % per_group) / gsize;
    const int64_t i0 = tm * MT, j0 = tn * NT;
    if (a.outmask && j0 > i0 + MT - 1) return;   // whole tile above the diagonal: nothing to write

    const int64_t z = blockIdx.z, zb = z / a.H, zh = z % a.H;
    const float* __restrict__ A = a.A + zb * a.sAb + zh * a.sAh;
    const float* __restrict__ B = a.B + zb * a.sBb + zh * a.sBh;
    float* C = a.C + zb * a.sCb + zh * a.sCh;

    int64_t kbeg = 0, kend = a.K;
    if (a.split) { kbeg = (int64_t)blockIdx.y * KC; kend = (kbeg + KC < a.K) ? kbeg + KC : a.K; }
    if (KR == 1) kend = (kend < i0 + MT) ? kend : i0 + MT;
    if (KR == 2) kbeg = (kbeg > i0) ? kbeg : i0;
    const int64_t kt0 = kbeg / KT, kt1 = (kend + KT - 1) / KT;

    v16f acc[2][2], tot[2][2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) { acc[r][c][e] = 0.0f; tot[r][c][e] = 0.0f; }
    bool have[2] = {false, false}, dirty[2] = {false, false};
    int64_t bi0[2];
    bi0[0] = i0 + wm * 64;
    bi0[1] = bi0[0] + 32;

    float ra[EA * W], rb[EB * W];
    auto load_global = [&](int64_t kt) {
        const int64_t k0 = kt * KT;
#pragma unroll
        for (int s = 0; s < EA; ++s) {
            const int q = tid + s * NTHR;
            int64_t gi, gk;
            if (AKC) { gi = i0 + q / (KT / W); gk = k0 + (q % (KT / W)) * W; }
            else { gk = k0 + q / (MT / W); gi = i0 + (q % (MT / W)) * W; }
            if (VEC) {
                if (gk < a.K && gi < a.M) {
                    const float4 v = AKC ? *reinterpret_cast<const float4*>(A + gi * a.lda + gk)
                                         : *reinterpret_cast<const float4*>(A + gk * a.lda + gi);
                    ra[s * 4 + 0] = v.x; ra[s * 4 + 1] = v.y; ra[s * 4 + 2] = v.z; ra[s * 4 + 3] = v.w;
                } else {
                    const float f = (gk >= a.K) ? -0.0f : 0.0f;
                    ra[s * 4 + 0] = f; ra[s * 4 + 1] = f; ra[s * 4 + 2] = f; ra[s * 4 + 3] = f;
                }
            } else {
                if (gk >= a.K) ra[s] = -0.0f;
                else if (gi >= a.M) ra[s] = 0.0f;
                else ra[s] = AKC ? A[gi * a.lda + gk] : A[gk * a.lda + gi];
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
    auto store_lds = [&]() {
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
    };
    auto a_lds = [&](int i, int k) -> float { return AKC ? As[i * ALD + k] : As[k * ALD + i]; };
    auto b_lds = [&](int k, int j) -> float { return BKC ? Bs[j * BLD + k] : Bs[k * BLD + j]; };
    auto fold = [&](int r) {
        if (!dirty[r]) return;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                tot[r][c][e] = have[r] ? tot[r][c][e] + acc[r][c][e] : acc[r][c][e];
                acc[r][c][e] = 0.0f;
            }
        have[r] = true;
        dirty[r] = false;
    };

    int64_t prev_chunk = -1;
    if (kt0 < kt1) load_global(kt0);
    for (int64_t kt = kt0; kt < kt1; ++kt) {
        const int64_t k0 = kt * KT;
        __syncthreads();
        store_lds();
        __syncthreads();
        if (kt + 1 < kt1) load_global(kt + 1);
        const int64_t chunk = (k0 / a.kseg) * (a.kseg / KC + 1) + (k0 % a.kseg) / KC;
        if (chunk != prev_chunk) {
            if (prev_chunk >= 0 && !a.split) { fold(0); fold(1); }
            prev_chunk = chunk;
        }
        // per row-block: 0 skip, 1 full tile on the matrix cores, 2 diagonal tile on the VALU
        int st[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            if (KR == 0) st[r] = 1;
            else if (KR == 1) st[r] = (k0 < bi0[r]) ? 1 : (k0 == bi0[r] ? 2 : 0);
            else st[r] = (k0 > bi0[r]) ? 1 : (k0 == bi0[r] ? 2 : 0);
            if (st[r]) dirty[r] = true;
        }
        const int lk = lane >> 5, li = lane & 31;
        if (st[0] == 1 && st[1] == 1) {
#pragma unroll 4
            for (int p = 0; p < KT / 2; ++p) {
                const int kk = 2 * p + lk;
                const float a0 = a_lds(wm * 64 + li, kk);
                const float a1 = a_lds(wm * 64 + 32 + li, kk);
                const float b0 = b_lds(kk, wn * 64 + li);
                const float b1 = b_lds(kk, wn * 64 + 32 + li);
                acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
                acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
                acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
                acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
            }
        } else if (KR != 0) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                if (st[r] == 1) {
                    for (int p = 0; p < KT / 2; ++p) {
                        const int kk = 2 * p + lk;
                        const float av = a_lds(wm * 64 + r * 32 + li, kk);
                        const float b0 = b_lds(kk, wn * 64 + li);
                        const float b1 = b_lds(kk, wn * 64 + 32 + li);
                        acc[r][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b0, acc[r][0], 0, 0, 0);
                        acc[r][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b1, acc[r][1], 0, 0, 0);
                    }
                } else if (st[r] == 2) {
                    // per-element chains over this tile's 32 k in ascending order
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const int jl = wn * 64 + c * 32 + li;
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int il = wm * 64 + r * 32 + 8 * (e >> 2) + 4 * lk + (e & 3);
                            const int64_t gi = i0 + il;
                            float v = acc[r][c][e];
                            for (int kk = 0; kk < KT; ++kk) {
                                const int64_t gk = k0 + kk;
                                const bool ok = (KR == 1 ? gk <= gi : gk >= gi) && gk < a.K;
                                if (ok) v = __builtin_fmaf(a_lds(il, kk), b_lds(kk, jl), v);
                            }
                            acc[r][c][e] = v;
                        }
                    }
                }
            }
        }
    }

    const int lk = lane >> 5, li = lane & 31;
    if (a.split) {
        float* part = a.part + (int64_t)blockIdx.y * a.M * a.N;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t gi = bi0[r] + 8 * (e >> 2) + 4 * lk + (e & 3);
                    const int64_t gj = j0 + wn * 64 + c * 32 + li;
                    if (gi < a.M && gj < a.N) part[gi * a.N + gj] = acc[r][c][e];
                }
        return;
    }
    fold(0);
    fold(1);
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t gi = bi0[r] + 8 * (e >> 2) + 4 * lk + (e & 3);
                const int64_t gj = j0 + wn * 64 + c * 32 + li;
                if (gi < a.M && gj < a.N && (!a.outmask || gj <= gi))
                    epilogue_store(a, C, gi, gj, have[r] ? tot[r][c][e] : 0.0f);
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
    epilogue_store(a, C, i, j, have ? total : 0.0f);
}

// total = part[0] + part[1] + ... in chunk order, then the epilogue.
__global__ __launch_bounds__(256) void k_fold(const float* __restrict__ part, int64_t nch, int64_t M,
                                              int64_t N, KArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t MN = M * N;
    if (idx >= MN) return;
    float t = part[idx];
    for (int64_t c = 1; c < nch; ++c) t = t + part[c * MN + idx];
    epilogue_store(a, a.C, idx / N, idx % N, t);
}

struct Cfg { int wm, wn; };

thread_local char g_launched[96];

template <bool AKC, bool BKC, int WM, int WN, int KR>
void launch_t(const KArgs& a, bool vec, dim3 grid, hipStream_t s) {
    std::snprintf(g_launched, sizeof g_launched, "k_gemm<%s, %s, %d, %d, %d, %s>", AKC ? "true" : "false",
                  BKC ? "true" : "false", WM, WN, KR, vec ? "true" : "false");
    if (vec) k_gemm<AKC, BKC, WM, WN, KR, true><<<grid, 64 * WM * WN, 0, s>>>(a);
    else k_gemm<AKC, BKC, WM, WN, KR, false><<<grid, 64 * WM * WN, 0, s>>>(a);
}

// Returns false when no tiled instantiation exists for the combination.
bool launch_tiled(const GemmDesc& d, KArgs a, int cfg, bool vec, int64_t nsplit, hipStream_t s) {
    const int WM = cfg == 0 ? 2 : 4, WN = cfg == 0 ? 2 : 1;
    a.tiles_m = (d.M + 64 * WM - 1) / (64 * WM);
    a.tiles_n = (d.N + 64 * WN - 1) / (64 * WN);
    a.ntiles = a.tiles_m * a.tiles_n;
    const dim3 grid((unsigned)a.ntiles, (unsigned)nsplit, (unsigned)d.batch);
    const int key = (d.a_kc ? 1 : 0) | (d.b_kc ? 2 : 0);
    if (d.krange == 0) {
        if (cfg == 0) {
            switch (key) {
                case 3: launch_t<true, true, 2, 2, 0>(a, vec, grid, s); return true;
                case 1: launch_t<true, false, 2, 2, 0>(a, vec, grid, s); return true;
                case 0: launch_t<false, false, 2, 2, 0>(a, vec, grid, s); return true;
                case 2: launch_t<false, true, 2, 2, 0>(a, vec, grid, s); return true;
            }
        } else {
            switch (key) {
                case 3: launch_t<true, true, 4, 1, 0>(a, vec, grid, s); return true;
                case 1: launch_t<true, false, 4, 1, 0>(a, vec, grid, s); return true;
                case 0: launch_t<false, false, 4, 1, 0>(a, vec, grid, s); return true;
                case 2: launch_t<false, true, 4, 1, 0>(a, vec, grid, s); return true;
            }
        }
    }
    if (d.krange == 1 && key == 1 && cfg == 1) { launch_t<true, false, 4, 1, 1>(a, vec, grid, s); return true; }
    if (d.krange == 2 && key == 0 && cfg == 1) { launch_t<false, false, 4, 1, 2>(a, vec, grid, s); return true; }
    return false;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

static bool desc_ok(const GemmDesc& d) {
    if (d.M < 0 || d.N < 0 || d.K < 0 || d.batch < 1 || d.H < 1 || d.batch % d.H != 0) return false;
    if (d.krange < 0 || d.krange > 2 || d.mode < 0 || d.mode > 3) return false;
    if (d.mode == 3 && (!d.R || d.batch != 1)) return false;
    if (d.K > 0 && (d.kseg <= 0 || d.K % d.kseg != 0)) return false;
    if (d.K > 0 && d.K / d.kseg > 1 && (d.kseg % KT != 0 || d.krange != 0)) return false;
    if (!d.A || !d.B || !d.C) return false;
    return true;
}

static int64_t nchunks(const GemmDesc& d) { return d.K > 0 ? (d.K + KC - 1) / KC : 0; }

// Whether per-chunk partials are worth it: only when the output has too few
// tiles to fill the chip. Never changes bits.
static bool split_useful(const GemmDesc& d, const GemmPlan& p) {
    if (p.split == 0 || d.krange != 0 || d.batch != 1 || d.outmask || d.K <= KC || d.K != d.kseg) return false;
    if (p.split == 1) return true;
    const int64_t tiles = ((d.M + 127) / 128) * ((d.N + 127) / 128);
    return tiles < 512;
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

int gemm(const GemmDesc& d, const GemmPlan& p, hipStream_t s) {
    std::snprintf(g_launched, sizeof g_launched, "none");
    if (!desc_ok(d)) return -1;
    if (d.M == 0 || d.N == 0) return 0;
    KArgs a{};
    a.M = d.M; a.N = d.N; a.K = d.K; a.kseg = d.K > 0 ? d.kseg : 1;
    a.A = d.A; a.lda = d.lda; a.B = d.B; a.ldb = d.ldb; a.C = d.C; a.ldc = d.ldc; a.R = d.R;
    a.H = d.H; a.sAb = d.sAb; a.sAh = d.sAh; a.sBb = d.sBb; a.sBh = d.sBh; a.sCb = d.sCb; a.sCh = d.sCh;
    a.outmask = d.outmask; a.mode = d.mode; a.krange = d.krange; a.scale = d.scale;
    a.split = 0; a.part = nullptr;
    if (p.simple || d.K == 0) {
        const int64_t n = d.M * d.N;
        const dim3 grid((unsigned)((n + 255) / 256), 1, (unsigned)d.batch);
        std::snprintf(g_launched, sizeof g_launched, "k_gemm_simple");
        k_gemm_simple<<<grid, 256, 0, s>>>(a, d.a_kc ? 1 : 0, d.b_kc ? 1 : 0);
        return hipGetLastError() == hipSuccess ? 0 : -3;
    }
    bool vec = aligned16(d.A) && aligned16(d.B) && d.lda % 4 == 0 && d.ldb % 4 == 0 &&
               d.sAb % 4 == 0 && d.sAh % 4 == 0 && d.sBb % 4 == 0 && d.sBh % 4 == 0;
    vec = vec && (d.a_kc ? d.K % 4 == 0 : d.M % 4 == 0) && (d.b_kc ? d.K % 4 == 0 : d.N % 4 == 0);
    int cfg = p.tile >= 0 ? p.tile : (d.N <= 64 ? 1 : 0);
    const bool split = want_split(d, p);
    int64_t nsplit = 1;
    if (split) {
        nsplit = nchunks(d);
        if (!p.scratch || p.scratch_floats < nsplit * d.M * d.N) return -2;
        a.split = 1;
        a.part = p.scratch;
    }
    if (!launch_tiled(d, a, cfg, vec, nsplit, s)) {
        if (split) return -1;
        const int64_t n = d.M * d.N;
        const dim3 grid((unsigned)((n + 255) / 256), 1, (unsigned)d.batch);
        std::snprintf(g_launched, sizeof g_launched, "k_gemm_simple");
        k_gemm_simple<<<grid, 256, 0, s>>>(a, d.a_kc ? 1 : 0, d.b_kc ? 1 : 0);
        return hipGetLastError() == hipSuccess ? 0 : -3;
    }
    if (hipGetLastError() != hipSuccess) return -3;
    if (split) {
        const int64_t n = d.M * d.N;
        k_fold<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p.scratch, nsplit, d.M, d.N, a);
        if (hipGetLastError() != hipSuccess) return -3;
    }
    return 0;
}

}  // namespace mlb
