// Lower-triangle contractions of attention: the scores S = (q . k) * scale and
// the probability gradient dP = dO . v, both over the head dimension (K <= 64,
// a single chunk of the G1024 rule: one fma chain per output from +0 in
// ascending k). Only outputs with j <= i are computed and written. For dP the
// softmax backward can run in the epilogue: dS = (P * (dP - D_i)) * scale,
// element by element, the same three roundings as a separate pass.
//
// Design: K is small, so a workgroup loads its whole 128 x K slices of both
// operands into LDS once (padded to 64 with A = -0, B = +0, which leaves every
// chain unchanged), runs K/2 k-pairs of v_mfma_f32_32x32x2_f32 per 32x32 block
// (ascending k, the same chain as the general contraction kernel), and writes
// the tile. Only tiles on or below the diagonal are launched (triangular tile
// numbering), so there are no empty workgroups; the kernel is bound by the
// HBM write of the triangle.
#include "mlb_device.hpp"
#include "mlb_internal.hpp"

namespace mlb {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
constexpr int TT = 128;       // tile edge
constexpr int KMAX = 64;      // largest K held in LDS
constexpr int LD = KMAX + 1;  // padded LDS row

struct TriArgs {
    int64_t T, K, H;
    const float* A; int64_t lda, sAb, sAh;
    const float* B; int64_t ldb, sBb, sBh;
    float* C; int64_t ldc, sCb, sCh;
    int scaled;
    float scale;
    int64_t nt;   // tiles per edge
    int vec;      // float4 loads: K % 4 == 0, 16-byte aligned rows and offsets
    int blk;      // C in the tiled 32x32 layout
    const float* P;   // non-null: write dS = (P * (t - D_i)) * ds_scale; P laid out as C
    const float* D;   // [batch, T]
    float ds_scale;
};

__global__ __launch_bounds__(256) void k_tri_nt(TriArgs a) {
    __shared__ float As[TT * LD];
    __shared__ float Bs[TT * LD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int lk = lane >> 5, li = lane & 31;
    // XCD-aware order (whole heads per XCD), then the triangular tile index
    // -> (tm, tn), tn <= tm
    const int64_t lb = xcd_logical_block();
    const int64_t x = lb % gridDim.x, z = lb / gridDim.x;
    int64_t tm = (int64_t)((__builtin_sqrt(8.0 * (double)x + 1.0) - 1.0) * 0.5);
    while ((tm + 1) * (tm + 2) / 2 <= x) ++tm;
    while (tm * (tm + 1) / 2 > x) --tm;
    const int64_t tn = x - tm * (tm + 1) / 2;
    const int64_t i0 = tm * TT, j0 = tn * TT;
    const int64_t zb = z / a.H, zh = z % a.H;
    const float* A = a.A + zb * a.sAb + zh * a.sAh;
    const float* B = a.B + zb * a.sBb + zh * a.sBh;
    float* C = a.C + zb * a.sCb + zh * a.sCh;
    const float* Pz = a.P ? a.P + zb * a.sCb + zh * a.sCh : nullptr;
    const float* Dz = a.D ? a.D + z * a.T : nullptr;

    if (a.vec) {
        // all 16 float4 loads of this thread in flight before any LDS store
        float4 va[8], vb[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int q = tid + 256 * s, r = q / (KMAX / 4), k = (q % (KMAX / 4)) * 4;
            const int64_t gi = i0 + r, gj = j0 + r;
            va[s] = (gi < a.T && k < a.K) ? *reinterpret_cast<const float4*>(A + gi * a.lda + k)
                                          : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            vb[s] = (gj < a.T && k < a.K) ? *reinterpret_cast<const float4*>(B + gj * a.ldb + k)
                                          : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int q = tid + 256 * s, r = q / (KMAX / 4), k = (q % (KMAX / 4)) * 4;
            const float av[4] = {va[s].x, va[s].y, va[s].z, va[s].w};
            const float bv[4] = {vb[s].x, vb[s].y, vb[s].z, vb[s].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                As[r * LD + k + e] = (k + e >= a.K) ? -0.0f : av[e];
                Bs[r * LD + k + e] = (k + e >= a.K) ? 0.0f : bv[e];
            }
        }
    } else {
        for (int q = tid; q < TT * KMAX; q += 256) {
            const int r = q / KMAX, k = q % KMAX;
            const int64_t gi = i0 + r, gj = j0 + r;
            float av, bv;
            if (k >= a.K) { av = -0.0f; bv = 0.0f; }
            else {
                av = gi < a.T ? A[gi * a.lda + k] : 0.0f;
                bv = gj < a.T ? B[gj * a.ldb + k] : 0.0f;
            }
            As[r * LD + k] = av;
            Bs[r * LD + k] = bv;
        }
    }
    __syncthreads();

    v16f c00, c01, c10, c11;
#pragma unroll
    for (int e = 0; e < 16; ++e) { c00[e] = 0.0f; c01[e] = 0.0f; c10[e] = 0.0f; c11[e] = 0.0f; }
    const int npair = (int)((a.K + 1) / 2);
    const int ra = wm * 64 + li, rb = wn * 64 + li;
    for (int p = 0; p < npair; ++p) {
        const int kk = 2 * p + lk;
        const float a0 = As[ra * LD + kk], a1 = As[(ra + 32) * LD + kk];
        const float b0 = Bs[rb * LD + kk], b1 = Bs[(rb + 32) * LD + kk];
        c00 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, c00, 0, 0, 0);
        c01 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, c01, 0, 0, 0);
        c10 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, c10, 0, 0, 0);
        c11 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, c11, 0, 0, 0);
    }
    auto offset = [&](int64_t gi, int64_t gj) -> int64_t {
        return a.blk ? ((((gi >> 5) * (a.ldc >> 5) + (gj >> 5)) << 10) + ((gi & 31) << 5) + (gj & 31))
                     : gi * a.ldc + gj;
    };
    // Tiles strictly below the diagonal and inside T store every element with
    // no per-element branch (a branch around each store makes each one wait
    // for the previous); the diagonal and edge tiles mask j <= i < T.
    const bool full = tn < tm && i0 + TT <= a.T;
    auto store = [&](const v16f& v, int rbase, int cbase) {
        const int64_t gj = j0 + wn * 64 + cbase + li;
        auto row = [&](int e) -> int64_t { return i0 + wm * 64 + rbase + 8 * (e >> 2) + 4 * lk + (e & 3); };
        float x[16];
        if (Pz) {
            // all loads of the block first (P and C are different arrays), then the stores
            float pv[16], dv[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t gi = row(e);
                const bool in = full || (gi < a.T && gj <= gi);
                pv[e] = in ? Pz[offset(gi, gj)] : 0.0f;
                dv[e] = in ? Dz[gi] : 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) x[e] = (pv[e] * (v[e] - dv[e])) * a.ds_scale;
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) x[e] = a.scaled ? v[e] * a.scale : v[e];
        }
        if (full) {
#pragma unroll
            for (int e = 0; e < 16; ++e) C[offset(row(e), gj)] = x[e];
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t gi = row(e);
                if (gi < a.T && gj <= gi) C[offset(gi, gj)] = x[e];
            }
        }
    };
    store(c00, 0, 0);
    store(c01, 0, 32);
    store(c10, 32, 0);
    store(c11, 32, 32);
}

// ----------------------------------------------------------------------------
// Causal contractions against the attention matrix for 64-wide heads:
//   KR 1: C[i][c] = sum over k <= i of P[i][k] B[k][c]   (O = P v, dQ = dS k)
//   KR 2: C[j][c] = sum over k >= j of P[k][j] B[k][c]   (dV = P^T dO, dK = dS^T q)
// P is [T, T] per head in 32x32 tiles (4 KiB contiguous, row-major inside,
// T/32 tiles per tile row); B and C are row-major with their own strides.
// G1024: every output is an fma chain from +0 in ascending k over each
// 1024-chunk of k intersected with its causal range; the non-empty chunk
// results are added left to right (here in registers: the chunk accumulator
// is folded into a running total when k crosses a multiple of 1024).
//
// A workgroup (4 waves, each one 32x32 MFMA block) owns 64 output rows x 64
// columns of two row tiles, r and T/64 - 1 - r, one after the other. Along the
// diagonal the k range of tile r has r + 1 (KR 1) or T/64 - r (KR 2) stages
// of 64, so every pair holds T/64 + 1 stages and all workgroups finish
// together. Each stage stages 64x64 of P and 64x64 of B through LDS with the
// next stage prefetched into registers (across the switch to the second tile
// as well). The 32x32 blocks that straddle the diagonal take the MFMA pair for
// rows that use both terms and one fma for the row that uses only one, in the
// same ascending order. Upper-triangle parts of P that a stage loads are never
// used.
constexpr int AV = 64;          // rows per tile, k per stage, output columns
constexpr int AV_BLD = AV + 4;  // LDS row of B, and of A when k-major (KR 2)

struct AvArgs {
    int64_t T, H, npairs;
    const float* A; int64_t sAb, sAh;
    const float* B; int64_t ldb, sBb, sBh;
    float* C; int64_t ldc, sCb, sCh;
};

template <int KR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void k_attn_av(AvArgs a) {
    // KR 1: A(i, k) = P[i][k], held i-major (row stride 65: the lanes of a
    // wave read 32 rows at one k without bank conflicts). KR 2: A(j, k) =
    // P[k][j], held k-major as loaded.
    constexpr int ALD = KR == 1 ? AV + 1 : AV_BLD;
    __shared__ float As[AV * ALD];
    __shared__ float Bs[AV * AV_BLD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave & 1, wc = wave >> 1;   // the wave's 32-row and 32-column block
    const int lk = lane >> 5, li = lane & 31;
    const int64_t lb = xcd_logical_block();   // whole heads per XCD: B stays in one L2
    const int64_t z = lb / a.npairs, pr = lb % a.npairs;
    const int64_t zb = z / a.H, zh = z % a.H;
    const float* __restrict__ P = a.A + zb * a.sAb + zh * a.sAh;
    const float* __restrict__ Bm = a.B + zb * a.sBb + zh * a.sBh;
    float* __restrict__ C = a.C + zb * a.sCb + zh * a.sCh;
    const int64_t nrt = a.T / AV, ptr = a.T / 32;   // row tiles; P tiles per tile row
    const int64_t ta = pr, tb = nrt - 1 - pr;       // tb == ta: a single tile
    auto nstages = [&](int64_t t) -> int64_t { return KR == 1 ? t + 1 : nrt - t; };
    auto first_k = [&](int64_t t) -> int64_t { return KR == 1 ? 0 : t * AV; };
    const int64_t na = nstages(ta), nsteps = na + (tb != ta ? nstages(tb) : 0);

    // prefetch registers as scalars and helpers forced inline: an array of
    // float4 captured by the lambdas was placed in scratch memory, which made
    // every load wait for its data at once
    float ra[16], rb[16];
    auto load = [&](int64_t st) __attribute__((always_inline)) {
        const int64_t t = st < na ? ta : tb;
        const int64_t k0 = first_k(t) + AV * (st < na ? st : st - na), r0 = t * AV;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int q = tid + 256 * s, b = q >> 8, w = q & 255;
            // P tile (b >> 1, b & 1) of the stage: KR 1 (rows r0.., k0..), KR 2 (rows k0.., cols r0..)
            const int64_t pr_ = (KR == 1 ? r0 : k0) / 32 + (b >> 1), pc_ = (KR == 1 ? k0 : r0) / 32 + (b & 1);
            const float4 va = *reinterpret_cast<const float4*>(P + ((pr_ * ptr + pc_) << 10) + w * 4);
            const float4 vb = *reinterpret_cast<const float4*>(Bm + (k0 + (q >> 4)) * a.ldb + (q & 15) * 4);
            ra[4 * s + 0] = va.x; ra[4 * s + 1] = va.y; ra[4 * s + 2] = va.z; ra[4 * s + 3] = va.w;
            rb[4 * s + 0] = vb.x; rb[4 * s + 1] = vb.y; rb[4 * s + 2] = vb.z; rb[4 * s + 3] = vb.w;
        }
    };
    auto store_lds = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int q = tid + 256 * s, b = q >> 8, w = q & 255;
            const int rr = 32 * (b >> 1) + (w >> 3), cc = 32 * (b & 1) + (w & 7) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                As[rr * ALD + cc + e] = ra[4 * s + e];
                Bs[(q >> 4) * AV_BLD + (q & 15) * 4 + e] = rb[4 * s + e];
            }
        }
    };
    auto a_lds = [&](int r, int k) -> float { return KR == 1 ? As[r * ALD + k] : As[k * ALD + r]; };
    const int rl = 32 * wr, cl = 32 * wc + li;   // wave's first local row; lane's local column

    v16f acc, tot;
#pragma unroll
    for (int e = 0; e < 16; ++e) { acc[e] = 0.0f; tot[e] = 0.0f; }
    bool have = false, dirty = false;
    load(0);
    for (int64_t st = 0; st < nsteps; ++st) {
        const bool second = st >= na;
        const int64_t t = second ? tb : ta, sl = second ? st - na : st;
        const int64_t k0 = first_k(t) + AV * sl, rb0 = t * AV + rl;   // stage k, the wave's first row
        __syncthreads();
        store_lds();
        __syncthreads();
        if (st + 1 < nsteps) load(st + 1);
        if (sl > 0 && k0 % 1024 == 0 && dirty) {   // a new chunk: fold the finished one
#pragma unroll
            for (int e = 0; e < 16; ++e) { tot[e] = have ? tot[e] + acc[e] : acc[e]; acc[e] = 0.0f; }
            have = true;
            dirty = false;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t kb0 = k0 + 32 * h;
            const int ko = 32 * h;
            const int stt = KR == 1 ? (kb0 < rb0 ? 1 : (kb0 == rb0 ? 2 : 0)) : (kb0 > rb0 ? 1 : (kb0 == rb0 ? 2 : 0));
            if (stt == 1) {
                dirty = true;
#pragma unroll 8
                for (int p = 0; p < 16; ++p) {
                    const int kk = ko + 2 * p + lk;
                    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a_lds(rl + li, kk), Bs[kk * AV_BLD + cl], acc, 0, 0, 0);
                }
            } else if (stt == 2) {
                // diagonal block: per k-pair (ka, kb) relative to the block's
                // first row, rows that take both terms keep the pair's result,
                // the one row whose range ends between them takes one fma
                dirty = true;
#pragma unroll 1
                for (int p = 0; p < 16; ++p) {
                    const int kk = ko + 2 * p + lk;
                    const v16f n = __builtin_amdgcn_mfma_f32_32x32x2f32(a_lds(rl + li, kk), Bs[kk * AV_BLD + cl], acc,
                                                                        0, 0, 0);
                    const int ka = 2 * p, kb = 2 * p + 1;
                    const int ks = KR == 1 ? ka : kb;   // the single term's k, also its row
                    const float as = a_lds(rl + ks, ko + ks), bs = Bs[(ko + ks) * AV_BLD + cl];
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int il = 8 * (e >> 2) + 4 * lk + (e & 3);
                        const bool both = KR == 1 ? (il >= kb) : (il <= ka);
                        const float s1 = __builtin_fmaf(as, bs, acc[e]);
                        acc[e] = both ? n[e] : (il == ks ? s1 : acc[e]);
                    }
                }
            }
        }
        const bool last = (st + 1 == nsteps) || (st + 1 == na);
        if (last) {   // the tile's outputs: fold the last chunk, store, reset
            float* Ct = C + (t * AV + rl) * a.ldc + 32 * wc + li;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float v = have ? (dirty ? tot[e] + acc[e] : tot[e]) : acc[e];
                Ct[(int64_t)(8 * (e >> 2) + 4 * lk + (e & 3)) * a.ldc] = v;
                acc[e] = 0.0f;
                tot[e] = 0.0f;
            }
            have = false;
            dirty = false;
        }
    }
}

}  // namespace

bool attn_av_fits(int64_t T, int64_t hd, int64_t batch, int64_t H, const float* P, int64_t ldp, int64_t sPb,
                  int64_t sPh, const float* B, int64_t ldb, int64_t sBb, int64_t sBh) {
    if (hd != AV || T <= 0 || T % AV != 0 || ldp != T || batch < 1 || H < 1 || batch % H) return false;
    return ((uintptr_t)P & 15u) == 0 && ((uintptr_t)B & 15u) == 0 && ldb % 4 == 0 && sBb % 4 == 0 && sBh % 4 == 0 &&
           sPb % 4 == 0 && sPh % 4 == 0;
}

int attn_av(int kr, int64_t T, int64_t hd, int64_t batch, int64_t H, const float* P, int64_t ldp, int64_t sPb,
            int64_t sPh, const float* B, int64_t ldb, int64_t sBb, int64_t sBh, float* C, int64_t ldc, int64_t sCb,
            int64_t sCh, hipStream_t s) {
    if (kr != 1 && kr != 2) return -1;
    if (!attn_av_fits(T, hd, batch, H, P, ldp, sPb, sPh, B, ldb, sBb, sBh)) return -2;
    const int64_t npairs = (T / AV + 1) / 2;
    AvArgs a{T, H, npairs, P, sPb, sPh, B, ldb, sBb, sBh, C, ldc, sCb, sCh};
    const dim3 grid((unsigned)(npairs * batch));
    if (kr == 1) k_attn_av<1><<<grid, 256, 0, s>>>(a);
    else k_attn_av<2><<<grid, 256, 0, s>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

int tri_nt(int64_t T, int64_t K, int64_t batch, int64_t H, const float* A, int64_t lda, int64_t sAb, int64_t sAh,
           const float* B, int64_t ldb, int64_t sBb, int64_t sBh, float* C, int64_t ldc, int64_t sCb, int64_t sCh,
           int scaled, float scale, int blk, const float* P, const float* D, float ds_scale, hipStream_t s) {
    if (T < 0 || K < 1 || K > KMAX || batch < 1 || H < 1 || batch % H) return -1;
    if ((P != nullptr) != (D != nullptr) || (P && scaled)) return -1;
    if (blk && (ldc % 32 != 0 || ldc < T)) return -1;
    if (T == 0) return 0;
    const bool vec = K % 4 == 0 && lda % 4 == 0 && ldb % 4 == 0 && sAb % 4 == 0 && sAh % 4 == 0 && sBb % 4 == 0 &&
                     sBh % 4 == 0 && ((uintptr_t)A & 15u) == 0 && ((uintptr_t)B & 15u) == 0;
    TriArgs a{T, K, H, A, lda, sAb, sAh, B, ldb, sBb, sBh, C, ldc, sCb, sCh, scaled, scale, (T + TT - 1) / TT,
              vec ? 1 : 0, blk ? 1 : 0, P, D, ds_scale};
    const int64_t ntri = a.nt * (a.nt + 1) / 2;
    k_tri_nt<<<dim3((unsigned)ntri, 1, (unsigned)batch), 256, 0, s>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace mlb
