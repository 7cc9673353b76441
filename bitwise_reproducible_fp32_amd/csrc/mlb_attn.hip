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
    // the wave index is uniform across the wave: saying so lets per-wave
    // branches be scalar branches instead of exec-mask divergence
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const float* rope_cos;   // non-null: inverse rotary embedding of the output rows (positions) before the store
    const float* rope_sin;
};

// Inverse rotary embedding of a wave's 32x32 output block at the end of a row
// tile: the pairs (i, i + 32) of a 64-wide head sit in the waves of column
// halves 0 and 1, so the block passes through LDS (buf, 64 rows of stride ld)
// and each lane takes its partner from the other half. The arithmetic is the
// rope kernel's backward rotation, element by element. Every wave of the
// workgroup calls it together.
__device__ __forceinline__ void rope_bwd_block(float (&q)[16], float* buf, int ld, int rl, int wc, int li, int lk,
                                               int64_t row0, const float* cosv, const float* sinv) {
    __syncthreads();   // every wave is done reading buf as an operand
#pragma unroll
    for (int e = 0; e < 16; ++e) buf[(rl + 8 * (e >> 2) + 4 * lk + (e & 3)) * ld + 32 * wc + li] = q[e];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int r = 8 * (e >> 2) + 4 * lk + (e & 3);
        const float other = buf[(rl + r) * ld + 32 * (1 - wc) + li];
        const int64_t t = row0 + r;
        const float c = cosv[t * 32 + li], sn = sinv[t * 32 + li];
        q[e] = wc == 0 ? (q[e] * c) + (other * sn) : (q[e] * c) - (other * sn);
    }
}

template <int KR, bool ROPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void k_attn_av(AvArgs a) {
    // KR 1: A(i, k) = P[i][k], held i-major (row stride 65: the lanes of a
    // wave read 32 rows at one k without bank conflicts). KR 2: A(j, k) =
    // P[k][j], held k-major as loaded.
    constexpr int ALD = KR == 1 ? AV + 1 : AV_BLD;
    __shared__ float As[AV * ALD];
    __shared__ float Bs[AV * AV_BLD];
    // the wave index is uniform across the wave: saying so lets per-wave
    // branches be scalar branches instead of exec-mask divergence
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    // Addresses: a workgroup-uniform base plus an unsigned 32-bit lane offset
    // (every offset inside one head is below 2^32 elements).
    auto load = [&](int64_t st) __attribute__((always_inline)) {
        const int64_t t = st < na ? ta : tb;
        const uint32_t k0 = (uint32_t)(first_k(t) + AV * (st < na ? st : st - na)), r0 = (uint32_t)(t * AV);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int q = tid + 256 * s, b = q >> 8, w = q & 255;
            // P tile (b >> 1, b & 1) of the stage: KR 1 (rows r0.., k0..), KR 2 (rows k0.., cols r0..)
            const uint32_t pr_ = (KR == 1 ? r0 : k0) / 32 + (uint32_t)(b >> 1);
            const uint32_t pc_ = (KR == 1 ? k0 : r0) / 32 + (uint32_t)(b & 1);
            const float4 va = *reinterpret_cast<const float4*>(P + (((pr_ * (uint32_t)ptr + pc_) << 10) + (uint32_t)w * 4));
            const float4 vb = *reinterpret_cast<const float4*>(
                Bm + ((k0 + (uint32_t)(q >> 4)) * (uint32_t)a.ldb + (uint32_t)(q & 15) * 4));
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
        // higher issue priority while this wave has matrix work (the waves of
        // the other workgroups on the SIMD are then staging or waiting)
        __builtin_amdgcn_s_setprio(1);
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
        __builtin_amdgcn_s_setprio(0);
        const bool last = (st + 1 == nsteps) || (st + 1 == na);
        if (last) {   // the tile's outputs: fold the last chunk, (rotate,) store, reset
            float v[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                v[e] = have ? (dirty ? tot[e] + acc[e] : tot[e]) : acc[e];
                acc[e] = 0.0f;
                tot[e] = 0.0f;
            }
            if (ROPE) rope_bwd_block(v, As, ALD, rl, wc, li, lk, t * AV + rl, a.rope_cos, a.rope_sin);
            const uint32_t co = (uint32_t)(t * AV + rl) * (uint32_t)a.ldc + (uint32_t)(32 * wc + li);
#pragma unroll
            for (int e = 0; e < 16; ++e) C[co + (uint32_t)(8 * (e >> 2) + 4 * lk + (e & 3)) * (uint32_t)a.ldc] = v[e];
            have = false;
            dirty = false;
        }
    }
}

// ----------------------------------------------------------------------------
// Row-strip kernels over the lower triangle for 64-wide heads. A workgroup
// owns two 64-row tiles (r and T/64 - 1 - r, so every workgroup has T/64 + 1
// steps) and walks each one's column tiles j0 = 0, 64, .., i0 in ascending
// order. Per step, each wave computes one 32x32 block of X Y^T over the 64
// head positions (an fma chain from +0 in ascending h, the rule for a single
// chunk) with the strip's X rows held in LDS for the whole row tile and the
// Y tile staged per step, the next one prefetched into registers.
//   scores (DS false): S = t * scale for j <= i, stored in the tiled layout.
//   DS true: t = dO . v (dP), dS = (P * (t - D_i)) * scale, stored tiled; and
//   in the same walk dQ_i = sum over j <= i of dS_ij k_j, whose ascending j
//   order is exactly its G1024 chain (chunks of 1024 folded in registers), so
//   dS is not read back for dQ. The diagonal block of dQ takes the MFMA pair
//   for rows that use both terms and one fma for the row that uses one.
struct RowsArgs {
    int64_t T, H, npairs;
    const float* X; int64_t ldx, sXb, sXh;   // q (scores) or dO (dS): rows i
    const float* Y; int64_t ldy, sYb, sYh;   // k (scores) or v (dS): rows j
    float* S; int64_t sSb, sSh;              // tiled [T, T] output
    float scale;
    const float* P;                          // dS: tiled P, strides of S
    const float* D;                          // dS: [batch][T]
    const float* K; int64_t ldk, sKb, sKh;   // dS: k rows (dQ's right operand)
    float* dQ; int64_t ldq, sQb, sQh;        // dS: dQ rows
};

template <bool DS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void k_attn_rows(RowsArgs a) {
    constexpr int LR = AV + 1;   // odd LDS row: 32 lanes reading 32 rows at one column hit 32 banks
    __shared__ float Xs[AV * LR];             // strip rows [i][h]
    __shared__ float Ys[AV * LR];             // Y tile [j][h], then (dS) the k tile [j][h]
    __shared__ float Ss[DS ? AV * LR : 1];    // dS tile [i][j] for the dQ contraction
    __shared__ float Dv[DS ? AV : 1];         // D of the strip's rows
    // the wave index is uniform across the wave: saying so lets per-wave
    // branches be scalar branches instead of exec-mask divergence
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave & 1, wc = wave >> 1;
    const int lk = lane >> 5, li = lane & 31;
    const int64_t lb = xcd_logical_block();
    const int64_t z = lb / a.npairs, pr = lb % a.npairs;
    const int64_t zb = z / a.H, zh = z % a.H;
    const float* __restrict__ X = a.X + zb * a.sXb + zh * a.sXh;
    const float* __restrict__ Y = a.Y + zb * a.sYb + zh * a.sYh;
    float* __restrict__ S = a.S + zb * a.sSb + zh * a.sSh;
    const float* __restrict__ Pz = DS ? a.P + zb * a.sSb + zh * a.sSh : nullptr;
    const float* __restrict__ Dz = DS ? a.D + z * a.T : nullptr;
    const float* __restrict__ Kz = DS ? a.K + zb * a.sKb + zh * a.sKh : nullptr;
    float* __restrict__ Q = DS ? a.dQ + zb * a.sQb + zh * a.sQh : nullptr;
    const int64_t nrt = a.T / AV, ptr = a.T / 32;
    const int64_t ta = pr, tb = nrt - 1 - pr;
    const int64_t na = ta + 1, nsteps = na + (tb != ta ? tb + 1 : 0);

    // prefetch registers (scalars, helpers inline: see k_attn_av)
    float rx[16], ry[16], rk[16];
    // Addresses are a workgroup-uniform base plus an unsigned 32-bit lane
    // offset (every per-head offset is below 2^32 / 4): one VGPR per address.
    // float4 s of thread tid: row (tid >> 3) + 32 (s & 1), columns 4 ((tid & 7) + 8 (s >> 1)) .. + 3
    // (a wave moves 8 rows x 8 float4: whole 128-byte lines from memory, and a
    // half-wave's LDS stores of one element cover 4 rows x 32 columns, 32 banks)
    auto load_rows = [&](const float* base, uint32_t ld, uint32_t r0, float* dst) __attribute__((always_inline)) {
        const uint32_t o = (r0 + (uint32_t)(tid >> 3)) * ld + (uint32_t)(tid & 7) * 4;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float4 v = *reinterpret_cast<const float4*>(base + (o + 32u * (uint32_t)(s & 1) * ld + 32u * (uint32_t)(s >> 1)));
            dst[4 * s + 0] = v.x; dst[4 * s + 1] = v.y; dst[4 * s + 2] = v.z; dst[4 * s + 3] = v.w;
        }
    };
    auto put_rows = [&](float* dst, const float* src) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int r = (tid >> 3) + 32 * (s & 1), c = 4 * ((tid & 7) + 8 * (s >> 1));
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[r * LR + c + e] = src[4 * s + e];
        }
    };
    auto tile_of = [&](int64_t st, int64_t& t, int64_t& sl) __attribute__((always_inline)) {
        const bool second = st >= na;
        t = second ? tb : ta;
        sl = second ? st - na : st;
    };
    // operands of step st: the strip rows (first step of a row tile) and the
    // Y tile; the k tile separately, later (it is used only after the dP part)
    auto prefetch_y = [&](int64_t st) __attribute__((always_inline)) {
        int64_t t, sl;
        tile_of(st, t, sl);
        if (sl == 0) load_rows(X, (uint32_t)a.ldx, (uint32_t)(t * AV), rx);
        load_rows(Y, (uint32_t)a.ldy, (uint32_t)(sl * AV), ry);
    };
    auto prefetch_k = [&](int64_t st) __attribute__((always_inline)) {
        int64_t t, sl;
        tile_of(st, t, sl);
        load_rows(Kz, (uint32_t)a.ldk, (uint32_t)(sl * AV), rk);
    };

    v16f qacc, qtot;
#pragma unroll
    for (int e = 0; e < 16; ++e) { qacc[e] = 0.0f; qtot[e] = 0.0f; }
    bool have = false, dirty = false;
    const int rl = 32 * wr;                   // the wave's first row in the strip
    auto row_of = [&](int e) -> int { return 8 * (e >> 2) + 4 * lk + (e & 3); };   // MFMA output row of element e
    prefetch_y(0);
    if (DS) prefetch_k(0);
    for (int64_t st = 0; st < nsteps; ++st) {
        int64_t t, sl;
        tile_of(st, t, sl);
        const int64_t i0 = t * AV, j0 = sl * AV;
        const bool diag_tile = sl == t;
        __syncthreads();                      // readers of the previous step's LDS are done
        if (sl == 0) {
            put_rows(Xs, rx);
            if (DS && tid < AV) Dv[tid] = Dz[i0 + tid];
        }
        put_rows(Ys, ry);
        __syncthreads();
        // this wave's block: rows i0 + rl, columns j0 + 32 wc; above the diagonal: nothing
        const bool active = !(diag_tile && wc > wr);
        // this wave's 32x32 block of the tiled [T, T] layouts, and the lane's column in it
        const uint32_t blk = ((uint32_t)((i0 + rl) >> 5) * (uint32_t)ptr + (uint32_t)((j0 >> 5) + wc)) << 10;
        // P is read once and S / dS written once: nontemporal, so that the
        // streams do not push the strip, v and k tiles out of L2
        float pv[16];
        if (DS && active) {
#pragma unroll
            for (int e = 0; e < 16; ++e) pv[e] = __builtin_nontemporal_load(Pz + (blk + (uint32_t)(row_of(e) * 32 + li)));
        }
        v16f acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
        if (active) {
#pragma unroll 8
            for (int p = 0; p < 32; ++p) {
                const int h = 2 * p + lk;
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Xs[(rl + li) * LR + h], Ys[(32 * wc + li) * LR + h], acc, 0,
                                                           0, 0);
            }
        }
        v16f& x = acc;   // the stored values, in place
        if (DS) {
#pragma unroll
            for (int e = 0; e < 16; ++e) x[e] = (pv[e] * (acc[e] - Dv[rl + row_of(e)])) * a.scale;
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) x[e] = acc[e] * a.scale;
        }
        if (active) {
            // The tiled block is contiguous (row r at r * 32). The diagonal
            // block is stored whole: its part above the diagonal is never
            // read as a value (the softmax and every contraction take j <= i
            // only, and the exported P shows +0 there).
#pragma unroll
            for (int e = 0; e < 16; ++e) __builtin_nontemporal_store(x[e], S + (blk + (uint32_t)(row_of(e) * 32 + li)));
        }
        if (DS) {
            __syncthreads();                  // every wave is done with the v tile
            if (active) {
#pragma unroll
                for (int e = 0; e < 16; ++e) Ss[(rl + row_of(e)) * LR + 32 * wc + li] = x[e];
            }
            put_rows(Ys, rk);                 // the k tile takes the v tile's place
            __syncthreads();
        }
        if (st + 1 < nsteps) prefetch_y(st + 1);
        if (DS) {
            // dQ rows i0 + rl, head columns 32 wc, over this tile's j
            if (sl > 0 && j0 % 1024 == 0 && dirty) {
#pragma unroll
                for (int e = 0; e < 16; ++e) { qtot[e] = have ? qtot[e] + qacc[e] : qacc[e]; qacc[e] = 0.0f; }
                have = true;
                dirty = false;
            }
            const int cq = 32 * wc + li;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int64_t kb0 = j0 + 32 * hh, rb0 = i0 + rl;
                const int ko = 32 * hh;
                const int stt = kb0 < rb0 ? 1 : (kb0 == rb0 ? 2 : 0);
                if (stt == 1) {
                    dirty = true;
#pragma unroll 8
                    for (int p = 0; p < 16; ++p) {
                        const int kk = ko + 2 * p + lk;
                        qacc = __builtin_amdgcn_mfma_f32_32x32x2f32(Ss[(rl + li) * LR + kk], Ys[kk * LR + cq], qacc, 0,
                                                                    0, 0);
                    }
                } else if (stt == 2) {
                    dirty = true;
#pragma unroll 1
                    for (int p = 0; p < 16; ++p) {
                        const int kk = ko + 2 * p + lk;
                        const v16f n = __builtin_amdgcn_mfma_f32_32x32x2f32(Ss[(rl + li) * LR + kk], Ys[kk * LR + cq],
                                                                            qacc, 0, 0, 0);
                        const int ka = 2 * p, kb = 2 * p + 1;
                        const float as = Ss[(rl + ka) * LR + ko + ka], bs = Ys[(ko + ka) * LR + cq];
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int il = row_of(e);
                            const float s1 = __builtin_fmaf(as, bs, qacc[e]);
                            qacc[e] = il >= kb ? n[e] : (il == ka ? s1 : qacc[e]);
                        }
                    }
                }
            }
            if (st + 1 < nsteps) prefetch_k(st + 1);
            if (diag_tile) {   // the row tile's last step: fold, store dQ, reset
                const uint32_t qo = (uint32_t)(i0 + rl) * (uint32_t)a.ldq + (uint32_t)cq;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    Q[qo + (uint32_t)row_of(e) * (uint32_t)a.ldq] = have ? (dirty ? qtot[e] + qacc[e] : qtot[e]) : qacc[e];
                    qacc[e] = 0.0f;
                    qtot[e] = 0.0f;
                }
                have = false;
                dirty = false;
            }
        }
    }
}

}  // namespace

bool attn_rows_fits(int64_t T, int64_t hd, int64_t batch, int64_t H, const float* X, int64_t ldx, int64_t sXb,
                    int64_t sXh, const float* Y, int64_t ldy, int64_t sYb, int64_t sYh, const float* S, int64_t ldS,
                    int64_t sSb, int64_t sSh) {
    if (hd != AV || T <= 0 || T % AV != 0 || ldS != T || batch < 1 || H < 1 || batch % H) return false;
    // lane offsets inside one head are unsigned 32-bit element counts
    const int64_t lim = (int64_t)1 << 32;
    if (T * T >= lim || T * ldx >= lim || T * ldy >= lim) return false;
    auto al = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
    return al(X) && al(Y) && al(S) && ldx % 4 == 0 && sXb % 4 == 0 && sXh % 4 == 0 && ldy % 4 == 0 && sYb % 4 == 0 &&
           sYh % 4 == 0 && sSb % 4 == 0 && sSh % 4 == 0;
}

int attn_rows(int64_t T, int64_t hd, int64_t batch, int64_t H, const float* X, int64_t ldx, int64_t sXb, int64_t sXh,
              const float* Y, int64_t ldy, int64_t sYb, int64_t sYh, float* S, int64_t ldS, int64_t sSb, int64_t sSh,
              float scale, const float* P, const float* D, const float* K, int64_t ldk, int64_t sKb, int64_t sKh,
              float* dQ, int64_t ldq, int64_t sQb, int64_t sQh, hipStream_t s) {
    if (!attn_rows_fits(T, hd, batch, H, X, ldx, sXb, sXh, Y, ldy, sYb, sYh, S, ldS, sSb, sSh)) return -2;
    const bool ds = P != nullptr;
    if (ds && (!D || !K || !dQ || ((uintptr_t)K & 15u) || ldk % 4 || sKb % 4 || sKh % 4 ||
               T * ldk >= ((int64_t)1 << 32) || T * ldq >= ((int64_t)1 << 32)))
        return -2;
    const int64_t npairs = (T / AV + 1) / 2;
    RowsArgs a{T, H, npairs, X, ldx, sXb, sXh, Y, ldy, sYb, sYh, S, sSb, sSh, scale,
               P, D, K, ldk, sKb, sKh, dQ, ldq, sQb, sQh};
    const dim3 grid((unsigned)(npairs * batch));
    if (ds) k_attn_rows<true><<<grid, 256, 0, s>>>(a);
    else k_attn_rows<false><<<grid, 256, 0, s>>>(a);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

bool attn_av_fits(int64_t T, int64_t hd, int64_t batch, int64_t H, const float* P, int64_t ldp, int64_t sPb,
                  int64_t sPh, const float* B, int64_t ldb, int64_t sBb, int64_t sBh) {
    if (hd != AV || T <= 0 || T % AV != 0 || ldp != T || batch < 1 || H < 1 || batch % H) return false;
    if (T * T >= ((int64_t)1 << 32) || T * ldb >= ((int64_t)1 << 32)) return false;   // 32-bit lane offsets
    return ((uintptr_t)P & 15u) == 0 && ((uintptr_t)B & 15u) == 0 && ldb % 4 == 0 && sBb % 4 == 0 && sBh % 4 == 0 &&
           sPb % 4 == 0 && sPh % 4 == 0;
}

int attn_av(int kr, int64_t T, int64_t hd, int64_t batch, int64_t H, const float* P, int64_t ldp, int64_t sPb,
            int64_t sPh, const float* B, int64_t ldb, int64_t sBb, int64_t sBh, float* C, int64_t ldc, int64_t sCb,
            int64_t sCh, const float* rope_cos, const float* rope_sin, hipStream_t s) {
    if (kr != 1 && kr != 2) return -1;
    if ((rope_cos != nullptr) != (rope_sin != nullptr)) return -1;
    if (!attn_av_fits(T, hd, batch, H, P, ldp, sPb, sPh, B, ldb, sBb, sBh)) return -2;
    const int64_t npairs = (T / AV + 1) / 2;
    AvArgs a{T, H, npairs, P, sPb, sPh, B, ldb, sBb, sBh, C, ldc, sCb, sCh, rope_cos, rope_sin};
    const dim3 grid((unsigned)(npairs * batch));
    // the rotary exchange is compiled only into the instances that use it
    if (kr == 1 && !rope_cos) k_attn_av<1, false><<<grid, 256, 0, s>>>(a);
    else if (kr == 1) k_attn_av<1, true><<<grid, 256, 0, s>>>(a);
    else if (!rope_cos) k_attn_av<2, false><<<grid, 256, 0, s>>>(a);
    else k_attn_av<2, true><<<grid, 256, 0, s>>>(a);
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
