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

}  // namespace

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
