// Row, elementwise and data-movement kernels of the training step.
//
// Each kernel follows one rule of the MLB-P1 profile (restated next to it);
// the reductions use the W64 lane assignment (element i to lane i mod 64,
// ascending, then the l <- l+s tree), which one wavefront realises directly.
// All of these kernels are bound by HBM bandwidth, so they read each input
// once or a few times with coalesced 64-lane accesses; none uses atomics on
// floating-point data.
#include <type_traits>

#include "mlb_device.hpp"
#include "mlb_internal.hpp"

namespace mlb {
namespace {

constexpr int64_t KC = 1024;

inline unsigned blocks(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

// Position of element j of row i in a [T, T] matrix, row-major or tiled
// (32x32 tiles of 4 KiB, see blk_index).
__device__ __forceinline__ int64_t pos(int blk, int64_t T, int64_t i, int64_t j) {
    return blk ? ((((i >> 5) * (T >> 5) + (j >> 5)) << 10) + ((i & 31) << 5) + (j & 31)) : i * T + j;
}

// Embedding lookup: an exact copy of table row ids[n]. An id outside [0, V)
// writes zeros and raises *err (no out-of-range read).
__global__ __launch_bounds__(256) void k_gather(const int32_t* __restrict__ ids, const float* __restrict__ tab,
                                                int64_t V, int64_t d, int64_t N, float* __restrict__ out,
                                                int* err) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= N * d) return;
    const int64_t n = idx / d, c = idx % d;
    const int32_t id = ids[n];
    if (id < 0 || id >= V) {
        out[idx] = 0.0f;
        if (c == 0) atomicOr(err, 1);
        return;
    }
    out[idx] = tab[(int64_t)id * d + c];
}

// RMSNorm forward, one wavefront per row:
// ss = DOT64(x, x); r = 1 / sqrt(ss / d + eps); y = (x * r) * w.
__global__ __launch_bounds__(256) void k_rmsnorm_fwd(const float* __restrict__ x, const float* __restrict__ w,
                                                     int64_t rows, int64_t d, float eps, float* __restrict__ y,
                                                     float* __restrict__ r) {
    const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const float* xr = x + row * d;
    float acc = 0.0f;
    for (int64_t c = lane; c < d; c += 64) acc = __builtin_fmaf(xr[c], xr[c], acc);
    const float ss = wave_tree_sum(acc);
    const float ms = ss / (float)d;
    const float rr = 1.0f / __builtin_sqrtf(ms + eps);
    if (lane == 0) r[row] = rr;
    float* yr = y + row * d;
    for (int64_t c = lane; c < d; c += 64) yr[c] = (xr[c] * rr) * w[c];
}

// RMSNorm backward (input gradient), one wavefront per row:
// xh = x * r; gw = dy * w; c = DOT64(gw, xh) / d; dx = r * (gw - xh * c).
__global__ __launch_bounds__(256) void k_rmsnorm_bwd_dx(const float* __restrict__ dy, const float* __restrict__ x,
                                                        const float* __restrict__ w, const float* __restrict__ r,
                                                        int64_t rows, int64_t d, const float* base, float* out) {
    const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const float rr = r[row];
    const float* xr = x + row * d;
    const float* dr = dy + row * d;
    float acc = 0.0f;
    for (int64_t c = lane; c < d; c += 64) {
        const float xh = xr[c] * rr;
        const float gw = dr[c] * w[c];
        acc = __builtin_fmaf(gw, xh, acc);
    }
    const float cc = wave_tree_sum(acc) / (float)d;
    float* o = out + row * d;
    const float* b = base ? base + row * d : nullptr;
    for (int64_t c = lane; c < d; c += 64) {
        const float xh = xr[c] * rr;
        const float gw = dr[c] * w[c];
        const float dx = rr * (gw - (xh * cc));
        o[c] = b ? b[c] + dx : dx;
    }
}

// Register-resident forms of the two row kernels above for rows of at most
// 64 E entries: each lane loads its E entries (c = lane + 64 e) at once,
// through range-checked buffer loads (entries past d read as 0, stores past d
// are dropped), instead of walking the row twice. Same expressions and chain
// order: forward, an entry past d adds fma(0, 0, acc) = acc (acc starts at +0
// and is never -0); backward, entries past d are left out by a select.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const float* p, int64_t d) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, (int)(d * 4), 0x00020000);
}
__device__ __forceinline__ float row_load(__amdgpu_buffer_rsrc_t rs, uint32_t c) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, c * 4u, 0, 0));
}
__device__ __forceinline__ void row_store(__amdgpu_buffer_rsrc_t rs, uint32_t c, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, c * 4u, 0, 0);
}

// In these row kernels the row is taken as uniform across the wave
// (readfirstlane): the row's buffer descriptors then sit in scalar registers,
// and no access needs a loop over distinct descriptors.
template <int E>
__global__ __launch_bounds__(256) void k_rmsnorm_fwd_reg(const float* __restrict__ x, const float* __restrict__ w,
                                                         int64_t rows, int64_t d, float eps, float* __restrict__ y,
                                                         float* __restrict__ r) {
    const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    if (row >= rows) return;
    const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + row * d, d), rw = row_rsrc(w, d), ry = row_rsrc(y + row * d, d);
    float v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = row_load(rx, lane + 64u * e);
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc = __builtin_fmaf(v[e], v[e], acc);
    const float ss = wave_tree_sum(acc);
    const float ms = ss / (float)d;
    const float rr = 1.0f / __builtin_sqrtf(ms + eps);
    if (lane == 0) r[row] = rr;
#pragma unroll
    for (int e = 0; e < E; ++e) row_store(ry, lane + 64u * e, (v[e] * rr) * row_load(rw, lane + 64u * e));
}

template <int E>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd_dx_reg(const float* __restrict__ dy, const float* __restrict__ x,
                                                            const float* __restrict__ w, const float* __restrict__ r,
                                                            int64_t rows, int64_t d, const float* base, float* out) {
    const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63;
    if (row >= rows) return;
    const float rr = r[row];
    const __amdgpu_buffer_rsrc_t rx = row_rsrc(x + row * d, d), rd = row_rsrc(dy + row * d, d), rw = row_rsrc(w, d);
    float xh[E], gw[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        xh[e] = row_load(rx, lane + 64u * e);
        gw[e] = row_load(rd, lane + 64u * e);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        xh[e] = xh[e] * rr;
        gw[e] = gw[e] * row_load(rw, lane + 64u * e);
    }
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc = (int64_t)(lane + 64u * e) < d ? __builtin_fmaf(gw[e], xh[e], acc) : acc;
    const float cc = wave_tree_sum(acc) / (float)d;
    const __amdgpu_buffer_rsrc_t ro = row_rsrc(out + row * d, d);
    if (base) {
        const __amdgpu_buffer_rsrc_t rb = row_rsrc(base + row * d, d);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float dx = rr * (gw[e] - (xh[e] * cc));
            row_store(ro, lane + 64u * e, row_load(rb, lane + 64u * e) + dx);
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) row_store(ro, lane + 64u * e, rr * (gw[e] - (xh[e] * cc)));
    }
}

// Per-chunk column partials of the gain gradient: for column c and chunk ch
// (rows [1024 ch, 1024 ch + 1024)), part[ch][c] is an fma chain from +0 over
// the chunk's rows in ascending order of dy[n][c] * (x[n][c] * r[n]). There
// are only d * chunks serial chains, so the loads, not the chains, set the
// time: a workgroup owns DW_CW columns of one chunk, and its sixteen waves
// stage DW_RB-row blocks of dy and x * r in LDS (two buffers) with the loads
// of the block after next already in flight (two register sets), while the
// first DW_CW lanes run the column chains through the staged block. The LDS
// blocks are column-major (one column's rows contiguous): a chain lane reads
// four rows of each operand with one 16-byte LDS read, and the chain over a
// full block is unrolled whole so that those reads run ahead of the fmas.
constexpr int DW_RB = 256;
constexpr int DW_CW = 32;      // columns (chains) per workgroup
constexpr int DW_THREADS = 1024;
template <int CW>
__global__ __launch_bounds__(DW_THREADS) void k_rmsnorm_dw_part(const float* __restrict__ dy,
                                                               const float* __restrict__ x,
                                                               const float* __restrict__ r, int64_t rows, int64_t d,
                                                               float* __restrict__ part) {
    constexpr int RS = DW_THREADS / CW;   // rows covered by one pass of the threads
    constexpr int PER = DW_RB / RS;       // values of each array per thread per block
    constexpr int RP = DW_RB + 4;         // row pitch of a column: 16-byte aligned, a 4-bank offset per column
    static_assert(PER % 4 == 0, "four consecutive rows per thread and array");
    __shared__ __align__(16) float sy[2][CW][RP];
    __shared__ __align__(16) float sx[2][CW][RP];
    const int tid = threadIdx.x, col = tid % CW, rsub = tid / CW;
    const int64_t c = (int64_t)blockIdx.x * CW + col;
    const bool live = c < d;
    const int64_t n0 = (int64_t)blockIdx.y * KC, n1 = (n0 + KC < rows) ? n0 + KC : rows;
    const int64_t nb = (n1 - n0 + DW_RB - 1) / DW_RB;
    // raw loads (x * r is formed at the LDS store, so that nothing waits for
    // a load before the block after next is issued); thread (col, rsub) holds
    // rows 4 RS h + 4 rsub + j, j < 4, of each block, and stores each four as
    // one 16-byte LDS write (eight lanes' writes cover the 32 banks)
    float ya[PER], xa[PER], ra[PER], yb[PER], xb[PER], rb[PER];
    // Unconditional loads from clamped positions (a guarded load became a
    // branch with a wait per row): rows past the chunk are never taken by
    // the chain and columns past d are never stored.
    const int64_t cc = live ? c : d - 1;
    auto load = [&](int64_t b, float (&vy)[PER], float (&vx)[PER], float (&vr)[PER]) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            int64_t n = n0 + b * DW_RB + 4 * RS * (q >> 2) + 4 * rsub + (q & 3);
            n = n < n1 ? n : n1 - 1;
            vy[q] = dy[n * d + cc];
            vx[q] = x[n * d + cc];
            vr[q] = r[n];
        }
    };
    auto store = [&](int buf, const float (&vy)[PER], const float (&vx)[PER], const float (&vr)[PER])
        __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < PER / 4; ++h) {
            const int o = 4 * RS * h + 4 * rsub;
            *reinterpret_cast<float4*>(&sy[buf][col][o]) =
                make_float4(vy[4 * h], vy[4 * h + 1], vy[4 * h + 2], vy[4 * h + 3]);
            *reinterpret_cast<float4*>(&sx[buf][col][o]) =
                make_float4(vx[4 * h] * vr[4 * h], vx[4 * h + 1] * vr[4 * h + 1], vx[4 * h + 2] * vr[4 * h + 2],
                            vx[4 * h + 3] * vr[4 * h + 3]);
        }
    };
    float acc = 0.0f;
    auto chain = [&](int64_t b) __attribute__((always_inline)) {
        if (tid < CW) {
            const int64_t len = (n1 - n0 - b * DW_RB) < DW_RB ? (n1 - n0 - b * DW_RB) : DW_RB;
            const int buf = (int)(b & 1);
            if (len == DW_RB) {
                const float4* y4 = reinterpret_cast<const float4*>(&sy[buf][col][0]);
                const float4* x4 = reinterpret_cast<const float4*>(&sx[buf][col][0]);
#pragma unroll
                for (int k = 0; k < DW_RB / 4; ++k) {
                    const float4 yv = y4[k], xv = x4[k];
                    acc = __builtin_fmaf(yv.x, xv.x, acc);
                    acc = __builtin_fmaf(yv.y, xv.y, acc);
                    acc = __builtin_fmaf(yv.z, xv.z, acc);
                    acc = __builtin_fmaf(yv.w, xv.w, acc);
                }
            } else {
                for (int k = 0; k < len; ++k) acc = __builtin_fmaf(sy[buf][col][k], sx[buf][col][k], acc);
            }
        }
    };
    // block b is staged in buffer b & 1; the registers alternate between
    // block b + 1 (set a for even b) and block b + 2 (the other set)
    // Loads past the last block re-read the last block (in bounds, never
    // chained): every iteration issues the same loads, so the hardware's
    // in-order load counter lets each store wait for its own set only.
    auto blk = [&](int64_t b) -> int64_t { return b < nb ? b : nb - 1; };
    load(0, ya, xa, ra);
    load(blk(1), yb, xb, rb);
    store(0, ya, xa, ra);
    __syncthreads();
    for (int64_t b = 0; b < nb; b += 2) {
        // even b: set a is free, set b holds block b + 1
        load(blk(b + 2), ya, xa, ra);
        chain(b);
        store(1, yb, xb, rb);
        __syncthreads();
        if (b + 1 >= nb) break;
        // odd b + 1: set b is free, set a holds block b + 2
        load(blk(b + 3), yb, xb, rb);
        chain(b + 1);
        store(0, ya, xa, ra);
        __syncthreads();
    }
    if (tid < CW && live) part[blockIdx.y * d + c] = acc;
}

// Left fold of per-chunk column partials, then dw = t (mode 0) or dw + t (mode 1).
__global__ __launch_bounds__(256) void k_fold_cols(const float* __restrict__ part, int64_t nch, int64_t d,
                                                   float* dw, int mode) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= d) return;
    float t = part[c];
    for (int64_t ch = 1; ch < nch; ++ch) t = t + part[ch * d + c];
    dw[c] = mode ? dw[c] + t : t;
}

// The folds of nprob gain gradients in one launch (problem p: partials at
// part + p * nch * d, output at base + offs[p]), each dw[c] = dw[c] + t with
// t the chunk partials added in chunk order, as k_fold_cols in mode 1.
__global__ __launch_bounds__(256) void k_fold_cols_batched(const float* __restrict__ part, int64_t nch, int64_t d,
                                                           const int64_t* __restrict__ offs, float* base) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= d) return;
    const float* pp = part + (int64_t)blockIdx.y * nch * d;
    float t = pp[c];
    for (int64_t ch = 1; ch < nch; ++ch) t = t + pp[ch * d + c];
    float* dw = base + offs[blockIdx.y];
    dw[c] = dw[c] + t;
}

// Rotary embedding, half-split pairing (element i with i + hd/2) at position
// t = n mod T, table values cos/sin[t][i].
__global__ __launch_bounds__(256) void k_rope(float* x, int64_t B, int64_t T, int64_t H, int64_t hd, int64_t ld,
                                              const float* __restrict__ cosv, const float* __restrict__ sinv,
                                              int backward) {
    const int64_t h2 = hd / 2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= B * T * H * h2) return;
    const int64_t i = idx % h2, h = (idx / h2) % H, n = idx / (h2 * H);
    const int64_t t = n % T;
    float* row = x + n * ld + h * hd;
    const float c = cosv[t * h2 + i], s = sinv[t * h2 + i];
    const float x0 = row[i], x1 = row[i + h2];
    if (!backward) {
        row[i] = (x0 * c) - (x1 * s);
        row[i + h2] = (x1 * c) + (x0 * s);
    } else {
        row[i] = (x0 * c) + (x1 * s);
        row[i + h2] = (x1 * c) - (x0 * s);
    }
}

// The same rotation on four adjacent pairs per thread (hd/2 % 4 == 0, 16-byte
// aligned rows and tables, fewer than 2^31 pairs in all and in a row's
// stride): float4 traffic and 32-bit index arithmetic, the same operations
// per element.
__global__ __launch_bounds__(256) void k_rope4(float* x, uint32_t npairs4, uint32_t T, uint32_t H, uint32_t hd,
                                               uint32_t ld, const float* __restrict__ cosv,
                                               const float* __restrict__ sinv, int backward) {
    const uint32_t q = blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= npairs4) return;
    const uint32_t h2 = hd / 2, idx = 4u * q;
    const uint32_t i = idx % h2, h = (idx / h2) % H, n = idx / (h2 * H);
    const uint32_t t = n % T;
    float* row = x + (size_t)n * ld + (size_t)h * hd;
    const float4 c4 = *reinterpret_cast<const float4*>(cosv + (size_t)t * h2 + i);
    const float4 s4 = *reinterpret_cast<const float4*>(sinv + (size_t)t * h2 + i);
    const float4 a4 = *reinterpret_cast<const float4*>(row + i);
    const float4 b4 = *reinterpret_cast<const float4*>(row + i + h2);
    const float cs[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
    const float x0[4] = {a4.x, a4.y, a4.z, a4.w}, x1[4] = {b4.x, b4.y, b4.z, b4.w};
    float r0[4], r1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (!backward) {
            r0[e] = (x0[e] * cs[e]) - (x1[e] * sn[e]);
            r1[e] = (x1[e] * cs[e]) + (x0[e] * sn[e]);
        } else {
            r0[e] = (x0[e] * cs[e]) + (x1[e] * sn[e]);
            r1[e] = (x1[e] * cs[e]) - (x0[e] * sn[e]);
        }
    }
    *reinterpret_cast<float4*>(row + i) = make_float4(r0[0], r0[1], r0[2], r0[3]);
    *reinterpret_cast<float4*>(row + i + h2) = make_float4(r1[0], r1[1], r1[2], r1[3]);
}

// exp_p without branches, bit for bit the same function: the reduction and
// polynomial run on 0 in place of a NaN or out-of-range input and the special
// result is selected at the end. Two steps use single instructions that give
// exactly the spelled values: the round-to-nearest-even of t (rndne; the
// spelling's (t + 1.5 * 2^23) - 1.5 * 2^23 rounds |t| < 2^22 to the nearest
// integer, ties to even, exactly) and the scaling p * 2^k (ldexp, one correct
// rounding; the spelling multiplies by two powers of two of which only the
// second can round). For code that evaluates many exponentials per thread,
// where the branches of exp_p would each hold an exec mask; every binary32
// input is checked against the oracle's exp.
__device__ __forceinline__ float exp_p_select(float x) {
    const bool nan = x != x, hi = x >= u2f(0x42B17218u), lo = x <= u2f(0xC2CFF1B5u);
    const float xs = (nan || hi || lo) ? 0.0f : x;
    const float t = xs * u2f(0x3FB8AA3Bu);
    const float kf = __builtin_rintf(t);
    const int ki = (int)kf;
    float r = __builtin_fmaf(-kf, u2f(0x3F317200u), xs);
    r = __builtin_fmaf(-kf, u2f(0x35BFBE8Eu), r);
    float p = u2f(0x39500D01u);
    p = __builtin_fmaf(p, r, u2f(0x3AB60B61u));
    p = __builtin_fmaf(p, r, u2f(0x3C088889u));
    p = __builtin_fmaf(p, r, u2f(0x3D2AAAABu));
    p = __builtin_fmaf(p, r, u2f(0x3E2AAAABu));
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const float v = __builtin_ldexpf(p, ki);
    return nan ? x : (hi ? __builtin_inff() : (lo ? 0.0f : v));
}

// Causal softmax in place, one wavefront per row i over j <= i:
// m = MAX64, e = exp(S - m), Z = SUM64(e), P = e * (1 / Z).
__global__ __launch_bounds__(256) void k_softmax(float* P, int64_t nbh, int64_t T, int blk) {
    const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= nbh * T) return;
    const int64_t i = row % T;
    float* p = P + (row / T) * T * T;
    const int64_t n = i + 1;
    float m = -__builtin_inff();
    for (int64_t j = lane; j < n; j += 64) m = max_keep(m, p[pos(blk, T, i, j)]);
    m = wave_tree_max(m);
    float acc = 0.0f;
    for (int64_t j = lane; j < n; j += 64) {
        const float e = exp_p(p[pos(blk, T, i, j)] - m);
        p[pos(blk, T, i, j)] = e;
        acc = acc + e;
    }
    const float Z = wave_tree_sum(acc);
    const float rz = 1.0f / Z;
    for (int64_t j = lane; j < n; j += 64) p[pos(blk, T, i, j)] = p[pos(blk, T, i, j)] * rz;
}

// The same rule with the row held in registers (lane l owns j = l + 64m,
// m < PER): one read and one write of the row instead of three and two.
// Element j = lane + 64 m of row i sits at base + m * stride inside the
// head's matrix (tiled: two 32-wide tiles further per m; T * T < 2^30).
template <int PER>
__global__ __launch_bounds__(256) void k_softmax_reg(float* P, int64_t nbh, int64_t T, int blk) {
    // the row is uniform across the wave: saying so keeps the row's pointer and
    // buffer descriptor in scalar registers
    const int64_t row = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= nbh * T) return;
    const int64_t i = row % T;
    float* p = P + (row / T) * T * T;
    const int64_t n = i + 1;
    // this lane's count of positions j = lane + 64 m inside the row
    int nvm = n > lane ? (int)((n - lane + 63) / 64) : 0;
    uint32_t base = (uint32_t)pos(blk, T, i, lane) * 4u;
    const uint32_t stride = (blk ? 2048u : 64u) * 4u;
    // buffer accesses over the head's matrix: element m at the lane's byte
    // offset plus m * stride (a scalar offset); positions past the row take an
    // offset beyond the buffer, which loads +0 and drops the store, so no lane
    // branches around a load or a store
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, (int)(T * T * 4), 0x00020000);
    auto vo = [&](int m) -> uint32_t { return m < nvm ? base : 0x80000000u; };
    // accesses past the row for every lane are not issued: the wave takes the
    // smallest multiple of PER / 4 of them that covers its row (a scalar branch)
    const int nw = (int)((n + 63) / 64);
    constexpr int Q = PER / 4;
    const int ng = (nw + Q - 1) / Q;   // 1 .. 4
    float v[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) v[m] = 0.0f;
    auto load_to = [&](auto cnt) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < decltype(cnt)::value; ++m)
            v[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, vo(m), (uint32_t)m * stride, 0));
    };
    if (ng <= 1) load_to(std::integral_constant<int, Q>{});
    else if (ng == 2) load_to(std::integral_constant<int, 2 * Q>{});
    else if (ng == 3) load_to(std::integral_constant<int, 3 * Q>{});
    else load_to(std::integral_constant<int, 4 * Q>{});
    float mx = -__builtin_inff();
#pragma unroll
    for (int m = 0; m < PER; ++m)
        if (m < nvm) mx = max_keep(mx, v[m]);
    mx = wave_tree_max(mx);
    float acc = 0.0f;
#pragma unroll
    for (int m = 0; m < PER; ++m)
        if (m < nvm) {
            v[m] = exp_p_select(v[m] - mx);
            acc = acc + v[m];
        }
    const float Z = wave_tree_sum(acc);
    const float rz = 1.0f / Z;
    // the offsets are formed again here rather than kept in PER registers
    asm volatile("" : "+v"(nvm), "+v"(base));
    auto store_to = [&](auto cnt) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < decltype(cnt)::value; ++m)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[m] * rz), rs, vo(m), (uint32_t)m * stride, 0);
    };
    if (ng <= 1) store_to(std::integral_constant<int, Q>{});
    else if (ng == 2) store_to(std::integral_constant<int, 2 * Q>{});
    else if (ng == 3) store_to(std::integral_constant<int, 3 * Q>{});
    else store_to(std::integral_constant<int, 4 * Q>{});
}

// D_i = DOT64 over the head dimension of dO and O. A wavefront takes
// ROWDOT_R consecutive rows (z, i) and, for heads of at most 64, loads all of
// them before the first chain, so that more loads are in flight per wave; each
// row is still its own lane chain and tree. ONE_HEAD (T a multiple of
// ROWDOT_R): a wave's rows are positions of one head, located by one division
// per wave; otherwise each row is located on its own.
constexpr int ROWDOT_R = 8;
template <bool ONE_HEAD>
__global__ __launch_bounds__(256) void k_rowdot(const float* __restrict__ dO, const float* __restrict__ O,
                                                int64_t B, int64_t H, int64_t T, int64_t hd, int64_t ld,
                                                float* __restrict__ D) {
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * ROWDOT_R;
    const int lane = threadIdx.x & 63;
    const int64_t nrows = B * H * T;
    if (row0 >= nrows) return;
    auto offset = [&](int64_t row) -> int64_t {
        const int64_t i = row % T, z = row / T;
        return ((z / H) * T + i) * ld + (z % H) * hd;
    };
    const int64_t off0 = offset(row0);
    auto off_of = [&](int k) -> int64_t { return ONE_HEAD ? off0 + k * ld : offset(row0 + k); };
    auto valid = [&](int k) -> bool { return ONE_HEAD || row0 + k < nrows; };
    if (hd <= 64) {
        float x[ROWDOT_R], y[ROWDOT_R];
        const bool in = lane < hd;
#pragma unroll
        for (int k = 0; k < ROWDOT_R; ++k) {
            const bool use = in && valid(k);
            const int64_t off = use ? off_of(k) + lane : 0;
            x[k] = use ? dO[off] : 0.0f;
            y[k] = use ? O[off] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < ROWDOT_R; ++k) {
            // a lane past hd holds no element: its chain stays +0 (fma(0, 0, +0) is +0)
            const float t = wave_tree_sum(__builtin_fmaf(x[k], y[k], 0.0f));
            if (lane == 0 && valid(k)) D[row0 + k] = t;
        }
        return;
    }
    for (int k = 0; k < ROWDOT_R && valid(k); ++k) {
        const int64_t off = off_of(k);
        float acc = 0.0f;
        for (int64_t c = lane; c < hd; c += 64) acc = __builtin_fmaf(dO[off + c], O[off + c], acc);
        const float t = wave_tree_sum(acc);
        if (lane == 0) D[row0 + k] = t;
    }
}

// dS = (P * (dP - D_i)) * scale over j <= i, written over dP.
__global__ __launch_bounds__(256) void k_softmax_bwd(const float* __restrict__ P, float* dP,
                                                     const float* __restrict__ D, int64_t T, float scale, int blk) {
    const int64_t i = blockIdx.x, z = blockIdx.y;
    const int64_t base = z * T * T;
    const float Di = D[z * T + i];
    for (int64_t j = threadIdx.x; j <= i; j += blockDim.x) {
        const int64_t o = base + pos(blk, T, i, j);
        dP[o] = (P[o] * (dP[o] - Di)) * scale;
    }
}

// SwiGLU: sig = 1 / (1 + exp(-g)); a = (g * sig) * u.
__global__ __launch_bounds__(256) void k_swiglu_fwd(const float* __restrict__ gu, int64_t rows, int64_t F,
                                                    float* __restrict__ a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * F) return;
    const int64_t n = idx / F, f = idx % F;
    const float g = gu[n * 2 * F + f], u = gu[n * 2 * F + F + f];
    const float sg = sigmoid_p(g);
    a[idx] = (g * sg) * u;
}

// du = dA * (g * sig); dsilu = sig * (1 + g * (1 - sig)); dg = (dA * u) * dsilu.
__global__ __launch_bounds__(256) void k_swiglu_bwd(const float* __restrict__ dA, const float* __restrict__ gu,
                                                    int64_t rows, int64_t F, float* __restrict__ dgu) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * F) return;
    const int64_t n = idx / F, f = idx % F;
    const float g = gu[n * 2 * F + f], u = gu[n * 2 * F + F + f];
    const float da = dA[idx];
    const float sg = sigmoid_p(g);
    const float silu = g * sg;
    const float dsilu = sg * (1.0f + (g * (1.0f - sg)));
    dgu[n * 2 * F + F + f] = da * silu;
    dgu[n * 2 * F + f] = (da * u) * dsilu;
}

// The same two kernels on four adjacent columns per thread (F % 4 == 0,
// 16-byte aligned rows, rows * F < 2^31): float4 traffic and 32-bit index
// arithmetic; every element takes exactly the operations above.
__global__ __launch_bounds__(256) void k_swiglu_fwd4(const float* __restrict__ gu, uint32_t n4, uint32_t F,
                                                     float* __restrict__ a) {
    const uint32_t q = blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= n4) return;
    const uint32_t idx = 4u * q, n = idx / F, f = idx % F;
    const float4 g = *reinterpret_cast<const float4*>(gu + (size_t)n * 2u * F + f);
    const float4 u = *reinterpret_cast<const float4*>(gu + (size_t)n * 2u * F + F + f);
    const float gs[4] = {g.x, g.y, g.z, g.w}, us[4] = {u.x, u.y, u.z, u.w};
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (gs[e] * sigmoid_p(gs[e])) * us[e];
    *reinterpret_cast<float4*>(a + idx) = make_float4(r[0], r[1], r[2], r[3]);
}

__global__ __launch_bounds__(256) void k_swiglu_bwd4(const float* __restrict__ dA, const float* __restrict__ gu,
                                                     uint32_t n4, uint32_t F, float* __restrict__ dgu) {
    const uint32_t q = blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= n4) return;
    const uint32_t idx = 4u * q, n = idx / F, f = idx % F;
    const size_t row = (size_t)n * 2u * F;
    const float4 g4 = *reinterpret_cast<const float4*>(gu + row + f);
    const float4 u4 = *reinterpret_cast<const float4*>(gu + row + F + f);
    const float4 d4 = *reinterpret_cast<const float4*>(dA + idx);
    const float gs[4] = {g4.x, g4.y, g4.z, g4.w}, us[4] = {u4.x, u4.y, u4.z, u4.w}, ds[4] = {d4.x, d4.y, d4.z, d4.w};
    float du[4], dg[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float sg = sigmoid_p(gs[e]);
        const float silu = gs[e] * sg;
        const float dsilu = sg * (1.0f + (gs[e] * (1.0f - sg)));
        du[e] = ds[e] * silu;
        dg[e] = (ds[e] * us[e]) * dsilu;
    }
    *reinterpret_cast<float4*>(dgu + row + F + f) = make_float4(du[0], du[1], du[2], du[3]);
    *reinterpret_cast<float4*>(dgu + row + f) = make_float4(dg[0], dg[1], dg[2], dg[3]);
}

// Cross-entropy, one wavefront per row: m = MAX64(l), Z = SUM64(exp(l - m)),
// loss = log(Z) - (l_y - m); dl = ((exp(l - m) * (1/Z)) - [v == y]) * invN
// (skipped when dl is null: inference keeps the logits).
// A target outside [0, V) raises *err and is read as 0 (no out-of-range read).
__global__ __launch_bounds__(256) void k_xent(const float* l_in, const int32_t* __restrict__ tg, int64_t N,
                                              int64_t V, int64_t ld, float invN, float* __restrict__ loss_rows,
                                              float* dl, int* err) {
    const int64_t n = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (n >= N) return;
    const float* l = l_in + n * ld;
    int64_t y = tg[n];
    if (y < 0 || y >= V) {
        if (lane == 0) atomicOr(err, 2);
        y = 0;
    }
    // Each lane walks v = lane, lane + 64, ... in ascending order (the W64
    // rule); U of its elements are loaded before any is used, so that U loads
    // per lane are in flight, and then taken in order.
    constexpr int U = 8;
    const int64_t vfull = lane + (V - lane) / (64 * U) * (64 * U);   // first v of the tail
    float m = -__builtin_inff();
    for (int64_t v = lane; v < vfull; v += 64 * U) {
        float x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = l[v + 64 * u];
#pragma unroll
        for (int u = 0; u < U; ++u) m = max_keep(m, x[u]);
    }
    for (int64_t v = vfull; v < V; v += 64) m = max_keep(m, l[v]);
    m = wave_tree_max(m);
    float acc = 0.0f;
    for (int64_t v = lane; v < vfull; v += 64 * U) {
        float x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = l[v + 64 * u];
#pragma unroll
        for (int u = 0; u < U; ++u) acc = acc + exp_p(x[u] - m);
    }
    for (int64_t v = vfull; v < V; v += 64) acc = acc + exp_p(l[v] - m);
    const float Z = wave_tree_sum(acc);
    const float ly = l[y];
    if (lane == 0) loss_rows[n] = log_p(Z) - (ly - m);
    if (!dl) return;
    const float rz = 1.0f / Z;
    float* o = dl + n * ld;   // may be the logits themselves: each element is read before it is written
    auto grad = [&](int64_t v, float x) -> float {
        const float p = exp_p(x - m) * rz;
        return ((v == y) ? (p - 1.0f) : p) * invN;
    };
    for (int64_t v = lane; v < vfull; v += 64 * U) {
        float x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = l[v + 64 * u];
#pragma unroll
        for (int u = 0; u < U; ++u) o[v + 64 * u] = grad(v + 64 * u, x[u]);
    }
    for (int64_t v = vfull; v < V; v += 64) o[v] = grad(v, l[v]);
}


// Cross-entropy of a long row read from HBM once: a workgroup of XR_W waves
// owns one row, and thread (w, lane) holds v = lane + 64 (w C + c), c < C,
// in registers, so the row is read once and dl written once (the three-pass
// kernel above reads it three times). The results are those of k_xent, bit
// for bit:
//  - m is the largest non-NaN entry. Any grouping gives that value; only the
//    sign of a zero maximum can differ, and no later result depends on it
//    (exp(x - m) and l_y - m give the same bits for m = +0 and m = -0).
//  - e = exp(l - m) is computed once per entry and kept.
//  - Z: each lane's chain adds its entries in ascending v from +0, wave 0's
//    share first, then wave 1's, and so on (the running sum passes through
//    LDS), then the same lane tree as k_xent. Positions past V hold +0, and
//    adding +0 leaves the chain's value unchanged (it starts at +0 and only
//    adds values >= +0 or NaN, so it is never -0).
constexpr int XR_W = 8;
template <int C>
__global__ __launch_bounds__(64 * XR_W) void k_xent_row(const float* l_in, const int32_t* __restrict__ tg, int64_t V,
                                                       int64_t ld, float invN, float* __restrict__ loss_rows,
                                                       float* dl, int* err) {
    __shared__ float wmax[XR_W];
    __shared__ float chain[64];
    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const float* l = l_in + n * ld;
    int64_t y = tg[n];
    if (y < 0 || y >= V) {
        if (tid == 0) atomicOr(err, 2);
        y = 0;
    }
    const uint32_t vb = (uint32_t)lane + 64u * (uint32_t)(w * C);
    // this lane's count of positions below V, and the c holding the target (or -1)
    const int64_t rem = V - (int64_t)vb;
    int nv = rem <= 0 ? 0 : (int)((rem + 63) / 64 < C ? (rem + 63) / 64 : C);
    const int64_t ty = y - (int64_t)vb;
    const int cy = (ty >= 0 && ty % 64 == 0 && ty / 64 < C) ? (int)(ty / 64) : -1;
    // every read of the row happens before the first barrier; dl may be the
    // logits themselves and is written only after the last one
    const float ly = l[y];
    // buffer accesses over the row's V entries: the hardware range check
    // returns 0 for a load past V and drops such a store, so no lane needs a
    // clamped address or a branch
    const __amdgpu_buffer_rsrc_t rin = __builtin_amdgcn_make_buffer_rsrc((void*)l, 0, (int)(V * 4), 0x00020000);
    float e[C];
#pragma unroll
    for (int c = 0; c < C; ++c)
        e[c] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rin, (vb + 64u * (uint32_t)c) * 4u, 0, 0));
    // every position of a full wave is below V: its lanes skip the position
    // tests (only the last wave of a row holds positions past V)
    const bool full = (int64_t)64 * C * (w + 1) <= V;
    if (!full) {
#pragma unroll
        for (int c = 0; c < C; ++c) e[c] = c < nv ? e[c] : -__builtin_inff();
    }
    // the position tests are made again below rather than kept as C lane masks
    asm volatile("" : "+v"(nv));
    float m = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < C; ++c) m = max_keep(m, e[c]);
    m = wave_tree_max(m);
    if (lane == 0) wmax[w] = m;
    __syncthreads();
    m = wmax[0];
#pragma unroll
    for (int k = 1; k < XR_W; ++k) m = max_keep(m, wmax[k]);
    if (full) {
#pragma unroll
        for (int c = 0; c < C; ++c) e[c] = exp_p_select(e[c] - m);
    } else {
#pragma unroll
        for (int c = 0; c < C; ++c) e[c] = exp_p_select(c < nv ? e[c] - m : -__builtin_inff());   // exp(-inf) = +0
    }
    for (int k = 0; k < XR_W; ++k) {
        if (w == k) {
            float acc = k == 0 ? 0.0f : chain[lane];
#pragma unroll
            for (int c = 0; c < C; ++c) acc = acc + e[c];
            chain[lane] = acc;
        }
        __syncthreads();
    }
    const float Z = wave_tree_sum(chain[lane]);
    if (tid == 0) loss_rows[n] = log_p(Z) - (ly - m);
    if (!dl) return;
    const float rz = 1.0f / Z;
    const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc((void*)(dl + n * ld), 0, (int)(V * 4), 0x00020000);
#pragma unroll
    for (int c = 0; c < C; ++c)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((e[c] * rz) * invN), rout, (vb + 64u * (uint32_t)c) * 4u,
                                              0, 0);
    // the target's entry, written again by the lane that holds it: its e is
    // exp_p(l_y - m), recomputed from the same l_y (the same bits as e[cy])
    if (cy >= 0)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(((exp_p_select(ly - m) * rz) - 1.0f) * invN), rout,
                                              (vb + 64u * (uint32_t)cy) * 4u, 0, 0);
}

// Greedy choice, one wavefront per selected row r (row index r * row_step +
// row_off of a [rows, ld] matrix): the index of the largest of the first V
// entries; NaN ranks below every number and ties go to the lowest index (a
// lane keeps its first maximum in ascending order, the lane tree prefers the
// lower index on equal values); 0 when every entry is NaN.
__global__ __launch_bounds__(256) void k_argmax_rows(const float* __restrict__ x, int64_t nsel, int64_t row_step,
                                                     int64_t row_off, int64_t ld, int64_t V, int32_t* out) {
    const int64_t r = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= nsel) return;
    const float* row = x + (r * row_step + row_off) * ld;
    float bv = -__builtin_inff();
    int64_t bi = V;
    for (int64_t v = lane; v < V; v += 64) {
        const float t = row[v];
        if (t > bv || (t == bv && v < bi)) { bv = t; bi = v; }
    }
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_down(bv, off);
        const int64_t oi = __shfl_down(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) out[r] = (int32_t)(bi < V ? bi : 0);
}

// out[0] = SUM64(v) * mul, one wavefront.
__global__ __launch_bounds__(64) void k_sum64(const float* __restrict__ v, int64_t n, float mul, float* out) {
    const int lane = threadIdx.x;
    float acc = 0.0f;
    // the lane's elements i = lane + 64 m in ascending m, 16 loads in flight
    // ahead of their additions
    constexpr int U = 16;
    for (int64_t i0 = lane; i0 < n; i0 += 64 * U) {
        float x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = i0 + 64 * u < n ? v[i0 + 64 * u] : 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + 64 * u < n) acc = acc + x[u];
    }
    const float t = wave_tree_sum(acc);
    if (lane == 0) out[0] = t * mul;
}

// Sort keys (id << 32 | n) in LDS, one workgroup per block of P positions
// (bitonic network; block b covers positions b*P .. b*P + P - 1, positions
// past N and ids outside [0, V) become ~0 and sort last). The keys are
// distinct, so each block's sorted order is unique: ids ascending, positions
// ascending within an id.
constexpr int SORT_MAX = 8192;   // 64 KiB of LDS keys
__global__ __launch_bounds__(1024) void k_sort_keys(const int32_t* __restrict__ ids, int64_t N, int64_t V,
                                                    int64_t P, uint64_t* __restrict__ out) {
    __shared__ uint64_t key[SORT_MAX];
    const int64_t base = (int64_t)blockIdx.x * P;
    for (int64_t q = threadIdx.x; q < P; q += blockDim.x) {
        uint64_t k = ~0ull;
        if (base + q < N) {
            const int32_t id = ids[base + q];
            if (id >= 0 && id < V) k = ((uint64_t)(uint32_t)id << 32) | (uint64_t)(base + q);
        }
        key[q] = k;
    }
    __syncthreads();
    // each thread takes whole compare-exchange pairs (q, q + stride): pair r
    // has q = r with a 0 bit inserted at the stride's position
    const int np = (int)P / 2;
    for (int size = 2; size <= (int)P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const int ls = __builtin_ctz((unsigned)stride);
            for (int r = (int)threadIdx.x; r < np; r += (int)blockDim.x) {
                const int q = ((r >> ls) << (ls + 1)) | (r & (stride - 1)), partner = q | stride;
                const bool up = (q & size) == 0;
                const uint64_t a = key[q], b = key[partner];
                if ((a > b) == up) { key[q] = b; key[partner] = a; }
            }
            __syncthreads();
        }
    }
    for (int64_t q = threadIdx.x; q < P; q += blockDim.x) out[base + q] = key[q];
}

// One pass of the merge sort above the LDS blocks: the sorted runs
// in[2rL .. 2rL + L) and in[2rL + L .. 2rL + 2L) become one sorted run of 2L.
// Each key goes to its rank: its index in its own run plus the count of keys
// of the other run below it (first run) or at most it (second run), so equal
// keys (only the ~0 fillers) keep the first run's ahead and every output slot
// is written exactly once. total is a multiple of 2L.
__global__ __launch_bounds__(256) void k_merge_runs(const uint64_t* __restrict__ in, uint64_t* __restrict__ out,
                                                    int64_t L, int64_t total) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= total) return;
    const int64_t base = g / (2 * L) * (2 * L), o = g - base;
    const bool first = o < L;
    const uint64_t x = in[g];
    const uint64_t* other = in + base + (first ? L : 0);
    int64_t lo = 0, hi = L;   // binary search for the count
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        const uint64_t y = other[mid];
        if (first ? y < x : y <= x) lo = mid + 1;
        else hi = mid;
    }
    out[base + (first ? o : o - L) + lo] = x;
}

// For each segment head q (first sorted key of an id): acc = init(v); for the
// segment's positions n in ascending order acc = acc + dh[n][c]; then write.
__global__ __launch_bounds__(256) void k_scatter_segments(const uint64_t* __restrict__ key, int64_t N,
                                                          const float* __restrict__ dh, int64_t d,
                                                          const float* src_init, float* dst, int mode) {
    const int64_t q = blockIdx.x;
    const int64_t c = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
    const uint64_t kq = key[q];
    if (kq == ~0ull || c >= d) return;
    const uint32_t v = (uint32_t)(kq >> 32);
    if (q > 0 && (uint32_t)(key[q - 1] >> 32) == v) return;    // not the head of its segment
    float acc = src_init ? src_init[(int64_t)v * d + c] : 0.0f;
    // the segment's terms in sorted order; keys and rows of the next U terms
    // are fetched before the first of them is added
    constexpr int U = 8;
    for (int64_t e0 = q; e0 < N; e0 += U) {
        // unconditional loads from clamped positions (a guarded load becomes a
        // branch and a wait); terms outside the segment are never added
        uint64_t ke[U];
#pragma unroll
        for (int u = 0; u < U; ++u) ke[u] = key[(e0 + u < N) ? e0 + u : N - 1];
        bool in[U];
        float t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            in[u] = e0 + u < N && ke[u] != ~0ull && (uint32_t)(ke[u] >> 32) == v;
            const int64_t n = in[u] ? (int64_t)(uint32_t)ke[u] : (int64_t)(uint32_t)kq;
            t[u] = dh[n * d + c];
        }
        bool more = true;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            more = more && in[u];   // keys are sorted: the segment ends at the first other key
            if (more) acc = acc + t[u];
        }
        if (!more) break;
    }
    float* o = dst + (int64_t)v * d + c;
    *o = mode ? *o + acc : acc;
}

// The same sort on 32-bit keys (id << 13 | n) when ids are below 2^19 - 1
// and positions below 8,192; invalid ids become 0xFFFFFFFF (never a valid
// key) and sort last. The keys are distinct, so the result is unique and
// equal to the 64-bit sort's order. Each of 1,024 threads holds 8 consecutive
// keys: compare-exchange stages with stride below 8 run in registers, strides
// 8 to 256 (partners in the same wavefront) through lane shuffles, and only
// strides of 512 and more go through LDS with barriers.
constexpr int SORT32_THREADS = 1024, SORT32_PER = 8;   // 8,192 slots
__global__ __launch_bounds__(SORT32_THREADS) void k_sort_keys32(const int32_t* __restrict__ ids, int64_t N, int64_t V,
                                                               uint32_t* __restrict__ out) {
    __shared__ uint32_t lds[SORT32_THREADS * SORT32_PER];
    const int t = threadIdx.x;
    uint32_t k[SORT32_PER];
#pragma unroll
    for (int r = 0; r < SORT32_PER; ++r) {
        const int q = SORT32_PER * t + r;
        uint32_t key = 0xFFFFFFFFu;
        if (q < N) {
            const int32_t id = ids[q];
            if (id >= 0 && id < V) key = ((uint32_t)id << 13) | (uint32_t)q;
        }
        k[r] = key;
    }
    // one compare-exchange of element i (value a) with its partner's value b
    auto keep = [](uint32_t a, uint32_t b, bool lower, bool up) -> uint32_t {
        const uint32_t lo = a < b ? a : b, hi = a < b ? b : a;
        return (lower == up) ? lo : hi;
    };
    // stages whose partner sits in this thread's registers: compile-time
    // strides, so the key array stays in registers
    auto reg_stage = [&](auto stride_c, int size) __attribute__((always_inline)) {
        constexpr int stride = decltype(stride_c)::value;
#pragma unroll
        for (int r = 0; r < SORT32_PER; ++r) {
            if ((r & stride) != 0) continue;
            const int i = SORT32_PER * t + r;
            const uint32_t a = k[r], b = k[r + stride];
            const bool up = (i & size) == 0;
            k[r] = keep(a, b, true, up);
            k[r + stride] = keep(b, a, false, up);
        }
    };
    for (int size = 2; size <= SORT32_THREADS * SORT32_PER; size <<= 1) {
        for (int stride = size >> 1; stride >= SORT32_PER; stride >>= 1) {
            if (stride >= 64 * SORT32_PER) {
                // partner in another wavefront: exchange through LDS
#pragma unroll
                for (int r = 0; r < SORT32_PER; ++r) lds[SORT32_PER * t + r] = k[r];
                __syncthreads();
#pragma unroll
                for (int r = 0; r < SORT32_PER; ++r) {
                    const int i = SORT32_PER * t + r;
                    k[r] = keep(k[r], lds[i ^ stride], (i & stride) == 0, (i & size) == 0);
                }
                __syncthreads();
            } else if (stride >= SORT32_PER) {
                // partner in another lane of this wavefront
                const int lx = stride / SORT32_PER;
#pragma unroll
                for (int r = 0; r < SORT32_PER; ++r) {
                    const int i = SORT32_PER * t + r;
                    const uint32_t b = (uint32_t)__shfl_xor((int)k[r], lx, 64);
                    k[r] = keep(k[r], b, (i & stride) == 0, (i & size) == 0);
                }
            }
        }
        if (size > 4) reg_stage(std::integral_constant<int, 4>{}, size);
        if (size > 2) reg_stage(std::integral_constant<int, 2>{}, size);
        reg_stage(std::integral_constant<int, 1>{}, size);
    }
#pragma unroll
    for (int r = 0; r < SORT32_PER; ++r) out[SORT32_PER * t + r] = k[r];
}

// For each segment head q of the 32-bit sorted keys (the first key of an id):
// acc = init(v); for the segment's positions n in ascending order
// acc = acc + dh[n][c]; then write. The segment's positions are staged in LDS
// first; the rows of two batches of SEG_U terms are in flight while the
// previous batch is added (loads past the segment repeat its last position
// and are never added).
constexpr int SEG_U = 32;
__global__ __launch_bounds__(256) void k_scatter_segments32(const uint32_t* __restrict__ key, int64_t N,
                                                            const float* __restrict__ dh, int64_t d,
                                                            const float* src_init, float* dst, int mode) {
    __shared__ uint32_t pos[SORT32_THREADS * SORT32_PER];
    const int64_t q = blockIdx.x;
    const uint32_t kq = key[q];
    if (kq == 0xFFFFFFFFu) return;
    const uint32_t v = kq >> 13;
    if (q > 0 && (key[q - 1] >> 13) == v) return;    // not the head of its segment
    const int tid = threadIdx.x, lane = tid & 63;
    // segment length: 64 keys per step, the first key of another id ends it
    int64_t len = 0;
    for (int64_t e0 = q;; e0 += 64) {
        const int64_t e = e0 + lane;
        const bool same = e < N && key[e] != 0xFFFFFFFFu && (key[e] >> 13) == v;
        const uint64_t m = __ballot(same);
        if (~m != 0) { len = e0 - q + (int64_t)__builtin_ctzll(~m); break; }
        if (e0 + 64 >= N) { len = N - q; break; }
    }
    for (int64_t e = tid; e < len; e += 256) pos[e] = key[q + e] & 0x1FFFu;
    __syncthreads();
    const int64_t c = (int64_t)blockIdx.y * 256 + tid;
    if (c >= d) return;
    float acc = src_init ? src_init[(int64_t)v * d + c] : 0.0f;
    float ba[SEG_U], bb[SEG_U];
    auto load = [&](int64_t e0, float (&b)[SEG_U]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < SEG_U; ++u) {
            const int64_t e = e0 + u < len ? e0 + u : len - 1;
            b[u] = dh[(int64_t)pos[e] * d + c];
        }
    };
    auto add = [&](int64_t e0, const float (&b)[SEG_U]) __attribute__((always_inline)) {
        if (e0 + SEG_U <= len) {
#pragma unroll
            for (int u = 0; u < SEG_U; ++u) acc = acc + b[u];
        } else {
            for (int u = 0; u < SEG_U && e0 + u < len; ++u) acc = acc + b[u];
        }
    };
    if (len <= SEG_U) {   // short segments (most of them): one batch, no padding loads
#pragma unroll
        for (int u = 0; u < SEG_U; ++u)
            if (u < len) ba[u] = dh[(int64_t)pos[u] * d + c];
        for (int u = 0; u < len; ++u) acc = acc + ba[u];
        float* o = dst + (int64_t)v * d + c;
        *o = mode ? *o + acc : acc;
        return;
    }
    load(0, ba);
    for (int64_t e0 = 0; e0 < len; e0 += 2 * SEG_U) {
        load(e0 + SEG_U, bb);
        add(e0, ba);
        if (e0 + SEG_U >= len) break;
        load(e0 + 2 * SEG_U, ba);
        add(e0 + SEG_U, bb);
    }
    float* o = dst + (int64_t)v * d + c;
    *o = mode ? *o + acc : acc;
}

__global__ __launch_bounds__(256) void k_add(float* out, const float* __restrict__ x, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = out[i] + x[i];
}

// AdamW, coupled form, one element per thread; the gradient accumulator is
// reset to +0 after use.
// m = b1*m + (1-b1)*g; v = b2*v + (1-b2)*(g*g); mh = m/bc1; vh = v/bc2;
// u = mh / (sqrt(vh) + eps); p = p - lr*(u + wd*p).
__global__ __launch_bounds__(256) void k_adamw(float* __restrict__ p, float* __restrict__ g, float* __restrict__ m,
                                               float* __restrict__ v, int64_t n, float lr, float b1, float b2,
                                               float eps, float wd, float bc1, float bc2) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float omb1 = 1.0f - b1, omb2 = 1.0f - b2;
    const float gi = g[i];
    const float mi = (b1 * m[i]) + (omb1 * gi);
    const float vi = (b2 * v[i]) + (omb2 * (gi * gi));
    const float mh = mi / bc1;
    const float vh = vi / bc2;
    const float u = mh / (__builtin_sqrtf(vh) + eps);
    const float pi = p[i];
    p[i] = pi - (lr * (u + (wd * pi)));
    m[i] = mi;
    v[i] = vi;
    g[i] = 0.0f;
}

__global__ __launch_bounds__(256) void k_unary(const float* __restrict__ x, float* __restrict__ y, int64_t n,
                                               int which) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const float v = x[i];
    y[i] = which == 0 ? exp_p(v) : (which == 1 ? log_p(v) : (which == 2 ? sigmoid_p(v) : exp_p_select(v)));
}

__global__ __launch_bounds__(256) void k_zero(float* x, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) x[i] = 0.0f;
}

typedef float v32f __attribute__((ext_vector_type(32)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

// One FP32 MFMA per wavefront on lane-held operands; D holds R values per lane.
template <int V>
__global__ __launch_bounds__(64) void k_mfma_probe(const float* A, const float* B, const float* Cin, float* D) {
    const int64_t t = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (V == 0) {
        v32f c;
        for (int r = 0; r < 32; ++r) c[r] = Cin[t * 32 + r];
        c = __builtin_amdgcn_mfma_f32_32x32x1f32(A[t], B[t], c, 0, 0, 0);
        for (int r = 0; r < 32; ++r) D[t * 32 + r] = c[r];
    } else if (V == 1) {
        v16f c;
        for (int r = 0; r < 16; ++r) c[r] = Cin[t * 16 + r];
        c = __builtin_amdgcn_mfma_f32_16x16x1f32(A[t], B[t], c, 0, 0, 0);
        for (int r = 0; r < 16; ++r) D[t * 16 + r] = c[r];
    } else if (V == 2) {
        v4f c;
        for (int r = 0; r < 4; ++r) c[r] = Cin[t * 4 + r];
        c = __builtin_amdgcn_mfma_f32_4x4x1f32(A[t], B[t], c, 0, 0, 0);
        for (int r = 0; r < 4; ++r) D[t * 4 + r] = c[r];
    } else if (V == 3) {
        v16f c;
        for (int r = 0; r < 16; ++r) c[r] = Cin[t * 16 + r];
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(A[t], B[t], c, 0, 0, 0);
        for (int r = 0; r < 16; ++r) D[t * 16 + r] = c[r];
    } else {
        v4f c;
        for (int r = 0; r < 4; ++r) c[r] = Cin[t * 4 + r];
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(A[t], B[t], c, 0, 0, 0);
        for (int r = 0; r < 4; ++r) D[t * 4 + r] = c[r];
    }
}

inline int ok() { return hipGetLastError() == hipSuccess ? 0 : -3; }

}  // namespace

int gather_rows(const int32_t* ids, const float* table, int64_t V, int64_t d, int64_t N, float* out, int* err,
                hipStream_t s) {
    if (N < 0 || d <= 0 || V <= 0) return -1;
    if (N == 0) return 0;
    k_gather<<<blocks(N * d, 256), 256, 0, s>>>(ids, table, V, d, N, out, err);
    return ok();
}

int rmsnorm_fwd(const float* x, const float* w, int64_t rows, int64_t d, float eps, float* y, float* r,
                hipStream_t s) {
    if (rows < 0 || d <= 0) return -1;
    if (rows == 0) return 0;
    const unsigned g = blocks(rows, 4);
    if (d <= 64 * 6) k_rmsnorm_fwd_reg<6><<<g, 256, 0, s>>>(x, w, rows, d, eps, y, r);
    else if (d <= 64 * 12) k_rmsnorm_fwd_reg<12><<<g, 256, 0, s>>>(x, w, rows, d, eps, y, r);
    else if (d <= 64 * 16) k_rmsnorm_fwd_reg<16><<<g, 256, 0, s>>>(x, w, rows, d, eps, y, r);
    else k_rmsnorm_fwd<<<g, 256, 0, s>>>(x, w, rows, d, eps, y, r);
    return ok();
}

int rmsnorm_bwd_dx(const float* dy, const float* x, const float* w, const float* r, int64_t rows, int64_t d,
                   const float* base, float* out, hipStream_t s) {
    if (rows < 0 || d <= 0) return -1;
    if (rows == 0) return 0;
    const unsigned g = blocks(rows, 4);
    if (d <= 64 * 6) k_rmsnorm_bwd_dx_reg<6><<<g, 256, 0, s>>>(dy, x, w, r, rows, d, base, out);
    else if (d <= 64 * 12) k_rmsnorm_bwd_dx_reg<12><<<g, 256, 0, s>>>(dy, x, w, r, rows, d, base, out);
    else if (d <= 64 * 16) k_rmsnorm_bwd_dx_reg<16><<<g, 256, 0, s>>>(dy, x, w, r, rows, d, base, out);
    else k_rmsnorm_bwd_dx<<<g, 256, 0, s>>>(dy, x, w, r, rows, d, base, out);
    return ok();
}

int rmsnorm_bwd_dw(const float* dy, const float* x, const float* r, int64_t rows, int64_t d, float* part,
                   float* dw, int mode, hipStream_t s) {
    if (rows < 0 || d <= 0) return -1;
    if (rows == 0) {
        if (mode == 0) k_zero<<<blocks(d, 256), 256, 0, s>>>(dw, d);
        return ok();
    }
    const int64_t nch = (rows + KC - 1) / KC;
    k_rmsnorm_dw_part<DW_CW><<<dim3(blocks(d, DW_CW), (unsigned)nch), DW_THREADS, 0, s>>>(dy, x, r, rows, d, part);
    k_fold_cols<<<blocks(d, 256), 256, 0, s>>>(part, nch, d, dw, mode);
    return ok();
}

int rmsnorm_bwd_dw_parts(const float* dy, const float* x, const float* r, int64_t rows, int64_t d, float* part,
                         hipStream_t s) {
    if (rows <= 0 || d <= 0) return -1;
    const int64_t nch = (rows + KC - 1) / KC;
    k_rmsnorm_dw_part<DW_CW><<<dim3(blocks(d, DW_CW), (unsigned)nch), DW_THREADS, 0, s>>>(dy, x, r, rows, d, part);
    return ok();
}

int fold_cols_batched(const float* part, int64_t rows, int64_t d, int64_t nprob, const int64_t* offs, float* base,
                      hipStream_t s) {
    if (rows <= 0 || d <= 0 || nprob <= 0 || nprob > 65535) return -1;
    const int64_t nch = (rows + KC - 1) / KC;
    k_fold_cols_batched<<<dim3(blocks(d, 256), (unsigned)nprob), 256, 0, s>>>(part, nch, d, offs, base);
    return ok();
}

int rope(float* x, int64_t B, int64_t T, int64_t H, int64_t hd, int64_t ld, const float* cosv,
         const float* sinv, int backward, hipStream_t s) {
    if (hd % 2 != 0 || B < 0 || T < 0 || H < 0) return -1;
    const int64_t n = B * T * H * (hd / 2);
    if (n == 0) return 0;
    const bool v4 = (hd / 2) % 4 == 0 && ld % 4 == 0 && hd % 4 == 0 && n < ((int64_t)1 << 31) &&
                    B * T * ld < ((int64_t)1 << 31) && ((uintptr_t)x & 15u) == 0 && ((uintptr_t)cosv & 15u) == 0 &&
                    ((uintptr_t)sinv & 15u) == 0;
    if (v4)
        k_rope4<<<blocks(n / 4, 256), 256, 0, s>>>(x, (uint32_t)(n / 4), (uint32_t)T, (uint32_t)H, (uint32_t)hd,
                                                    (uint32_t)ld, cosv, sinv, backward);
    else k_rope<<<blocks(n, 256), 256, 0, s>>>(x, B, T, H, hd, ld, cosv, sinv, backward);
    return ok();
}

int softmax_causal(float* P, int64_t nbh, int64_t T, int blk, hipStream_t s) {
    if (nbh < 0 || T < 0 || (blk && T % 32) || T * T >= ((int64_t)1 << 32)) return -1;
    if (nbh * T == 0) return 0;
    if (T <= 512) k_softmax_reg<8><<<blocks(nbh * T, 4), 256, 0, s>>>(P, nbh, T, blk);
    else if (T <= 2048) k_softmax_reg<32><<<blocks(nbh * T, 4), 256, 0, s>>>(P, nbh, T, blk);
    else k_softmax<<<blocks(nbh * T, 4), 256, 0, s>>>(P, nbh, T, blk);
    return ok();
}

int attn_rowdot(const float* dO, const float* O, int64_t B, int64_t H, int64_t T, int64_t hd, int64_t ld,
                float* D, hipStream_t s) {
    if (B * H * T == 0) return 0;
    if (T % ROWDOT_R == 0) k_rowdot<true><<<blocks(B * H * T, 4 * ROWDOT_R), 256, 0, s>>>(dO, O, B, H, T, hd, ld, D);
    else k_rowdot<false><<<blocks(B * H * T, 4 * ROWDOT_R), 256, 0, s>>>(dO, O, B, H, T, hd, ld, D);
    return ok();
}

int softmax_bwd(const float* P, float* dP, const float* D, int64_t nbh, int64_t T, float scale, int blk,
                hipStream_t s) {
    if (blk && T % 32) return -1;
    if (nbh * T == 0) return 0;
    k_softmax_bwd<<<dim3((unsigned)T, (unsigned)nbh), 256, 0, s>>>(P, dP, D, T, scale, blk);
    return ok();
}

// The float4 SwiGLU kernels: whole vectors of a row, 16-byte aligned, and
// 32-bit element indices (2 * rows * F < 2^31).
static bool vec4_ok(int64_t rows, int64_t F, const float* gu, const float* out) {
    return F % 4 == 0 && 2 * rows * F < ((int64_t)1 << 31) && ((uintptr_t)gu & 15u) == 0 && ((uintptr_t)out & 15u) == 0;
}

int swiglu_fwd(const float* gu, int64_t rows, int64_t F, float* a, hipStream_t s) {
    if (rows * F == 0) return 0;
    if (vec4_ok(rows, F, gu, a)) k_swiglu_fwd4<<<blocks(rows * F / 4, 256), 256, 0, s>>>(gu, (uint32_t)(rows * F / 4), (uint32_t)F, a);
    else k_swiglu_fwd<<<blocks(rows * F, 256), 256, 0, s>>>(gu, rows, F, a);
    return ok();
}

int swiglu_bwd(const float* dA, const float* gu, int64_t rows, int64_t F, float* dgu, hipStream_t s) {
    if (rows * F == 0) return 0;
    if (vec4_ok(rows, F, gu, dgu) && ((uintptr_t)dA & 15u) == 0)
        k_swiglu_bwd4<<<blocks(rows * F / 4, 256), 256, 0, s>>>(dA, gu, (uint32_t)(rows * F / 4), (uint32_t)F, dgu);
    else k_swiglu_bwd<<<blocks(rows * F, 256), 256, 0, s>>>(dA, gu, rows, F, dgu);
    return ok();
}

int cross_entropy(const float* logits, const int32_t* tg, int64_t N, int64_t V, int64_t ld, float* loss_rows,
                  float* dl, int* err, hipStream_t s) {
    if (N < 0 || V <= 0 || ld < V) return -1;
    if (N == 0) return 0;
    const float invN = 1.0f / (float)N;
    // rows of 25,345..50,688 entries (the 50,257-token vocabulary) are held in
    // registers by one workgroup each; other lengths take the three-pass kernel
    constexpr int XR_C = 99;
    if (V > 64 * XR_W * XR_C / 2 && V <= 64 * XR_W * XR_C && N < ((int64_t)1 << 31))
        k_xent_row<XR_C><<<(unsigned)N, 64 * XR_W, 0, s>>>(logits, tg, V, ld, invN, loss_rows, dl, err);
    else
        k_xent<<<blocks(N, 4), 256, 0, s>>>(logits, tg, N, V, ld, invN, loss_rows, dl, err);
    return ok();
}

int argmax_rows(const float* x, int64_t nsel, int64_t row_step, int64_t row_off, int64_t ld, int64_t V,
                int32_t* out, hipStream_t s) {
    if (nsel < 0 || V <= 0 || ld < V) return -1;
    if (nsel == 0) return 0;
    k_argmax_rows<<<blocks(nsel, 4), 256, 0, s>>>(x, nsel, row_step, row_off, ld, V, out);
    return ok();
}

int sum64_scaled(const float* v, int64_t n, float mul, float* out, hipStream_t s) {
    k_sum64<<<1, 64, 0, s>>>(v, n, mul, out);
    return ok();
}

static bool keys32(int64_t N, int64_t V) { return V < (1 << 19) - 1 && N <= SORT32_THREADS * SORT32_PER; }

static int64_t pow2_at_least(int64_t n) {
    int64_t p = 1;
    while (p < n) p <<= 1;
    return p;
}

int64_t embed_key_slots(int64_t N) { return N <= SORT_MAX ? SORT_MAX : 2 * pow2_at_least(N); }

int embed_sort(const int32_t* ids, int64_t N, int64_t V, uint64_t* keys, hipStream_t s) {
    if (N < 0 || V <= 0 || N > EMBED_MAX_POSITIONS) return -2;
    if (N == 0) return 0;
    if (keys32(N, V)) {
        k_sort_keys32<<<1, SORT32_THREADS, 0, s>>>(ids, N, V, reinterpret_cast<uint32_t*>(keys));
        return ok();
    }
    if (N <= SORT_MAX) {
        k_sort_keys<<<1, 1024, 0, s>>>(ids, N, V, pow2_at_least(N), keys);
        return ok();
    }
    // blocks of SORT_MAX sorted in LDS, then merge passes that double the run
    // length, alternating between the two halves of keys so that the last
    // pass writes the first half
    const int64_t P = pow2_at_least(N);
    int passes = 0;
    for (int64_t L = SORT_MAX; L < P; L <<= 1) ++passes;
    uint64_t* src = passes % 2 ? keys + P : keys;
    uint64_t* dst = passes % 2 ? keys : keys + P;
    k_sort_keys<<<(unsigned)(P / SORT_MAX), 1024, 0, s>>>(ids, N, V, SORT_MAX, src);
    for (int64_t L = SORT_MAX; L < P; L <<= 1) {
        k_merge_runs<<<(unsigned)(P / 256), 256, 0, s>>>(src, dst, L, P);
        uint64_t* t = src; src = dst; dst = t;
    }
    return ok();
}

int embed_scatter_sorted(const uint64_t* keys, const float* dh, int64_t N, int64_t d, int64_t V,
                         const float* src_init, float* dst, int mode, hipStream_t s) {
    if (N < 0 || d <= 0 || V <= 0 || N > EMBED_MAX_POSITIONS) return -2;
    if (N == 0) return 0;
    if (keys32(N, V))
        k_scatter_segments32<<<dim3((unsigned)N, blocks(d, 256)), 256, 0, s>>>(
            reinterpret_cast<const uint32_t*>(keys), N, dh, d, src_init, dst, mode);
    else
        k_scatter_segments<<<dim3((unsigned)N, blocks(d, 256)), 256, 0, s>>>(keys, N, dh, d, src_init, dst, mode);
    return ok();
}

int embed_scatter(const int32_t* ids, const float* dh, int64_t N, int64_t d, int64_t V, const float* src_init,
                  float* dst, int mode, uint64_t* keys, hipStream_t s) {
    if (N < 0 || d <= 0 || V <= 0 || N > EMBED_MAX_POSITIONS) return -2;
    const int r = embed_sort(ids, N, V, keys, s);
    return r ? r : embed_scatter_sorted(keys, dh, N, d, V, src_init, dst, mode, s);
}

int add_inplace(float* out, const float* x, int64_t n, hipStream_t s) {
    if (n <= 0) return n == 0 ? 0 : -1;
    k_add<<<blocks(n, 256), 256, 0, s>>>(out, x, n);
    return ok();
}

int adamw(float* p, float* g, float* m, float* v, int64_t n, float lr, float b1, float b2, float eps, float wd,
          float bc1, float bc2, hipStream_t s) {
    if (n <= 0) return n == 0 ? 0 : -1;
    k_adamw<<<blocks(n, 256), 256, 0, s>>>(p, g, m, v, n, lr, b1, b2, eps, wd, bc1, bc2);
    return ok();
}

int exp_array(const float* x, float* y, int64_t n, int which, hipStream_t s) {
    if (n <= 0 || which < 0 || which > 3) return n == 0 ? 0 : -1;
    k_unary<<<blocks(n, 256), 256, 0, s>>>(x, y, n, which);
    return ok();
}

int fill_zero(float* x, int64_t n, hipStream_t s) {
    if (n <= 0) return n == 0 ? 0 : -1;
    k_zero<<<blocks(n, 256), 256, 0, s>>>(x, n);
    return ok();
}

int mfma_probe(int variant, const float* A, const float* B, const float* C, float* D, int64_t nwaves,
               hipStream_t s) {
    if (nwaves <= 0) return -1;
    const dim3 g((unsigned)nwaves);
    switch (variant) {
        case 0: k_mfma_probe<0><<<g, 64, 0, s>>>(A, B, C, D); break;
        case 1: k_mfma_probe<1><<<g, 64, 0, s>>>(A, B, C, D); break;
        case 2: k_mfma_probe<2><<<g, 64, 0, s>>>(A, B, C, D); break;
        case 3: k_mfma_probe<3><<<g, 64, 0, s>>>(A, B, C, D); break;
        case 4: k_mfma_probe<4><<<g, 64, 0, s>>>(A, B, C, D); break;
        default: return -1;
    }
    return ok();
}

}  // namespace mlb
