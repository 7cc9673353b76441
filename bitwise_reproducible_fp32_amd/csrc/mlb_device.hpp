// Device-side arithmetic of the MLB-P1 profile: exp/log spellings, the
// sigmoid, and the 64-lane wavefront reduction trees.
//
// The pages fix the categories a frozen profile must pin - transcendental
// spellings, reduction order, FMA policy, tie rules (mojolearn PyPI page,
// "What bitwise identity means") - but print no concrete rule. The rules
// used here are this library's profile MLB-P1:
//  * exp: Cody-Waite reduction x = k ln2 + r with ln2 split into a 15-bit
//    head and a rounded tail, degree-7 Taylor polynomial (coefficients RN(1/n!))
//    in Horner form with fma, scale by 2^k from exponent bits (two multiplies
//    when 2^k is not normal). Inputs >= 0x42B17218 give +inf, inputs
//    <= 0xC2CFF1B5 give +0, NaN is returned unchanged.
//  * log: x = m 2^e with m in [sqrt(1/2), sqrt(2)], s = (m-1)/(2+(m-1)),
//    log m = 2s + 2s z P(z) with z = s^2 and P = 1/3 + z/5 + ... + z^4/11
//    (Horner, fma), log x = e LN2_HI + (e LN2_LO + log m). Subnormals are
//    pre-scaled by 2^23; 0 gives -inf, negatives give the quiet NaN.
//  * W64 reduction: element i goes to lane i mod 64 in ascending order, then
//    lane l absorbs lane l+s for s = 32..1; MAX keeps the earlier operand on
//    ties ((b > a) ? b : a).
// Every expression is a single IEEE binary32 operation per operator: the
// library is compiled with -ffp-contract=off and without fast-math, and the
// f32 denormal mode is IEEE (no flush).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlb {

__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }

__device__ __forceinline__ float exp_p(float x) {
    if (x != x) return x;
    if (x >= u2f(0x42B17218u)) return __builtin_inff();
    if (x <= u2f(0xC2CFF1B5u)) return 0.0f;
    const float shifter = 12582912.0f;                  // 1.5 * 2^23
    const float t = x * u2f(0x3FB8AA3Bu);               // x / ln2
    const float kf = (t + shifter) - shifter;           // round to nearest integer
    const int ki = (int)kf;
    float r = __builtin_fmaf(-kf, u2f(0x3F317200u), x);
    r = __builtin_fmaf(-kf, u2f(0x35BFBE8Eu), r);
    float p = u2f(0x39500D01u);                         // 1/7!
    p = __builtin_fmaf(p, r, u2f(0x3AB60B61u));         // 1/6!
    p = __builtin_fmaf(p, r, u2f(0x3C088889u));         // 1/5!
    p = __builtin_fmaf(p, r, u2f(0x3D2AAAABu));         // 1/4!
    p = __builtin_fmaf(p, r, u2f(0x3E2AAAABu));         // 1/3!
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    if (ki > 127) return (p * u2f(0x7F000000u)) * 2.0f;
    if (ki < -126) return (p * u2f((uint32_t)(ki + 253) << 23)) * u2f(0x00800000u);
    return p * u2f((uint32_t)(ki + 127) << 23);
}

__device__ __forceinline__ float log_p(float x) {
    if (x != x) return x;
    uint32_t u = f2u(x);
    if (u == 0x7F800000u) return x;
    if (x == 0.0f) return -__builtin_inff();
    if (u >> 31) return u2f(0x7FC00000u);
    int eadj = 0;
    if (u < 0x00800000u) { x = x * 8388608.0f; u = f2u(x); eadj = -23; }
    int e = (int)(u >> 23) - 127 + eadj;
    uint32_t mb = (u & 0x007FFFFFu) | 0x3F800000u;
    if (mb > 0x3FB504F3u) { mb -= 0x00800000u; e += 1; }
    const float m = u2f(mb);
    const float f = m - 1.0f;
    const float s = f / (2.0f + f);
    const float z = s * s;
    float P = u2f(0x3DBA2E8Cu);                         // 1/11
    P = __builtin_fmaf(P, z, u2f(0x3DE38E39u));         // 1/9
    P = __builtin_fmaf(P, z, u2f(0x3E124925u));         // 1/7
    P = __builtin_fmaf(P, z, u2f(0x3E4CCCCDu));         // 1/5
    P = __builtin_fmaf(P, z, u2f(0x3EAAAAABu));         // 1/3
    const float ts = s + s;
    const float corr = (ts * z) * P;
    const float lm = ts + corr;
    const float ef = (float)e;
    return (ef * u2f(0x3F317200u)) + ((ef * u2f(0x35BFBE8Eu)) + lm);
}

__device__ __forceinline__ float sigmoid_p(float x) { return 1.0f / (1.0f + exp_p(-x)); }

__device__ __forceinline__ float max_keep(float a, float b) { return (b > a) ? b : a; }

// Workgroups are dealt to the 8 XCDs (each with its own L2) round-robin by
// linear id. This maps the linear id of the whole grid (x fastest) to a
// logical index such that each XCD runs one contiguous range of logical work,
// so neighbouring tiles (and whole problems of a batch) share one L2. It is a
// bijection on [0, total) and never changes what a tile computes.
__device__ __forceinline__ int64_t xcd_logical_block() {
    const int64_t L = (int64_t)blockIdx.x + (int64_t)gridDim.x * ((int64_t)blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
    const int64_t total = (int64_t)gridDim.x * gridDim.y * gridDim.z;
    const int64_t xcd = L & 7, idx = L >> 3, base = total >> 3, rem = total & 7;
    return xcd * base + (xcd < rem ? xcd : rem) + idx;
}

// Lane tree of the W64 rule; the result is valid in lane 0 and returned to all lanes.
__device__ __forceinline__ float wave_tree_sum(float acc) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        const float o = __shfl_down(acc, (unsigned)s, 64);
        acc = acc + o;
    }
    return __shfl(acc, 0, 64);
}

__device__ __forceinline__ float wave_tree_max(float acc) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        const float o = __shfl_down(acc, (unsigned)s, 64);
        acc = max_keep(acc, o);
    }
    return __shfl(acc, 0, 64);
}

}  // namespace mlb
