// CPU oracle for the MLB-P1 bitwise FP32 training-step profile.
//
// TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
// CPU-baseline leg are the only callers. The product path never links it.
//
// What the oracle follows. The pages describe one training step of a
// Llama-style decoder (MojoLearn 162M model card, comparison table and
// "Training" table: pre-norm RMSNorm eps 1e-6 without a final norm, rotary
// positions with theta 10,000, SwiGLU, no biases, untied tables, AdamW with
// beta (0.9, 0.95), eps 1e-8, weight decay 0.1, shard gradients summed in a
// fixed order) trained under a frozen numerical profile (mojolearn PyPI page,
// "What bitwise identity means": reduction order, partitioning, FMA policy,
// flush seams, transcendental spellings and tie rules are all fixed). The
// pages print none of the concrete rules, so the profile below (MLB-P1) is
// the reading adopted here; every rule is restated where it is used.
//
// Arithmetic environment: IEEE binary32, round-to-nearest-even, gradual
// underflow (no FTZ/DAZ), no contraction (built with -ffp-contract=off), no
// libm in the step (exp/log are spelled out below), division and square root
// correctly rounded. Every expression below is one IEEE operation per
// operator, evaluated in the written parenthesisation.

#include "oracle.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#include <xmmintrin.h>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

int g_threads = 1;

// Sabotage arms (tests only): each breaks one rule of the profile so a test can
// show that the rule moves bits. 0 = the profile as written.
enum {
    SAB_NONE = 0, SAB_GEMM_REVERSE_K, SAB_GEMM_KC512, SAB_GEMM_PAIRWISE, SAB_GEMM_MULADD,
    SAB_W64_MIRROR, SAB_W32, SAB_LIBM_EXP, SAB_FTZ_DAZ, SAB_SOFTMAX_DIVIDE, SAB_ADAMW_DECOUPLED,
    SAB_SCATTER_REVERSE, SAB_LIBM_LOG, SAB_RMS_DW_UNCHUNKED, SAB_SWIGLU_BWD_SPELLING,
    SAB_DS_SPELLING, SAB_W64_BLOCKS, SAB_COUNT
};
int g_sab = SAB_NONE;

inline uint32_t fbits(float x) { uint32_t u; std::memcpy(&u, &x, 4); return u; }
inline float bitsf(uint32_t u) { float x; std::memcpy(&x, &u, 4); return x; }

constexpr int64_t KC = 1024;  // contraction chunk length (G1024)

// ---------------------------------------------------------------- exp / log
// exp_p: Cody & Waite range reduction x = k*ln2 + r with a two-part ln2,
// degree-7 Taylor polynomial in Horner form with fma, scaling by 2^k built
// from exponent bits (two steps when 2^k is not a normal number).
const float EXP_HI = bitsf(0x42B17218u);   // first input whose exp overflows binary32
const float EXP_LO = bitsf(0xC2CFF1B5u);   // inputs at or below give exp < 2^-150
const float L2E = bitsf(0x3FB8AA3Bu);      // RN(1/ln 2)
const float LN2_HI = bitsf(0x3F317200u);   // ln 2 cut to 15 significant bits
const float LN2_LO = bitsf(0x35BFBE8Eu);   // RN(ln 2 - LN2_HI)
const float SHIFTER = 12582912.0f;         // 1.5 * 2^23: adding it rounds to an integer
const float EC[8] = {bitsf(0x3F800000u), bitsf(0x3F800000u), bitsf(0x3F000000u),
                     bitsf(0x3E2AAAABu), bitsf(0x3D2AAAABu), bitsf(0x3C088889u),
                     bitsf(0x3AB60B61u), bitsf(0x39500D01u)};  // RN(1/n!)

float exp_p(float x) {
    if (g_sab == SAB_LIBM_EXP) return std::exp(x);
    if (x != x) return x;
    if (x >= EXP_HI) return INFINITY;
    if (x <= EXP_LO) return 0.0f;
    float t = x * L2E;
    float kf = (t + SHIFTER) - SHIFTER;
    int ki = (int)kf;
    float r = std::fma(-kf, LN2_HI, x);
    r = std::fma(-kf, LN2_LO, r);
    float p = EC[7];
    for (int n = 6; n >= 0; --n) p = std::fma(p, r, EC[n]);
    if (ki > 127) return (p * bitsf(0x7F000000u)) * 2.0f;
    if (ki < -126) return (p * bitsf((uint32_t)(ki + 253) << 23)) * bitsf(0x00800000u);
    return p * bitsf((uint32_t)(ki + 127) << 23);
}

// log_p: x = m * 2^e with m in [sqrt(1/2), sqrt(2)], f = m - 1, s = f/(2+f),
// log m = 2 atanh(s) = 2s + 2s z P(z) with z = s^2 and P the atanh series
// 1/3 + z/5 + z^2/7 + z^3/9 + z^4/11 in Horner form with fma; then
// log x = e*LN2_HI + (e*LN2_LO + log m).
const float LC[5] = {bitsf(0x3EAAAAABu), bitsf(0x3E4CCCCDu), bitsf(0x3E124925u),
                     bitsf(0x3DE38E39u), bitsf(0x3DBA2E8Cu)};  // RN(1/(2n+3))

float log_p(float x) {
    if (g_sab == SAB_LIBM_LOG) return std::log(x);
    if (x != x) return x;
    uint32_t u = fbits(x);
    if (u == 0x7F800000u) return x;
    if (x == 0.0f) return -INFINITY;
    if (u >> 31) return bitsf(0x7FC00000u);
    int eadj = 0;
    if (u < 0x00800000u) { x = x * 8388608.0f; u = fbits(x); eadj = -23; }
    int e = (int)(u >> 23) - 127 + eadj;
    uint32_t mb = (u & 0x007FFFFFu) | 0x3F800000u;
    if (mb > 0x3FB504F3u) { mb -= 0x00800000u; e += 1; }
    float mm = bitsf(mb);
    float f = mm - 1.0f;
    float s = f / (2.0f + f);
    float z = s * s;
    float P = LC[4];
    for (int n = 3; n >= 0; --n) P = std::fma(P, z, LC[n]);
    float ts = s + s;
    float corr = (ts * z) * P;
    float lm = ts + corr;
    float ef = (float)e;
    return (ef * LN2_HI) + ((ef * LN2_LO) + lm);
}

inline float sigmoid_p(float x) { return 1.0f / (1.0f + exp_p(-x)); }

// ------------------------------------------------------------ W64 reductions
// Element i goes to lane i mod 64 in ascending i; each lane accumulates in
// that order; then lanes are combined pairwise, lane l with lane l+s for
// s = 32, 16, 8, 4, 2, 1. The result is lane 0.
inline float max_keep(float a, float b) { return (b > a) ? b : a; }  // ties keep the earlier operand

inline int lanes() { return g_sab == SAB_W32 ? 32 : 64; }
template <class Op> float tree(float* acc, Op op) {
    for (int s = lanes() / 2; s >= 1; s >>= 1)
        for (int l = 0; l < s; ++l)
            acc[l] = (g_sab == SAB_W64_MIRROR) ? op(acc[l], acc[2 * s - 1 - l]) : op(acc[l], acc[l + s]);
    return acc[0];
}
inline float addf(float a, float b) { return a + b; }

// Lane of element i of n (the sabotage arm deals contiguous blocks instead).
inline int64_t lane_of(int64_t i, int64_t n, int W) {
    if (g_sab == SAB_W64_BLOCKS) { const int64_t blk = (n + W - 1) / W; return i / blk; }
    return i % W;
}

float sum64(const float* v, int64_t n) {
    float acc[64];
    const int W = lanes();
    for (int l = 0; l < 64; ++l) acc[l] = 0.0f;
    for (int64_t i = 0; i < n; ++i) { const int64_t l = lane_of(i, n, W); acc[l] = acc[l] + v[i]; }
    return tree(acc, addf);
}

float dot64(const float* a, const float* b, int64_t n) {
    float acc[64];
    const int W = lanes();
    for (int l = 0; l < 64; ++l) acc[l] = 0.0f;
    for (int64_t i = 0; i < n; ++i) { const int64_t l = lane_of(i, n, W); acc[l] = std::fma(a[i], b[i], acc[l]); }
    return tree(acc, addf);
}

float max64(const float* v, int64_t n) {
    float acc[64];
    const int W = lanes();
    for (int l = 0; l < 64; ++l) acc[l] = -INFINITY;
    for (int64_t i = 0; i < n; ++i) { const int64_t l = lane_of(i, n, W); acc[l] = max_keep(acc[l], v[i]); }
    return tree(acc, max_keep);
}

// ----------------------------------------------------------- G1024 contraction
struct Gemm {
    int64_t M, N, K, kseg;
    const float* A; int64_t sam, sak;
    const float* B; int64_t sbk, sbn;
    int mode; float scale; int krange; int outmask;
};

// Sabotage arms of the chain: descending k, or a rounded product then an add.
void chain_sabotaged(const Gemm& g, const float* Bt, int64_t i, int64_t lo, int64_t hi, float* acc) {
    for (int64_t kk = lo; kk < hi; ++kk) {
        const int64_t k = (g_sab == SAB_GEMM_REVERSE_K) ? (hi - 1 - (kk - lo)) : kk;
        const float a = g.A[i * g.sam + k * g.sak];
        const float* b = Bt + k * g.N;
        for (int64_t j = 0; j < g.N; ++j)
            acc[j] = (g_sab == SAB_GEMM_MULADD) ? acc[j] + (a * b[j]) : std::fma(a, b[j], acc[j]);
    }
}

// Computes output row i into C (length N) following the chunk rule.
// Bt is B laid out k-major: Bt[k*N + j] = B(k, j).
void gemm_row(const Gemm& g, const float* Bt, int64_t i, float* C, float* acc, float* tot) {
    int64_t klo = 0, khi = g.K;
    if (g.krange == 1) khi = std::min<int64_t>(g.K, i + 1);
    if (g.krange == 2) klo = std::max<int64_t>(0, i);
    bool have = false;
    const int64_t nseg = g.K / g.kseg;
    const int64_t kc = (g_sab == SAB_GEMM_KC512) ? 512 : KC;
    std::vector<std::vector<float>> parts;                   // sabotage arm only
    for (int64_t s = 0; s < nseg; ++s) {
        for (int64_t c0 = 0; c0 < g.kseg; c0 += kc) {
            int64_t a0 = s * g.kseg + c0;
            int64_t a1 = s * g.kseg + std::min<int64_t>(c0 + kc, g.kseg);
            int64_t lo = std::max(a0, klo), hi = std::min(a1, khi);
            if (lo >= hi) continue;                          // empty chunk: skipped
            for (int64_t j = 0; j < g.N; ++j) acc[j] = 0.0f;
            if (g_sab == SAB_GEMM_REVERSE_K || g_sab == SAB_GEMM_MULADD) {
                chain_sabotaged(g, Bt, i, lo, hi, acc);
            } else {
                for (int64_t k = lo; k < hi; ++k) {          // CHAIN: ascending k, fma from +0
                    const float a = g.A[i * g.sam + k * g.sak];
                    const float* b = Bt + k * g.N;
                    for (int64_t j = 0; j < g.N; ++j) acc[j] = std::fma(a, b[j], acc[j]);
                }
            }
            if (g_sab == SAB_GEMM_PAIRWISE) { parts.emplace_back(acc, acc + g.N); have = true; continue; }
            if (!have) { for (int64_t j = 0; j < g.N; ++j) tot[j] = acc[j]; have = true; }
            else { for (int64_t j = 0; j < g.N; ++j) tot[j] = tot[j] + acc[j]; }   // left fold
        }
    }
    if (g_sab == SAB_GEMM_PAIRWISE && !parts.empty()) {
        while (parts.size() > 1) {
            std::vector<std::vector<float>> nx;
            for (size_t q = 0; q + 1 < parts.size(); q += 2) {
                for (int64_t j = 0; j < g.N; ++j) parts[q][j] = parts[q][j] + parts[q + 1][j];
                nx.push_back(parts[q]);
            }
            if (parts.size() % 2) nx.push_back(parts.back());
            parts.swap(nx);
        }
        for (int64_t j = 0; j < g.N; ++j) tot[j] = parts[0][j];
    }
    if (!have) for (int64_t j = 0; j < g.N; ++j) tot[j] = 0.0f;
    const int64_t jend = g.outmask ? std::min<int64_t>(g.N, i + 1) : g.N;
    for (int64_t j = 0; j < jend; ++j) {
        if (g.mode == 0) C[j] = tot[j];
        else if (g.mode == 1) C[j] = C[j] + tot[j];
        else C[j] = tot[j] * g.scale;
    }
}

bool gemm_check(const Gemm& g) {
    if (g.M < 0 || g.N < 0 || g.K < 0) return false;
    if (g.K > 0 && (g.kseg <= 0 || g.K % g.kseg != 0)) return false;
    if (g.mode < 0 || g.mode > 2 || g.krange < 0 || g.krange > 2) return false;
    return true;
}

std::vector<float> make_bt(const Gemm& g) {
    std::vector<float> bt((size_t)std::max<int64_t>(1, g.K * g.N));
    for (int64_t k = 0; k < g.K; ++k)
        for (int64_t j = 0; j < g.N; ++j) bt[(size_t)(k * g.N + j)] = g.B[k * g.sbk + j * g.sbn];
    return bt;
}

void gemm_run(const Gemm& g, float* C, int64_t ldc) {
    std::vector<float> bt = make_bt(g);
    const float* Bt = bt.data();
#pragma omp parallel num_threads(g_threads)
    {
        std::vector<float> acc((size_t)std::max<int64_t>(1, g.N)), tot((size_t)std::max<int64_t>(1, g.N));
#pragma omp for schedule(static)
        for (int64_t i = 0; i < g.M; ++i) gemm_row(g, Bt, i, C + i * ldc, acc.data(), tot.data());
    }
}

// ------------------------------------------------------------------ RMSNorm
// y = (x * r) * w with r = 1 / sqrt(ss / d + eps), ss = DOT64(x, x).
void rmsnorm_fwd(const float* x, const float* w, int64_t rows, int64_t d, float eps, float* y, float* r) {
    const float df = (float)d;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t n = 0; n < rows; ++n) {
        const float* xr = x + n * d;
        float ss = dot64(xr, xr, d);
        float ms = ss / df;
        float rr = 1.0f / std::sqrt(ms + eps);
        r[n] = rr;
        for (int64_t c = 0; c < d; ++c) y[n * d + c] = (xr[c] * rr) * w[c];
    }
}

// xh = x * r, gw = dy * w, c = DOT64(gw, xh) / d, dx = r * (gw - xh * c);
// dw[c] = contraction over rows n of dy[n,c] * xh[n,c] (G1024 over n).
void rmsnorm_bwd(const float* dy, const float* x, const float* w, const float* r,
                 int64_t rows, int64_t d, float* dx, float* dw) {
    const float df = (float)d;
#pragma omp parallel num_threads(g_threads)
    {
        std::vector<float> xh((size_t)d), gw((size_t)d);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < rows; ++n) {
            const float rr = r[n];
            for (int64_t c = 0; c < d; ++c) { xh[c] = x[n * d + c] * rr; gw[c] = dy[n * d + c] * w[c]; }
            float cc = dot64(gw.data(), xh.data(), d) / df;
            for (int64_t c = 0; c < d; ++c) dx[n * d + c] = rr * (gw[c] - (xh[c] * cc));
        }
    }
    // gain gradient: per column, chunks of 1024 rows, fma chain from +0, left fold
    // (the sabotage arm runs one chain over all rows)
    std::vector<float> acc((size_t)d), tot((size_t)d);
    bool have = false;
    const int64_t kc = (g_sab == SAB_RMS_DW_UNCHUNKED) ? std::max<int64_t>(rows, 1) : KC;
    for (int64_t c0 = 0; c0 < rows; c0 += kc) {
        const int64_t c1 = std::min<int64_t>(rows, c0 + kc);
        for (int64_t c = 0; c < d; ++c) acc[c] = 0.0f;
        for (int64_t n = c0; n < c1; ++n) {
            const float rr = r[n];
            for (int64_t c = 0; c < d; ++c) acc[c] = std::fma(dy[n * d + c], x[n * d + c] * rr, acc[c]);
        }
        if (!have) { for (int64_t c = 0; c < d; ++c) tot[c] = acc[c]; have = true; }
        else { for (int64_t c = 0; c < d; ++c) tot[c] = tot[c] + acc[c]; }
    }
    for (int64_t c = 0; c < d; ++c) dw[c] = have ? tot[c] : 0.0f;
}

// --------------------------------------------------------------------- RoPE
// Half-split pairing: element i is rotated with element i + hd/2 by the
// angle t * theta^(-2i/hd); the table is computed in binary64 and rounded.
void rope_table(int64_t T, int64_t hd, float theta, float* cosv, float* sinv) {
    const int64_t h2 = hd / 2;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t i = 0; i < h2; ++i) {
            double ex = -(2.0 * (double)i) / (double)hd;
            double inv = std::pow((double)theta, ex);
            double ang = (double)t * inv;
            cosv[t * h2 + i] = (float)std::cos(ang);
            sinv[t * h2 + i] = (float)std::sin(ang);
        }
}

void rope_apply(float* x, int64_t B, int64_t T, int64_t H, int64_t hd, int64_t ld,
                const float* cosv, const float* sinv, bool backward) {
    const int64_t h2 = hd / 2;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t n = 0; n < B * T; ++n) {
        const int64_t t = n % T;
        for (int64_t h = 0; h < H; ++h) {
            float* row = x + n * ld + h * hd;
            for (int64_t i = 0; i < h2; ++i) {
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
        }
    }
}

// ---------------------------------------------------------------- attention
// S[i][j] = CHAIN_c(q_i, k_j) * scale for j <= i; m = MAX64, e = exp(S - m),
// Z = SUM64(e), P = e * (1 / Z); O = G1024 over j <= i of P[i][j] v[j].
float attn_scale(int64_t hd) { return (float)(1.0 / std::sqrt((double)hd)); }

void attention_fwd(int64_t B, int64_t H, int64_t T, int64_t hd, const float* q, const float* k,
                   const float* v, int64_t ld, float* P, float* O, int64_t ldo) {
    const float scale = attn_scale(hd);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h) {
            const int64_t off = b * T * ld + h * hd;
            float* Pb = P + (b * H + h) * T * T;
            Gemm gs{T, T, hd, hd, q + off, ld, 1, k + off, 1, ld, 2, scale, 0, 1};
            gemm_run(gs, Pb, T);
#pragma omp parallel num_threads(g_threads)
            {
                std::vector<float> e((size_t)T);
#pragma omp for schedule(static)
                for (int64_t i = 0; i < T; ++i) {
                    float* row = Pb + i * T;
                    const int64_t n = i + 1;
                    float m = max64(row, n);
                    for (int64_t j = 0; j < n; ++j) e[j] = exp_p(row[j] - m);
                    float Z = sum64(e.data(), n);
                    float rz = 1.0f / Z;
                    for (int64_t j = 0; j < n; ++j)
                        row[j] = (g_sab == SAB_SOFTMAX_DIVIDE) ? e[j] / Z : e[j] * rz;
                }
            }
            Gemm gpv{T, hd, T, T, Pb, T, 1, v + off, ld, 1, 0, 1.0f, 1, 0};
            gemm_run(gpv, O + b * T * ldo + h * hd, ldo);
        }
}

// D_i = DOT64(dO_i, O_i); dP = CHAIN(dO_i, v_j) for j <= i;
// dS = (P * (dP - D_i)) * scale; dq = G1024_{j<=i} dS v->k; dk = G1024_{i>=j} dS^T q;
// dv = G1024_{i>=j} P^T dO.
void attention_bwd(int64_t B, int64_t H, int64_t T, int64_t hd, const float* q, const float* k,
                   const float* v, int64_t ld, const float* P, const float* O, const float* dO,
                   int64_t ldo, float* dq, float* dk, float* dv) {
    const float scale = attn_scale(hd);
    std::vector<float> dS((size_t)(T * T));
    std::vector<float> D((size_t)T);
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h) {
            const int64_t off = b * T * ld + h * hd;
            const int64_t offo = b * T * ldo + h * hd;
            const float* Pb = P + (b * H + h) * T * T;
            for (int64_t i = 0; i < T; ++i) D[i] = dot64(dO + offo + i * ldo, O + offo + i * ldo, hd);
            Gemm gdp{T, T, hd, hd, dO + offo, ldo, 1, v + off, 1, ld, 0, 1.0f, 0, 1};
            gemm_run(gdp, dS.data(), T);
#pragma omp parallel for num_threads(g_threads) schedule(static)
            for (int64_t i = 0; i < T; ++i)
                for (int64_t j = 0; j <= i; ++j)
                    dS[i * T + j] = (g_sab == SAB_DS_SPELLING)
                                        ? ((Pb[i * T + j] * dS[i * T + j]) - (Pb[i * T + j] * D[i])) * scale
                                        : (Pb[i * T + j] * (dS[i * T + j] - D[i])) * scale;
            Gemm gq{T, hd, T, T, dS.data(), T, 1, k + off, ld, 1, 0, 1.0f, 1, 0};
            gemm_run(gq, dq + off, ld);
            Gemm gk{T, hd, T, T, dS.data(), 1, T, q + off, ld, 1, 0, 1.0f, 2, 0};
            gemm_run(gk, dk + off, ld);
            Gemm gv{T, hd, T, T, Pb, 1, T, dO + offo, ldo, 1, 0, 1.0f, 2, 0};
            gemm_run(gv, dv + off, ld);
        }
}

// ------------------------------------------------------------------- SwiGLU
// sig = 1/(1 + exp(-g)); a = (g * sig) * u.
// Backward: du = dA * (g * sig); dsilu = sig * (1 + g * (1 - sig)); dg = (dA * u) * dsilu.
void swiglu_fwd(const float* gu, int64_t rows, int64_t F, int64_t ldgu, float* a, int64_t lda) {
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t n = 0; n < rows; ++n)
        for (int64_t f = 0; f < F; ++f) {
            const float g = gu[n * ldgu + f], u = gu[n * ldgu + F + f];
            const float sg = sigmoid_p(g);
            a[n * lda + f] = (g * sg) * u;
        }
}

void swiglu_bwd(const float* dA, int64_t ldda, const float* gu, int64_t rows, int64_t F, int64_t ldgu, float* dgu) {
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t n = 0; n < rows; ++n)
        for (int64_t f = 0; f < F; ++f) {
            const float g = gu[n * ldgu + f], u = gu[n * ldgu + F + f];
            const float da = dA[n * ldda + f];
            const float sg = sigmoid_p(g);
            const float silu = g * sg;
            const float dsilu = (g_sab == SAB_SWIGLU_BWD_SPELLING) ? sg + (silu * (1.0f - sg))
                                                                   : sg * (1.0f + (g * (1.0f - sg)));
            dgu[n * ldgu + F + f] = da * silu;
            dgu[n * ldgu + f] = (da * u) * dsilu;
        }
}

// ------------------------------------------------------------- cross-entropy
// Per row: m = MAX64(l), Z = SUM64(exp(l - m)), loss = log(Z) - (l_y - m);
// dl = ((exp(l - m) * (1/Z)) - [v == y]) * (1/N). Shard loss = SUM64(loss) * (1/N).
float cross_entropy(const float* logits, const int32_t* tg, int64_t N, int64_t V, float* loss_rows, float* dl) {
    const float invN = 1.0f / (float)N;
#pragma omp parallel num_threads(g_threads)
    {
        std::vector<float> e((size_t)V);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            const float* l = logits + n * V;
            const int64_t y = tg[n];
            float m = max64(l, V);
            for (int64_t v = 0; v < V; ++v) e[v] = exp_p(l[v] - m);
            float Z = sum64(e.data(), V);
            float lz = log_p(Z);
            loss_rows[n] = lz - (l[y] - m);
            float rz = 1.0f / Z;
            float* o = dl + n * V;
            for (int64_t v = 0; v < V; ++v) {
                float p = (g_sab == SAB_SOFTMAX_DIVIDE) ? e[v] / Z : e[v] * rz;
                float t = (v == y) ? (p - 1.0f) : p;
                o[v] = t * invN;
            }
        }
    }
    return sum64(loss_rows, N) * invN;
}

// ---------------------------------------------------------- embedding scatter
// SEQ: for n ascending, dE[ids[n]] = dE[ids[n]] + dh[n] column by column.
void embed_scatter(const int32_t* ids, const float* dh, int64_t N, int64_t d, float* dE) {
    for (int64_t nn = 0; nn < N; ++nn) {
        const int64_t n = (g_sab == SAB_SCATTER_REVERSE) ? N - 1 - nn : nn;
        float* row = dE + (int64_t)ids[n] * d;
        for (int64_t c = 0; c < d; ++c) row[c] = row[c] + dh[n * d + c];
    }
}

// -------------------------------------------------------------------- AdamW
// bc_t = RN(1 - beta^t) with beta^t a binary64 product of the binary32 beta.
float bias_correction(float beta, int64_t t) {
    double b = 1.0;
    for (int64_t i = 0; i < t; ++i) b *= (double)beta;
    return (float)(1.0 - b);
}

// m = b1*m + (1-b1)*g; v = b2*v + (1-b2)*(g*g); mh = m/bc1; vh = v/bc2;
// u = mh / (sqrt(vh) + eps); p = p - lr*(u + wd*p). 1-b is formed in binary32.
void adamw(float* p, const float* g, float* m, float* v, int64_t n, float lr, float b1, float b2,
           float eps, float wd, float bc1, float bc2) {
    const float omb1 = 1.0f - b1, omb2 = 1.0f - b2;
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const float gi = g[i];
        const float mi = (b1 * m[i]) + (omb1 * gi);
        const float vi = (b2 * v[i]) + (omb2 * (gi * gi));
        const float mh = mi / bc1;
        const float vh = vi / bc2;
        const float u = mh / (std::sqrt(vh) + eps);
        if (g_sab == SAB_ADAMW_DECOUPLED) p[i] = (p[i] * (1.0f - (lr * wd))) - (lr * u);
        else p[i] = p[i] - (lr * (u + (wd * p[i])));
        m[i] = mi;
        v[i] = vi;
    }
}

// ------------------------------------------------------------------ SHA-256
// FIPS 180-4.
struct Sha256 {
    uint32_t h[8];
    uint8_t buf[64];
    uint64_t len = 0;
    size_t fill = 0;
    static uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }
    Sha256() {
        const uint32_t iv[8] = {0x6a09e667, 0xbb67ae85, 0x3c6ef372, 0xa54ff53a,
                                0x510e527f, 0x9b05688c, 0x1f83d9ab, 0x5be0cd19};
        std::memcpy(h, iv, sizeof iv);
    }
    void block(const uint8_t* p) {
        static const uint32_t K[64] = {
            0x428a2f98, 0x71374491, 0xb5c0fbcf, 0xe9b5dba5, 0x3956c25b, 0x59f111f1, 0x923f82a4, 0xab1c5ed5,
            0xd807aa98, 0x12835b01, 0x243185be, 0x550c7dc3, 0x72be5d74, 0x80deb1fe, 0x9bdc06a7, 0xc19bf174,
            0xe49b69c1, 0xefbe4786, 0x0fc19dc6, 0x240ca1cc, 0x2de92c6f, 0x4a7484aa, 0x5cb0a9dc, 0x76f988da,
            0x983e5152, 0xa831c66d, 0xb00327c8, 0xbf597fc7, 0xc6e00bf3, 0xd5a79147, 0x06ca6351, 0x14292967,
            0x27b70a85, 0x2e1b2138, 0x4d2c6dfc, 0x53380d13, 0x650a7354, 0x766a0abb, 0x81c2c92e, 0x92722c85,
            0xa2bfe8a1, 0xa81a664b, 0xc24b8b70, 0xc76c51a3, 0xd192e819, 0xd6990624, 0xf40e3585, 0x106aa070,
            0x19a4c116, 0x1e376c08, 0x2748774c, 0x34b0bcb5, 0x391c0cb3, 0x4ed8aa4a, 0x5b9cca4f, 0x682e6ff3,
            0x748f82ee, 0x78a5636f, 0x84c87814, 0x8cc70208, 0x90befffa, 0xa4506ceb, 0xbef9a3f7, 0xc67178f2};
        uint32_t w[64];
        for (int i = 0; i < 16; ++i)
            w[i] = (uint32_t)p[4 * i] << 24 | (uint32_t)p[4 * i + 1] << 16 | (uint32_t)p[4 * i + 2] << 8 | p[4 * i + 3];
        for (int i = 16; i < 64; ++i) {
            uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
            uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
            w[i] = w[i - 16] + s0 + w[i - 7] + s1;
        }
        uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
        for (int i = 0; i < 64; ++i) {
            uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
            uint32_t ch = (e & f) ^ (~e & g);
            uint32_t t1 = hh + S1 + ch + K[i] + w[i];
            uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
            uint32_t mj = (a & b) ^ (a & c) ^ (b & c);
            uint32_t t2 = S0 + mj;
            hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
        }
        h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
    }
    void update(const uint8_t* p, size_t n) {
        len += n;
        while (n > 0) {
            size_t take = std::min<size_t>(64 - fill, n);
            std::memcpy(buf + fill, p, take);
            fill += take; p += take; n -= take;
            if (fill == 64) { block(buf); fill = 0; }
        }
    }
    void final(uint8_t out[32]) {
        uint64_t bits = len * 8;
        uint8_t pad = 0x80;
        update(&pad, 1);
        uint8_t z = 0;
        while (fill != 56) update(&z, 1);
        uint8_t lb[8];
        for (int i = 0; i < 8; ++i) lb[i] = (uint8_t)(bits >> (56 - 8 * i));
        update(lb, 8);
        for (int i = 0; i < 8; ++i) {
            out[4 * i] = (uint8_t)(h[i] >> 24); out[4 * i + 1] = (uint8_t)(h[i] >> 16);
            out[4 * i + 2] = (uint8_t)(h[i] >> 8); out[4 * i + 3] = (uint8_t)h[i];
        }
    }
};

void sha256(const uint8_t* data, size_t len, uint8_t out[32]) {
    Sha256 s;
    s.update(data, len);
    s.final(out);
}

// -------------------------------------------------------------------- model
// Canonical parameter order: E_in [V,d]; per layer: attn_norm_w [d], Wq, Wk, Wv
// [d,d], Wo [d,d], mlp_norm_w [d], Wg [F,d], Wu [F,d], Wd [d,F]; W_out [V,d]
// when untied. Linear weights are [out_features, in_features].
struct Layout {
    int64_t E, W_out, nparams;
    std::vector<int64_t> w1, wqkv, wo, w2, wgu, wd;
};

Layout make_layout(const orc_cfg& c) {
    Layout L;
    const int64_t V = c.vocab, d = c.d_model, F = c.ffn_hidden;
    int64_t o = 0;
    L.E = o; o += V * d;
    for (int l = 0; l < c.n_layers; ++l) {
        L.w1.push_back(o); o += d;
        L.wqkv.push_back(o); o += 3 * d * d;
        L.wo.push_back(o); o += d * d;
        L.w2.push_back(o); o += d;
        L.wgu.push_back(o); o += 2 * F * d;
        L.wd.push_back(o); o += d * F;
    }
    if (c.tied) L.W_out = L.E;
    else { L.W_out = o; o += V * d; }
    L.nparams = o;
    return L;
}

bool cfg_ok(const orc_cfg& c) {
    if (c.vocab <= 0 || c.d_model <= 0 || c.n_layers <= 0 || c.n_heads <= 0 || c.head_dim <= 0) return false;
    if (c.ffn_hidden <= 0 || c.batch <= 0 || c.seq_len <= 0) return false;
    if ((int64_t)c.n_heads * c.head_dim != c.d_model || c.head_dim % 2 != 0) return false;
    return true;
}

struct Model {
    orc_cfg c;
    Layout L;
    int64_t N;
    std::vector<float> p, G, m, v, g;
    int64_t step = 0;
    bool have_fwd = false;
    int n_accum = 0;
    std::vector<float> cosv, sinv;
    std::vector<int32_t> ids, tg;
    // activations of the last forward
    std::vector<std::vector<float>> h_in, xn1, r1, qkv, P, O, h_mid, xn2, r2, gu, a;
    std::vector<float> h_L, logits, loss_rows;
    float loss = 0.0f;
};

// keep_logits: inference; the logits stay in M.logits and the loss (when
// targets are given) is computed into a separate d-logits buffer.
void model_forward(Model& M, bool keep_logits = false, bool with_loss = true) {
    const orc_cfg& c = M.c;
    const int64_t N = M.N, d = c.d_model, F = c.ffn_hidden, V = c.vocab, H = c.n_heads, hd = c.head_dim;
    const int64_t B = c.batch, T = c.seq_len;
    std::vector<float> h((size_t)(N * d));
    for (int64_t n = 0; n < N; ++n)                                         // embedding lookup
        std::memcpy(&h[(size_t)(n * d)], &M.p[(size_t)(M.L.E + (int64_t)M.ids[n] * d)], (size_t)d * 4);
    for (int l = 0; l < c.n_layers; ++l) {
        M.h_in[l] = h;
        rmsnorm_fwd(h.data(), &M.p[M.L.w1[l]], N, d, c.rms_eps, M.xn1[l].data(), M.r1[l].data());
        Gemm gq{N, 3 * d, d, d, M.xn1[l].data(), d, 1, &M.p[M.L.wqkv[l]], 1, d, 0, 1.0f, 0, 0};
        gemm_run(gq, M.qkv[l].data(), 3 * d);
        rope_apply(M.qkv[l].data(), B, T, H, hd, 3 * d, M.cosv.data(), M.sinv.data(), false);
        rope_apply(M.qkv[l].data() + d, B, T, H, hd, 3 * d, M.cosv.data(), M.sinv.data(), false);
        attention_fwd(B, H, T, hd, M.qkv[l].data(), M.qkv[l].data() + d, M.qkv[l].data() + 2 * d, 3 * d,
                      M.P[l].data(), M.O[l].data(), d);
        Gemm go{N, d, d, d, M.O[l].data(), d, 1, &M.p[M.L.wo[l]], 1, d, 1, 1.0f, 0, 0};
        gemm_run(go, h.data(), d);                                          // h = h + O Wo^T
        M.h_mid[l] = h;
        rmsnorm_fwd(h.data(), &M.p[M.L.w2[l]], N, d, c.rms_eps, M.xn2[l].data(), M.r2[l].data());
        Gemm ggu{N, 2 * F, d, d, M.xn2[l].data(), d, 1, &M.p[M.L.wgu[l]], 1, d, 0, 1.0f, 0, 0};
        gemm_run(ggu, M.gu[l].data(), 2 * F);
        swiglu_fwd(M.gu[l].data(), N, F, 2 * F, M.a[l].data(), F);
        Gemm gd{N, d, F, F, M.a[l].data(), F, 1, &M.p[M.L.wd[l]], 1, F, 1, 1.0f, 0, 0};
        gemm_run(gd, h.data(), d);                                          // h = h + a Wd^T
    }
    M.h_L = h;
    Gemm gh{N, V, d, d, h.data(), d, 1, &M.p[M.L.W_out], 1, d, 0, 1.0f, 0, 0};
    gemm_run(gh, M.logits.data(), V);
    if (!keep_logits) {
        M.loss = cross_entropy(M.logits.data(), M.tg.data(), N, V, M.loss_rows.data(), M.logits.data());
    } else if (with_loss) {
        std::vector<float> dl_scratch(M.logits.size());
        M.loss = cross_entropy(M.logits.data(), M.tg.data(), N, V, M.loss_rows.data(), dl_scratch.data());
    }
}

void model_backward(Model& M) {
    const orc_cfg& c = M.c;
    const int64_t N = M.N, d = c.d_model, F = c.ffn_hidden, V = c.vocab, H = c.n_heads, hd = c.head_dim;
    const int64_t B = c.batch, T = c.seq_len;
    std::fill(M.g.begin(), M.g.end(), 0.0f);
    const float* dl = M.logits.data();                                      // d-logits (in place)
    std::vector<float> dh((size_t)(N * d)), dA((size_t)(N * F)), dgu((size_t)(N * 2 * F));
    std::vector<float> dxn((size_t)(N * d)), dx((size_t)(N * d)), dO((size_t)(N * d)), dqkv((size_t)(N * 3 * d));
    // head: dh = dl W_out (K = V); dW_out = dl^T h_L (K = N)
    Gemm g1{N, d, V, V, dl, V, 1, &M.p[M.L.W_out], d, 1, 0, 1.0f, 0, 0};
    gemm_run(g1, dh.data(), d);
    Gemm g2{V, d, N, N, dl, 1, V, M.h_L.data(), d, 1, 0, 1.0f, 0, 0};
    gemm_run(g2, &M.g[M.L.W_out], d);
    for (int l = c.n_layers - 1; l >= 0; --l) {
        // MLP branch
        Gemm ga{N, F, d, d, dh.data(), d, 1, &M.p[M.L.wd[l]], F, 1, 0, 1.0f, 0, 0};
        gemm_run(ga, dA.data(), F);                                         // dA = dh Wd
        Gemm gwd{d, F, N, N, dh.data(), 1, d, M.a[l].data(), F, 1, 0, 1.0f, 0, 0};
        gemm_run(gwd, &M.g[M.L.wd[l]], F);                                  // dWd = dh^T a
        swiglu_bwd(dA.data(), F, M.gu[l].data(), N, F, 2 * F, dgu.data());
        Gemm gwgu{2 * F, d, N, N, dgu.data(), 1, 2 * F, M.xn2[l].data(), d, 1, 0, 1.0f, 0, 0};
        gemm_run(gwgu, &M.g[M.L.wgu[l]], d);                                // dWg, dWu
        Gemm gx2{N, d, 2 * F, F, dgu.data(), 2 * F, 1, &M.p[M.L.wgu[l]], d, 1, 0, 1.0f, 0, 0};
        gemm_run(gx2, dxn.data(), d);                                       // segments [dg Wg, du Wu]
        rmsnorm_bwd(dxn.data(), M.h_mid[l].data(), &M.p[M.L.w2[l]], M.r2[l].data(), N, d, dx.data(), &M.g[M.L.w2[l]]);
        for (int64_t i = 0; i < N * d; ++i) dh[i] = dh[i] + dx[i];
        // attention branch
        Gemm gdo{N, d, d, d, dh.data(), d, 1, &M.p[M.L.wo[l]], d, 1, 0, 1.0f, 0, 0};
        gemm_run(gdo, dO.data(), d);                                        // dO = dh Wo
        Gemm gwo{d, d, N, N, dh.data(), 1, d, M.O[l].data(), d, 1, 0, 1.0f, 0, 0};
        gemm_run(gwo, &M.g[M.L.wo[l]], d);                                  // dWo = dh^T O
        const float* qkv = M.qkv[l].data();
        attention_bwd(B, H, T, hd, qkv, qkv + d, qkv + 2 * d, 3 * d, M.P[l].data(), M.O[l].data(), dO.data(), d,
                      dqkv.data(), dqkv.data() + d, dqkv.data() + 2 * d);
        rope_apply(dqkv.data(), B, T, H, hd, 3 * d, M.cosv.data(), M.sinv.data(), true);
        rope_apply(dqkv.data() + d, B, T, H, hd, 3 * d, M.cosv.data(), M.sinv.data(), true);
        Gemm gwq{3 * d, d, N, N, dqkv.data(), 1, 3 * d, M.xn1[l].data(), d, 1, 0, 1.0f, 0, 0};
        gemm_run(gwq, &M.g[M.L.wqkv[l]], d);                                // dWq, dWk, dWv
        Gemm gx1{N, d, 3 * d, d, dqkv.data(), 3 * d, 1, &M.p[M.L.wqkv[l]], d, 1, 0, 1.0f, 0, 0};
        gemm_run(gx1, dxn.data(), d);                                       // segments [dq Wq, dk Wk, dv Wv]
        rmsnorm_bwd(dxn.data(), M.h_in[l].data(), &M.p[M.L.w1[l]], M.r1[l].data(), N, d, dx.data(), &M.g[M.L.w1[l]]);
        for (int64_t i = 0; i < N * d; ++i) dh[i] = dh[i] + dx[i];
    }
    // embedding: tied tables already hold the head gradient; rows add in token order
    embed_scatter(M.ids.data(), dh.data(), N, d, &M.g[M.L.E]);
    // shard accumulation: G = G + g_s
    for (int64_t i = 0; i < M.L.nparams; ++i) M.G[i] = M.G[i] + M.g[i];
}

// Checkpoint bytes (MLBC v1), all little-endian:
//  [0,8) "MLBCKPT1"; u32 format 1; u32 profile 1; 9 u32 config ints (vocab,
//  d_model, n_layers, n_heads, head_dim, ffn_hidden, tied, batch, seq_len);
//  6 f32 (rope_theta, rms_eps, beta1, beta2, adam_eps, weight_decay); u32 0;
//  u64 step; u64 n_params; SHA-256 of params, of m, of v; SHA-256 of bytes
//  [0,192); zero padding to 256; then f32 params, m, v.
constexpr int64_t HDR = 256;

void put32(uint8_t* p, uint32_t v) { for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i)); }
void put64(uint8_t* p, uint64_t v) { for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i)); }
uint32_t get32(const uint8_t* p) { uint32_t v = 0; for (int i = 0; i < 4; ++i) v |= (uint32_t)p[i] << (8 * i); return v; }
uint64_t get64(const uint8_t* p) { uint64_t v = 0; for (int i = 0; i < 8; ++i) v |= (uint64_t)p[i] << (8 * i); return v; }

void write_header(const Model& M, uint8_t* h) {
    std::memset(h, 0, HDR);
    std::memcpy(h, "MLBCKPT1", 8);
    put32(h + 8, 1); put32(h + 12, 1);
    const int32_t ci[9] = {M.c.vocab, M.c.d_model, M.c.n_layers, M.c.n_heads, M.c.head_dim,
                           M.c.ffn_hidden, M.c.tied, M.c.batch, M.c.seq_len};
    for (int i = 0; i < 9; ++i) put32(h + 16 + 4 * i, (uint32_t)ci[i]);
    const float cf[6] = {M.c.rope_theta, M.c.rms_eps, M.c.beta1, M.c.beta2, M.c.adam_eps, M.c.weight_decay};
    for (int i = 0; i < 6; ++i) put32(h + 52 + 4 * i, fbits(cf[i]));
    put32(h + 76, 0);
    put64(h + 80, (uint64_t)M.step);
    put64(h + 88, (uint64_t)M.L.nparams);
    const size_t nb = (size_t)M.L.nparams * 4;
    sha256((const uint8_t*)M.p.data(), nb, h + 96);
    sha256((const uint8_t*)M.m.data(), nb, h + 128);
    sha256((const uint8_t*)M.v.data(), nb, h + 160);
    sha256(h, 192, h + 192);
}

}  // namespace

// ====================================================================== C API
extern "C" {

void orc_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int orc_set_sabotage(int arm) {
    if (arm < 0 || arm >= SAB_COUNT) return -1;
    g_sab = arm;
    // The flush arm turns on FTZ and DAZ for the calling thread (run it with one thread).
    if (arm == SAB_FTZ_DAZ) _mm_setcsr(_mm_getcsr() | 0x8040u);
    else _mm_setcsr(_mm_getcsr() & ~0x8040u);
    return 0;
}
int orc_sabotage_count(void) { return SAB_COUNT; }
int orc_get_threads(void) { return g_threads; }
int orc_ftz_daz_set(void) { return (_mm_getcsr() & 0x8040u) != 0; }

float orc_exp(float x) { return exp_p(x); }
float orc_log(float x) { return log_p(x); }
float orc_fma(float a, float b, float c) { return std::fma(a, b, c); }
void orc_exp_array(const float* x, float* y, int64_t n) {
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = exp_p(x[i]);
}
void orc_log_array(const float* x, float* y, int64_t n) {
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = log_p(x[i]);
}
void orc_fma_array(const float* a, const float* b, const float* c, float* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = std::fma(a[i], b[i], c[i]);
}
void orc_sigmoid_array(const float* x, float* y, int64_t n) {
#pragma omp parallel for num_threads(g_threads) schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = sigmoid_p(x[i]);
}

float orc_sum64(const float* v, int64_t n) { return sum64(v, n); }
float orc_dot64(const float* a, const float* b, int64_t n) { return dot64(a, b, n); }
float orc_max64(const float* v, int64_t n) { return max64(v, n); }

int orc_gemm(int64_t M, int64_t N, int64_t K, int64_t kseg, const float* A, int64_t sam, int64_t sak,
             const float* B, int64_t sbk, int64_t sbn, float* C, int64_t ldc, int mode, float scale,
             int krange, int outmask) {
    Gemm g{M, N, K, kseg > 0 ? kseg : K, A, sam, sak, B, sbk, sbn, mode, scale, krange, outmask};
    if (K == 0) g.kseg = 1;
    if (!gemm_check(g)) return -1;
    gemm_run(g, C, ldc);
    return 0;
}

int orc_gemm_rows(int64_t M, int64_t N, int64_t K, int64_t kseg, const float* A, int64_t sam, int64_t sak,
                  const float* B, int64_t sbk, int64_t sbn, const int64_t* rows, int64_t nrows, float* C,
                  int64_t ldc, int mode, float scale, int krange, int outmask) {
    Gemm g{M, N, K, kseg > 0 ? kseg : K, A, sam, sak, B, sbk, sbn, mode, scale, krange, outmask};
    if (K == 0) g.kseg = 1;
    if (!gemm_check(g)) return -1;
    for (int64_t r = 0; r < nrows; ++r) if (rows[r] < 0 || rows[r] >= M) return -1;
    std::vector<float> bt = make_bt(g);
#pragma omp parallel num_threads(g_threads)
    {
        std::vector<float> acc((size_t)std::max<int64_t>(1, N)), tot((size_t)std::max<int64_t>(1, N));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < nrows; ++r) gemm_row(g, bt.data(), rows[r], C + r * ldc, acc.data(), tot.data());
    }
    return 0;
}

void orc_rmsnorm_fwd(const float* x, const float* w, int64_t rows, int64_t d, float eps, float* y, float* r) {
    rmsnorm_fwd(x, w, rows, d, eps, y, r);
}
void orc_rmsnorm_bwd(const float* dy, const float* x, const float* w, const float* r, int64_t rows, int64_t d,
                     float* dx, float* dw) {
    rmsnorm_bwd(dy, x, w, r, rows, d, dx, dw);
}
void orc_rope_table(int64_t T, int64_t hd, float theta, float* cosv, float* sinv) { rope_table(T, hd, theta, cosv, sinv); }
void orc_rope_fwd(float* x, int64_t B, int64_t T, int64_t H, int64_t hd, int64_t ld, const float* cosv, const float* sinv) {
    rope_apply(x, B, T, H, hd, ld, cosv, sinv, false);
}
void orc_rope_bwd(float* dx, int64_t B, int64_t T, int64_t H, int64_t hd, int64_t ld, const float* cosv, const float* sinv) {
    rope_apply(dx, B, T, H, hd, ld, cosv, sinv, true);
}
float orc_attn_scale(int64_t hd) { return attn_scale(hd); }
void orc_attention_fwd(int64_t B, int64_t H, int64_t T, int64_t hd, const float* q, const float* k, const float* v,
                       int64_t ld, float* P, float* O, int64_t ldo) {
    attention_fwd(B, H, T, hd, q, k, v, ld, P, O, ldo);
}
void orc_attention_bwd(int64_t B, int64_t H, int64_t T, int64_t hd, const float* q, const float* k, const float* v,
                       int64_t ld, const float* P, const float* O, const float* dO, int64_t ldo, float* dq, float* dk,
                       float* dv) {
    attention_bwd(B, H, T, hd, q, k, v, ld, P, O, dO, ldo, dq, dk, dv);
}
void orc_swiglu_fwd(const float* gu, int64_t rows, int64_t F, int64_t ldgu, float* a, int64_t lda) {
    swiglu_fwd(gu, rows, F, ldgu, a, lda);
}
void orc_swiglu_bwd(const float* dA, int64_t ldda, const float* gu, int64_t rows, int64_t F, int64_t ldgu, float* dgu) {
    swiglu_bwd(dA, ldda, gu, rows, F, ldgu, dgu);
}
float orc_cross_entropy(const float* logits, const int32_t* targets, int64_t N, int64_t V, float* loss_rows, float* dl) {
    return cross_entropy(logits, targets, N, V, loss_rows, dl);
}
void orc_embed_scatter(const int32_t* ids, const float* dh, int64_t N, int64_t d, float* dE) {
    embed_scatter(ids, dh, N, d, dE);
}
float orc_bias_correction(float beta, int64_t t) { return bias_correction(beta, t); }
void orc_adamw(float* p, const float* g, float* m, float* v, int64_t n, float lr, float beta1, float beta2, float eps,
               float wd, float bc1, float bc2) {
    adamw(p, g, m, v, n, lr, beta1, beta2, eps, wd, bc1, bc2);
}
void orc_sha256(const uint8_t* data, int64_t len, uint8_t out[32]) { sha256(data, (size_t)len, out); }

int64_t orc_param_count(const orc_cfg* cfg) {
    if (!cfg || !cfg_ok(*cfg)) return -1;
    return make_layout(*cfg).nparams;
}

void orc_splitmix64(uint64_t seed, int64_t n, uint64_t* out) {
    uint64_t state = seed;
    for (int64_t i = 0; i < n; ++i) {
        state += 0x9E3779B97F4A7C15ull;
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        out[i] = z ^ (z >> 31);
    }
}

void orc_seed_params(const orc_cfg* cfg, uint64_t seed, float* out) {
    if (!cfg || !cfg_ok(*cfg) || !out) return;
    const Layout L = make_layout(*cfg);
    const int64_t d = cfg->d_model;
    // which canonical positions are norm gains
    std::vector<char> gain((size_t)L.nparams, 0);
    for (int l = 0; l < cfg->n_layers; ++l)
        for (int64_t c = 0; c < d; ++c) { gain[(size_t)(L.w1[l] + c)] = 1; gain[(size_t)(L.w2[l] + c)] = 1; }
    const double two_pi = 6.283185307179586;   // binary64 nearest to 2 pi
    const double two_m53 = 1.0 / 9007199254740992.0;
    uint64_t pair[2];
    uint64_t state_seed = seed;
    for (int64_t k = 0; k < L.nparams; ++k) {
        orc_splitmix64(state_seed, 2, pair);        // outputs 2k and 2k+1
        state_seed += 2 * 0x9E3779B97F4A7C15ull;
        const double u1 = (double)((pair[0] >> 11) + 1) * two_m53;
        const double u2 = (double)(pair[1] >> 11) * two_m53;
        const double radius = std::sqrt(-2.0 * std::log(u1));
        const double z = radius * std::cos(two_pi * u2);
        const double w = 0.02 * z;
        out[k] = gain[(size_t)k] ? (float)(1.0 + w) : (float)w;
    }
}

void* orc_model_new(const orc_cfg* cfg, const float* init) {
    if (!cfg || !cfg_ok(*cfg) || !init) return nullptr;
    Model* M = new Model();
    M->c = *cfg;
    M->L = make_layout(*cfg);
    const orc_cfg& c = M->c;
    const int64_t n = M->L.nparams, N = (int64_t)c.batch * c.seq_len, d = c.d_model, F = c.ffn_hidden;
    M->N = N;
    M->p.assign(init, init + n);
    M->G.assign((size_t)n, 0.0f); M->m.assign((size_t)n, 0.0f); M->v.assign((size_t)n, 0.0f); M->g.assign((size_t)n, 0.0f);
    M->cosv.resize((size_t)(c.seq_len * c.head_dim / 2)); M->sinv.resize(M->cosv.size());
    rope_table(c.seq_len, c.head_dim, c.rope_theta, M->cosv.data(), M->sinv.data());
    const int L = c.n_layers;
    auto alloc = [&](std::vector<std::vector<float>>& v, int64_t sz) { v.assign(L, std::vector<float>((size_t)sz)); };
    alloc(M->h_in, N * d); alloc(M->xn1, N * d); alloc(M->r1, N); alloc(M->qkv, N * 3 * d);
    alloc(M->P, (int64_t)c.batch * c.n_heads * c.seq_len * c.seq_len); alloc(M->O, N * d);
    alloc(M->h_mid, N * d); alloc(M->xn2, N * d); alloc(M->r2, N); alloc(M->gu, N * 2 * F); alloc(M->a, N * F);
    M->h_L.resize((size_t)(N * d)); M->logits.resize((size_t)(N * c.vocab)); M->loss_rows.resize((size_t)N);
    return M;
}

void orc_model_free(void* m) { delete (Model*)m; }

int orc_model_forward(void* mp, const int32_t* inputs, const int32_t* targets, float* loss) {
    Model& M = *(Model*)mp;
    for (int64_t i = 0; i < M.N; ++i)
        if (inputs[i] < 0 || inputs[i] >= M.c.vocab || targets[i] < 0 || targets[i] >= M.c.vocab) {
            if (loss) *loss = NAN;
            return -1;
        }
    M.ids.assign(inputs, inputs + M.N);
    M.tg.assign(targets, targets + M.N);
    model_forward(M);
    M.have_fwd = true;
    if (loss) *loss = M.loss;
    return 0;
}

int orc_model_infer(void* mp, const int32_t* inputs, const int32_t* targets, float* logits, float* loss) {
    Model& M = *(Model*)mp;
    for (int64_t i = 0; i < M.N; ++i)
        if (inputs[i] < 0 || inputs[i] >= M.c.vocab || (targets && (targets[i] < 0 || targets[i] >= M.c.vocab)))
            return -1;
    M.ids.assign(inputs, inputs + M.N);
    if (targets) M.tg.assign(targets, targets + M.N);
    model_forward(M, true, targets != nullptr);
    M.have_fwd = false;
    if (logits) std::memcpy(logits, M.logits.data(), M.logits.size() * 4);
    if (loss) *loss = targets ? M.loss : NAN;
    return 0;
}

int64_t orc_argmax(const float* x, int64_t n) {
    int64_t best = -1;
    for (int64_t i = 0; i < n; ++i)
        if (!std::isnan(x[i]) && (best < 0 || x[i] > x[best])) best = i;
    return best < 0 ? 0 : best;
}

int orc_model_backward(void* mp) {
    Model& M = *(Model*)mp;
    if (!M.have_fwd) return -1;
    model_backward(M);
    M.have_fwd = false;
    M.n_accum += 1;
    return 0;
}

int orc_model_adamw(void* mp, float lr) {
    Model& M = *(Model*)mp;
    if (M.n_accum < 1) return -1;
    M.step += 1;
    const float bc1 = bias_correction(M.c.beta1, M.step), bc2 = bias_correction(M.c.beta2, M.step);
    adamw(M.p.data(), M.G.data(), M.m.data(), M.v.data(), M.L.nparams, lr, M.c.beta1, M.c.beta2, M.c.adam_eps,
          M.c.weight_decay, bc1, bc2);
    std::fill(M.G.begin(), M.G.end(), 0.0f);
    M.n_accum = 0;
    return 0;
}

void orc_model_read(void* mp, int which, float* dst) {
    Model& M = *(Model*)mp;
    const std::vector<float>* src = which == 0 ? &M.p : which == 1 ? &M.G : which == 2 ? &M.m : &M.v;
    std::memcpy(dst, src->data(), src->size() * 4);
}

int64_t orc_model_step(void* mp) { return ((Model*)mp)->step; }

int64_t orc_model_save(void* mp, uint8_t* buf, int64_t cap) {
    Model& M = *(Model*)mp;
    const int64_t nb = M.L.nparams * 4;
    const int64_t total = HDR + 3 * nb;
    if (!buf) return total;
    if (cap < total || M.n_accum != 0) return -1;
    write_header(M, buf);
    std::memcpy(buf + HDR, M.p.data(), (size_t)nb);
    std::memcpy(buf + HDR + nb, M.m.data(), (size_t)nb);
    std::memcpy(buf + HDR + 2 * nb, M.v.data(), (size_t)nb);
    return total;
}

int orc_model_load(void* mp, const uint8_t* buf, int64_t len) {
    Model& M = *(Model*)mp;
    const int64_t nb = M.L.nparams * 4;
    if (len != HDR + 3 * nb) return -1;
    if (std::memcmp(buf, "MLBCKPT1", 8) != 0 || get32(buf + 8) != 1 || get32(buf + 12) != 1) return -2;
    uint8_t hd[32];
    sha256(buf, 192, hd);
    if (std::memcmp(hd, buf + 192, 32) != 0) return -3;
    Model tmp;
    tmp.c = M.c; tmp.L = M.L; tmp.step = (int64_t)get64(buf + 80);
    tmp.p.assign((const float*)(buf + HDR), (const float*)(buf + HDR) + M.L.nparams);
    tmp.m.assign((const float*)(buf + HDR + nb), (const float*)(buf + HDR + nb) + M.L.nparams);
    tmp.v.assign((const float*)(buf + HDR + 2 * nb), (const float*)(buf + HDR + 2 * nb) + M.L.nparams);
    uint8_t expect[HDR];
    write_header(tmp, expect);
    if (std::memcmp(expect, buf, HDR) != 0) return -4;       // config, count or array digest mismatch
    M.p = tmp.p; M.m = tmp.m; M.v = tmp.v; M.step = tmp.step;
    std::fill(M.G.begin(), M.G.end(), 0.0f);
    M.n_accum = 0;
    M.have_fwd = false;
    return 0;
}

int64_t orc_model_stage(void* mp, int stage, int layer, float* dst) {
    Model& M = *(Model*)mp;
    const std::vector<float>* s = nullptr;
    if (layer < 0 || layer >= M.c.n_layers) layer = 0;
    switch (stage) {
        case 0: s = &M.h_in[layer]; break;
        case 1: s = &M.xn1[layer]; break;
        case 2: s = &M.r1[layer]; break;
        case 3: s = &M.qkv[layer]; break;
        case 4: s = &M.P[layer]; break;
        case 5: s = &M.O[layer]; break;
        case 6: s = &M.h_mid[layer]; break;
        case 7: s = &M.xn2[layer]; break;
        case 8: s = &M.r2[layer]; break;
        case 9: s = &M.gu[layer]; break;
        case 10: s = &M.a[layer]; break;
        case 11: s = &M.h_L; break;
        case 12: s = &M.logits; break;
        case 13: s = &M.loss_rows; break;
        default: return -1;
    }
    if (dst) std::memcpy(dst, s->data(), s->size() * 4);
    if (dst && stage == 4) {   // canonical export: +0 above the diagonal (those entries are not part of P)
        const int64_t T = M.c.seq_len, nz = (int64_t)s->size() / (T * T);
        for (int64_t z = 0; z < nz; ++z)
            for (int64_t i = 0; i < T; ++i)
                for (int64_t j = i + 1; j < T; ++j) dst[(z * T + i) * T + j] = 0.0f;
    }
    return (int64_t)s->size();
}

}  // extern "C"
