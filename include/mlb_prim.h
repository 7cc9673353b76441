/*
 * mlb_prim.h - the step's kernels as standalone C-ABI calls (device pointers).
 *
 * These expose each stage of the MLB-P1 training step on its own so that it can
 * be checked bit for bit at full size and timed. All pointers are device
 * memory owned by the caller; sizes are element counts; every call enqueues on
 * hip_stream (may be null) and does not synchronise. Return values are
 * mlb_status codes from mlb.h. Where a call needs scratch memory the caller
 * passes it (ws, ws_bytes) and the required size is stated next to the call;
 * a smaller ws gives MLB_E_ARENA_TOO_SMALL.
 */
#ifndef MLB_PRIM_H
#define MLB_PRIM_H
#include <stddef.h>
#include <stdint.h>
#include "mlb.h"
#ifdef __cplusplus
extern "C" {
#endif

/* G1024 contraction t(i,j) = sum_k A(i,k) B(k,j) (the profile's only product
 * rule; mojolearn PyPI page, "What bitwise identity means": fixed reduction
 * order and partitioning). K is cut into segments of kseg (0 = K), each cut
 * into chunks at multiples of 1024 of its own index; krange 1 keeps k <= i,
 * 2 keeps k >= i; each chunk is an fma chain from +0 in ascending k; non-empty
 * chunks add left to right; empty contraction = +0.
 * A(i,k) = a_kc ? A[i*lda+k] : A[k*lda+i]; B(k,j) = b_kc ? B[j*ldb+k] : B[k*ldb+j];
 * C(i,j) = C[i*ldc+j]. mode 0 C = t, 1 C = C + t, 2 C = t * scale. outmask 1
 * writes j <= i only. batch = number of problems, heads divides batch, problem
 * z = zb*heads + zh offsets A by zb*sAb + zh*sAh (same for B, C).
 * Launch choices that never change bits: tile (-1 auto, 0 128x128, 1 256x64,
 * 2 128x64; causal ranges need 2),
 * split (-1 auto, 0 off, 1 per-chunk partials folded by a second kernel; needs
 * ws of ceil(K/1024)*M*N floats; for a causal range in mode 0, -1 and 1 run
 * one launch per chunk that stores the first chunk and adds the later ones,
 * 0 keeps the running total in registers), simple (1 = one thread per output). */
mlb_status mlb_prim_gemm(int64_t M, int64_t N, int64_t K, int64_t kseg, const float* A, int64_t lda, int a_kc,
                         const float* B, int64_t ldb, int b_kc, float* C, int64_t ldc, int krange, int outmask,
                         int mode, float scale, int64_t batch, int64_t heads, int64_t sAb, int64_t sAh,
                         int64_t sBb, int64_t sBh, int64_t sCb, int64_t sCh, int tile, int split, int simple,
                         void* ws, size_t ws_bytes, void* hip_stream);

/* Two independent contractions of one kind in one launch, as the training
 * step runs the q/k/v and Wo weight gradients: problem 0 (M0 x N0) and problem
 * 1 (M1 x N1), both over K (one segment), both with the layout a_kc/b_kc and
 * mode (0 store, 1 accumulate) of mlb_prim_gemm, under its automatic plan. When
 * they cannot share a launch (a causal range, a mask, 64-wide outputs, other
 * load widths) they run one after the other; the bits are the same either way.
 * ws: the per-chunk partials of both (ceil(K/1024)*(M0*N0 + M1*N1) floats)
 * when K > 1024; too small a ws makes them run unsplit. */
mlb_status mlb_prim_gemm_pair(int64_t M0, int64_t N0, int64_t M1, int64_t N1, int64_t K, const float* A0,
                              int64_t lda0, const float* B0, int64_t ldb0, float* C0, int64_t ldc0, const float* A1,
                              int64_t lda1, const float* B1, int64_t ldb1, float* C1, int64_t ldc1, int a_kc, int b_kc,
                              int mode, void* ws, size_t ws_bytes, void* hip_stream);

/* RMSNorm over rows of d (model card: RMSNorm eps 1e-6, pre-norm):
 * r = 1/sqrt(DOT64(x,x)/d + eps), y = (x*r)*w. x,y [rows,d], r [rows]. */
mlb_status mlb_prim_rmsnorm_fwd(const float* x, const float* w, int64_t rows, int64_t d, float eps, float* y,
                                float* r, void* hip_stream);
/* dx = r*(dy*w - (x*r)*c), c = DOT64(dy*w, x*r)/d; dw = contraction over rows of
 * dy*(x*r) in 1024-row chunks. ws: ceil(rows/1024)*d floats. */
mlb_status mlb_prim_rmsnorm_bwd(const float* dy, const float* x, const float* w, const float* r, int64_t rows,
                                int64_t d, float* dx, float* dw, void* ws, size_t ws_bytes, void* hip_stream);

/* Rotary positions (model card: rotary, theta 10,000), half-split pairs (i,
 * i+hd/2), angle t*theta^(-2i/hd) tabulated in binary64 on the host and rounded.
 * x rows [B*T, ld], heads at column h*hd; t = row mod T. backward 1 applies the
 * transposed rotation. In place. */
mlb_status mlb_prim_rope(float* x, int64_t B, int64_t T, int64_t H, int64_t hd, int64_t ld, float theta,
                         int backward, void* hip_stream);

/* Causal attention for B*H heads (model card: 12 heads x 64, context 2,048):
 * S = (q.k)*RN(1/sqrt(hd)) for j <= i, P = softmax with MAX64/SUM64 and
 * e*(1/Z), O = G1024 over j <= i of P v. q,k,v point at head (0,0); head (b,h)
 * row t at ptr[(b*T+t)*ld + h*hd]. P holds B*H matrices of T*T floats (only
 * j <= i written): row-major when p_tiled = 0, else the training step's
 * layout of 32x32 tiles (element (i,j) at ((i/32)*(T/32) + j/32)*1024 +
 * (i%32)*32 + j%32; needs T % 32 == 0 and hd <= 64). O rows at stride ldo. */
mlb_status mlb_prim_attention_fwd(int64_t B, int64_t H, int64_t T, int64_t hd, const float* q, const float* k,
                                  const float* v, int64_t ld, float* P, float* O, int64_t ldo, int p_tiled,
                                  void* hip_stream);
/* D = DOT64(dO,O); dP = dO.v; dS = (P*(dP-D))*scale; dq = dS k (j <= i);
 * dk = dS^T q, dv = P^T dO (i >= j). dq/dk/dv use the q layout.
 * ws: B*H*T*T + B*H*T floats. */
mlb_status mlb_prim_attention_bwd(int64_t B, int64_t H, int64_t T, int64_t hd, const float* q, const float* k,
                                  const float* v, int64_t ld, const float* P, const float* O, const float* dO,
                                  int64_t ldo, float* dq, float* dk, float* dv, int p_tiled, void* ws,
                                  size_t ws_bytes, void* hip_stream);

/* SwiGLU (model card: SwiGLU, 2,048 wide): gu rows [g | u] of 2F, a = (g*sig(g))*u,
 * sig(x) = 1/(1+exp(-x)). Backward writes dgu [rows, 2F]. */
mlb_status mlb_prim_swiglu_fwd(const float* gu, int64_t rows, int64_t F, float* a, void* hip_stream);
mlb_status mlb_prim_swiglu_bwd(const float* dA, const float* gu, int64_t rows, int64_t F, float* dgu,
                               void* hip_stream);

/* Cross-entropy (mojolearn project page: cross entropy in the verified chain):
 * per row loss = log(Z) - (l_y - m), dl = ((exp(l-m)*(1/Z)) - [v=y]) * (1/N);
 * loss_dev[0] = SUM64(rows)*(1/N). dl may alias logits. A target outside
 * [0, V) gives MLB_E_BAD_TOKEN (the stream is synchronised to check). */
mlb_status mlb_prim_cross_entropy(const float* logits, const int32_t* targets, int64_t N, int64_t V,
                                  float* loss_rows, float* dl, float* loss_dev, void* hip_stream);

/* Embedding-gradient scatter (model card: the input table is a lookup): for
 * each row v, in increasing position n with ids[n] = v, dE[v] = dE[v] + dh[n]
 * (sorted segments, no floating-point atomics). N <= 65,536; ids outside
 * [0, V) are skipped. ws: 131,072 bytes for N <= 8,192, else 16*P bytes with P
 * the smallest power of two >= N (the sort keys and their merge buffer); a
 * smaller ws gives MLB_E_ARENA_TOO_SMALL, a larger N MLB_E_UNSUPPORTED. */
mlb_status mlb_prim_embed_scatter(const int32_t* ids, const float* dh, int64_t N, int64_t d, int64_t V, float* dE,
                                  void* ws, size_t ws_bytes, void* hip_stream);

/* The embedding-gradient scatter above without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the sort keys live in
 * a static device array of the library (64 KiB per GPU, held until the process
 * ends), so the call allocates nothing. Same arguments, rule and bits as
 * mlb_prim_embed_scatter. N above 8,192 gives MLB_E_UNSUPPORTED. Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (several
 * streams or threads at once) race and must not be made. */
mlb_status mlb_prim_embed_scatter_noalloc(const int32_t* ids, const float* dh, int64_t N, int64_t d, int64_t V,
                                          float* dE, void* hip_stream);

/* AdamW (model card "Training" table: beta (0.9, 0.95), eps 1e-8, wd 0.1),
 * coupled form, step t >= 1: bias corrections RN(1 - beta^t) from a binary64
 * product. Updates p, m, v in place and sets g to +0. */
mlb_status mlb_prim_adamw(float* p, float* g, float* m, float* v, int64_t n, float lr, float beta1, float beta2,
                          float eps, float wd, int64_t t, void* hip_stream);

/* Elementwise spellings: which 0 exp, 1 log, 2 sigmoid, 3 exp in its branch-free
 * form (the same bits as 0, as the cross-entropy of long rows evaluates it). */
mlb_status mlb_prim_unary(const float* x, float* y, int64_t n, int which, void* hip_stream);

/* Matrix-core probe: one FP32 MFMA per wavefront on lane-held operands, for
 * checking its rounding and accumulation order against a CPU fma chain.
 * variant 0 32x32x1 (2 blocks, 32 out/lane), 1 16x16x1 (4 blocks, 16), 2 4x4x1
 * (16 blocks, 4), 3 32x32x2 (16), 4 16x16x4 (4). A, B: nwaves*64; C, D:
 * nwaves*64*out_per_lane floats, lane-major. */
mlb_status mlb_diag_mfma(int variant, const float* A, const float* B, const float* C, float* D, int64_t nwaves,
                         void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif
