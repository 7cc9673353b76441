/*
 * CPU oracle for the MLB-P1 bitwise FP32 training-step profile.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls
 * this library: only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do. It shares no code, header, table or constant generator with the
 * HIP library; both are written from the profile's prose definition.
 *
 * The oracle computes, step by step and in plain loops, what the pages'
 * identical mode promises (mojolearn PyPI page, "What bitwise identity means":
 * a frozen profile fixing reduction order, partitioning, FMA policy, flush
 * seams, transcendental spellings and tie rules). The concrete rules are this
 * build's reading of that category list and are restated next to each function
 * in oracle.cpp.
 *
 * All float arguments are IEEE binary32. Pointers are host memory owned by the
 * caller. Functions never allocate memory that outlives the call, except the
 * model handle (orc_model_new / orc_model_free).
 */
#ifndef MLB_ORACLE_H
#define MLB_ORACLE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

/* Number of OpenMP threads used across independent outputs (default 1).
 * Every output is computed by the same operation sequence whatever the count. */
void orc_set_threads(int n);
int orc_get_threads(void);
/* Tests only: select a sabotage arm that breaks one profile rule (0 = none).
 * 1 reverse k, 2 chunk 512, 3 pairwise chunk tree, 4 mul+add, 5 mirror lane
 * pairing, 6 32 lanes, 7 libm exp, 8 FTZ/DAZ, 9 divide by Z, 10 decoupled
 * AdamW, 11 reversed scatter, 12 libm log. Returns -1 for an unknown arm. */
int orc_set_sabotage(int arm);
int orc_sabotage_count(void);
/* Returns 1 if the x86 MXCSR has FTZ or DAZ set (the profile forbids both). */
int orc_ftz_daz_set(void);

/* Elementary spellings (exp, log, fma) and their array forms. */
float orc_exp(float x);
float orc_log(float x);
float orc_fma(float a, float b, float c);
void orc_exp_array(const float* x, float* y, int64_t n);
void orc_log_array(const float* x, float* y, int64_t n);
void orc_fma_array(const float* a, const float* b, const float* c, float* y, int64_t n);
void orc_sigmoid_array(const float* x, float* y, int64_t n);

/* W64 row reductions over v[0..n). */
float orc_sum64(const float* v, int64_t n);
float orc_dot64(const float* a, const float* b, int64_t n);
float orc_max64(const float* v, int64_t n);

/* G1024 contraction, the only matrix-product rule:
 *   t(i,j) = sum over k of A(i,k) * B(k,j), with
 *   A(i,k) = A[i*sam + k*sak], B(k,j) = B[k*sbk + j*sbn].
 * The K range [0,K) is split into segments of length kseg (K % kseg == 0);
 * each segment is cut into chunks at multiples of 1024 of its own local index;
 * krange 1 keeps k <= i only, krange 2 keeps k >= i only (absolute k); empty
 * chunks are skipped; each chunk is an fma chain from +0 in ascending k; the
 * chunk results are added left to right in list order. An empty contraction
 * is +0.
 * mode 0: C = t; mode 1: C = C + t; mode 2: C = t * scale.
 * outmask 1: only outputs with j <= i are written.
 * Returns 0, or -1 on bad arguments. */
int orc_gemm(int64_t M, int64_t N, int64_t K, int64_t kseg,
             const float* A, int64_t sam, int64_t sak,
             const float* B, int64_t sbk, int64_t sbn,
             float* C, int64_t ldc, int mode, float scale, int krange, int outmask);
/* Same contraction for an explicit list of output rows only (rows[0..nrows)),
 * written densely to C[r*ldc + j]. Used to check sampled outputs at full size. */
int orc_gemm_rows(int64_t M, int64_t N, int64_t K, int64_t kseg,
                  const float* A, int64_t sam, int64_t sak,
                  const float* B, int64_t sbk, int64_t sbn,
                  const int64_t* rows, int64_t nrows, float* C, int64_t ldc,
                  int mode, float scale, int krange, int outmask);

/* RMSNorm over rows of length d (row stride d). y and r are written. */
void orc_rmsnorm_fwd(const float* x, const float* w, int64_t rows, int64_t d, float eps,
                     float* y, float* r);
/* RMSNorm backward: dx written; dw written as the contraction over rows. */
void orc_rmsnorm_bwd(const float* dy, const float* x, const float* w, const float* r,
                     int64_t rows, int64_t d, float* dx, float* dw);

/* Rotary embedding, half-split pairing, on rows of a [B*T, ld] array. Heads
 * start at column offsets h*hd for h < H. cosv/sinv are [T, hd/2] tables. */
void orc_rope_table(int64_t T, int64_t hd, float theta, float* cosv, float* sinv);
void orc_rope_fwd(float* x, int64_t B, int64_t T, int64_t H, int64_t hd, int64_t ld,
                  const float* cosv, const float* sinv);
void orc_rope_bwd(float* dx, int64_t B, int64_t T, int64_t H, int64_t hd, int64_t ld,
                  const float* cosv, const float* sinv);

/* Causal attention for B*H heads of length T. q,k,v point at head (0,0);
 * head (b,h) row t lives at ptr[(b*T + t)*ld + h*hd]. P is [B*H, T, T]
 * (only j <= i written), O rows use ldo. scale = RN(1/sqrt(hd)). */
float orc_attn_scale(int64_t hd);
void orc_attention_fwd(int64_t B, int64_t H, int64_t T, int64_t hd,
                       const float* q, const float* k, const float* v, int64_t ld,
                       float* P, float* O, int64_t ldo);
/* Backward. dS overwrites nothing of P; dq/dk/dv written (ld layout like q). */
void orc_attention_bwd(int64_t B, int64_t H, int64_t T, int64_t hd,
                       const float* q, const float* k, const float* v, int64_t ld,
                       const float* P, const float* O, const float* dO, int64_t ldo,
                       float* dq, float* dk, float* dv);

/* SwiGLU on rows: g at gu[n*ldgu + f], u at gu[n*ldgu + F + f]. */
void orc_swiglu_fwd(const float* gu, int64_t rows, int64_t F, int64_t ldgu, float* a, int64_t lda);
void orc_swiglu_bwd(const float* dA, int64_t ldda, const float* gu, int64_t rows, int64_t F,
                    int64_t ldgu, float* dgu);

/* Cross-entropy rows: per-row losses written to loss_rows, d-logits written to
 * dl (may alias logits). Returns the shard loss (sum64 of rows times 1/N). */
float orc_cross_entropy(const float* logits, const int32_t* targets, int64_t N, int64_t V,
                        float* loss_rows, float* dl);

/* Embedding-gradient scatter: for n ascending, dE[ids[n]] += dh[n] (row-wise). */
void orc_embed_scatter(const int32_t* ids, const float* dh, int64_t N, int64_t d, float* dE);

/* AdamW over n elements, in place on p, m, v. */
float orc_bias_correction(float beta, int64_t t);
void orc_adamw(float* p, const float* g, float* m, float* v, int64_t n, float lr,
               float beta1, float beta2, float eps, float wd, float bc1, float bc2);

void orc_sha256(const uint8_t* data, int64_t len, uint8_t out[32]);

/* Model. */
typedef struct orc_cfg {
    int32_t vocab, d_model, n_layers, n_heads, head_dim, ffn_hidden, tied, batch, seq_len;
    float rope_theta, rms_eps, beta1, beta2, adam_eps, weight_decay;
} orc_cfg;
int64_t orc_param_count(const orc_cfg* cfg);
/* The first n outputs of SplitMix64 started at seed (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", 2014): the state advances
 * by the golden gamma 0x9E3779B97F4A7C15 and each output is the state passed
 * through the variant-13 finaliser. */
void orc_splitmix64(uint64_t seed, int64_t n, uint64_t* out);
/* Step-0 parameters from a seed, for a caller that passes none: parameter k of
 * the canonical order takes SplitMix64 outputs 2k and 2k+1; u1 = (first >> 11
 * plus 1) * 2^-53 in (0, 1], u2 = (second >> 11) * 2^-53; the Box-Muller
 * transform (1958) in binary64 gives z = sqrt(-2 log u1) * cos(2 pi u2); norm
 * gains take 1 + 0.02 z, every other parameter 0.02 z, each rounded once to
 * binary32. out holds orc_param_count(cfg) floats. */
void orc_seed_params(const orc_cfg* cfg, uint64_t seed, float* out);
void* orc_model_new(const orc_cfg* cfg, const float* init_params);
void orc_model_free(void* m);
/* Forward and loss of one micro-batch; stores activations. Returns -1 (and sets
 * *loss to NaN) on an out-of-range token. */
int orc_model_forward(void* m, const int32_t* inputs, const int32_t* targets, float* loss);
/* Inference forward of one batch: logits [tokens, vocab] (may be NULL) and,
 * when targets is not NULL, the mean loss; nothing is kept for a backward.
 * Returns -1 on an out-of-range token. */
int orc_model_infer(void* m, const int32_t* inputs, const int32_t* targets, float* logits, float* loss);
/* Index of the largest entry of x[0..n): NaN ranks below every number, ties go
 * to the lowest index, 0 when every entry is NaN. */
int64_t orc_argmax(const float* x, int64_t n);
/* Backward of the last forward; folds its gradient into G. */
int orc_model_backward(void* m);
/* AdamW step with learning rate lr; G is then reset to +0. */
int orc_model_adamw(void* m, float lr);
/* which: 0 params, 1 G, 2 adam m, 3 adam v. */
void orc_model_read(void* m, int which, float* dst);
int64_t orc_model_step(void* m);
/* Exact state bytes (checkpoint). With buf NULL returns the size. */
int64_t orc_model_save(void* m, uint8_t* buf, int64_t cap);
int orc_model_load(void* m, const uint8_t* buf, int64_t len);
/* Activation export of the last forward (stage id, layer); returns element count. */
/* Stage 4 (P) is exported dense with +0 above the diagonal. */
int64_t orc_model_stage(void* m, int stage, int layer, float* dst);

#ifdef __cplusplus
}
#endif
#endif
