// Internal launch interface between the C-ABI host code and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlb {

// One G1024 contraction (the profile's only matrix-product rule):
//   t(i,j) = sum_k A(i,k) B(k,j)
// The K range is split into segments of length kseg; each segment is cut into
// chunks at multiples of 1024 of its local index; krange 1 keeps k <= i and
// krange 2 keeps k >= i; every chunk is an fma chain from +0 in ascending k;
// the non-empty chunks are added left to right. An empty contraction is +0.
// Epilogue: mode 0 C = t, mode 1 C = C + t, mode 2 C = t * scale, mode 3
// C = R + t (R a separate residual input with the C layout); outmask writes
// only j <= i.
// Layouts: a_kc means A(i,k) = A[i*lda + k] (k contiguous), otherwise
// A(i,k) = A[k*lda + i]. b_kc means B(k,j) = B[j*ldb + k], otherwise
// B(k,j) = B[k*ldb + j]. C(i,j) = C[i*ldc + j].
// Batches: z = zb*H + zh adds zb*s?b + zh*s?h to each base pointer.
struct GemmDesc {
    int64_t M = 0, N = 0, K = 0, kseg = 0;
    const float* A = nullptr; int64_t lda = 0; bool a_kc = true;
    // A stored as 32x32 tiles (blk layout below) with logical row length lda;
    // a_kc then means A(i,k) = X(i,k), else A(i,k) = X(k,i). Causal ranges only.
    bool a_blk = false;
    const float* B = nullptr; int64_t ldb = 0; bool b_kc = true;
    float* C = nullptr; int64_t ldc = 0;
    const float* R = nullptr;
    int64_t batch = 1, H = 1;
    int64_t sAb = 0, sAh = 0, sBb = 0, sBh = 0, sCb = 0, sCh = 0;
    int krange = 0, outmask = 0, mode = 0;
    float scale = 1.0f;
    // Rotary embedding in the epilogue (mode 0, 64-wide heads): output columns
    // [0, rope_cols) are heads of 64 whose pairs (i, i + 32) at position
    // t = row mod rope_T are rotated by cos/sin[t][i] exactly as the rope
    // kernel does. Needs 128-row tiles (128x128 or 128x64: a wave's 64 columns
    // are one head, and a lane holds both elements of its pairs) and no split.
    const float* rope_cos = nullptr;
    const float* rope_sin = nullptr;
    int64_t rope_T = 0, rope_cols = 0;
};

// Tiled square layout of the attention matrices P and dS: element (r, c) of a
// matrix with logical row length ld (a multiple of 32) sits at
// ((r/32)*(ld/32) + c/32)*1024 + (r%32)*32 + c%32, so every 32x32 tile is one
// contiguous 4 KiB run.
inline int64_t blk_index(int64_t ld, int64_t r, int64_t c) {
    return ((r / 32) * (ld / 32) + c / 32) * 1024 + (r % 32) * 32 + (c % 32);
}

// Host-side launch options. They never change a result bit: the split and
// tile choices only change which workgroup computes which chunk.
struct GemmPlan {
    int tile = -1;            // -1 auto, else a tile configuration index
    int split = -1;           // -1 auto, 0 never split K into per-chunk partials, 1 split
    float* scratch = nullptr; // split partial buffer (floats)
    int64_t scratch_floats = 0;
    int simple = 0;           // 1: use the one-thread-per-output reference kernel
};

// Observer of single kernel dispatches: begin runs before a launch, end after
// it with the kernel's name and its algorithmic work (FLOPs, 2 per valid
// multiply-add; or minimal HBM bytes for a kernel without a contraction).
struct LaunchTrace {
    void* ctx = nullptr;
    void (*begin)(void* ctx) = nullptr;
    void (*end)(void* ctx, const char* kernel, double flops, double bytes) = nullptr;
};

// Floats of scratch the split path needs for d (0 when it would not split).
int64_t gemm_split_scratch(const GemmDesc& d, const GemmPlan& p);
// Returns 0, or a negative value when the description is invalid or unsupported.
// tr (may be null) sees every dispatch: the contraction launches (one, or one
// per chunk of a causal range) and the split path's k_fold.
int gemm(const GemmDesc& d, const GemmPlan& p, hipStream_t s, const LaunchTrace* tr = nullptr);
// Two independent contractions: in one launch (one grid, d0's workgroups
// first, then d1's, the second filling the first's part-filled last wave)
// when both are plain (no causal range, mask, batch or rotary epilogue) and
// share the layout, load width and split choice under the automatic plan;
// otherwise one after the other. With split partials, d1's follow d0's in the
// plan's scratch. Bits equal those of two gemm() calls.
int gemm_pair(const GemmDesc& d0, const GemmDesc& d1, const GemmPlan& p, hipStream_t s,
              const LaunchTrace* tr = nullptr);
// FLOPs of the valid multiply-adds of d with k in [kb, ke), all problems.
double gemm_flops(const GemmDesc& d, int64_t kb, int64_t ke);
// Name of the contraction kernel the last gemm() call on this thread launched.
const char* gemm_last_kernel();

// Lower triangle of a batched contraction over a short K (<= 64, one chunk):
// C(i,j) = t(i,j) (times scale when scaled) for j <= i < T, with
// t(i,j) = fma chain over k of A[i*lda + k] * B[j*ldb + k] (mlb_attn.hip).
// blk: C is stored in the tiled layout (ldc = T, a multiple of 32).
// P and D non-null (scaled 0): softmax backward in the epilogue, C(i,j) =
// (P(i,j) * (t(i,j) - D[z*T + i])) * ds_scale, with P laid out as C.
int tri_nt(int64_t T, int64_t K, int64_t batch, int64_t H, const float* A, int64_t lda, int64_t sAb, int64_t sAh,
           const float* B, int64_t ldb, int64_t sBb, int64_t sBh, float* C, int64_t ldc, int64_t sCb, int64_t sCh,
           int scaled, float scale, int blk, const float* P, const float* D, float ds_scale, hipStream_t s);

// Lower-triangle row-strip kernels for 64-wide heads (mlb_attn.hip), S tiled
// [T, T] per head with row length ldS == T. P == nullptr: S = (X . Y) * scale
// for j <= i (the scores, X = q, Y = k). P != nullptr: t = X . Y with X = dO,
// Y = v; S = dS = (P * (t - D_i)) * scale; and dQ = sum over j <= i of
// dS_ij K_j (G1024), stored to dQ. Returns -2 when the shape is not one it
// runs (the caller then uses tri_nt and the general contraction).
bool attn_rows_fits(int64_t T, int64_t hd, int64_t batch, int64_t H, const float* X, int64_t ldx, int64_t sXb,
                    int64_t sXh, const float* Y, int64_t ldy, int64_t sYb, int64_t sYh, const float* S, int64_t ldS,
                    int64_t sSb, int64_t sSh);
int attn_rows(int64_t T, int64_t hd, int64_t batch, int64_t H, const float* X, int64_t ldx, int64_t sXb, int64_t sXh,
              const float* Y, int64_t ldy, int64_t sYb, int64_t sYh, float* S, int64_t ldS, int64_t sSb, int64_t sSh,
              float scale, const float* P, const float* D, const float* K, int64_t ldk, int64_t sKb, int64_t sKh,
              float* dQ, int64_t ldq, int64_t sQb, int64_t sQh, hipStream_t s);

// Causal contraction of 64-wide heads against the tiled attention matrix P
// ([T, T] per head in 32x32 tiles, row length ldp == T): kr 1 C[i] = sum over
// k <= i of P[i][k] B[k], kr 2 C[j] = sum over k >= j of P[k][j] B[k], the
// G1024 rule, mode 0 (mlb_attn.hip); rope_cos/rope_sin ([T][32] tables)
// rotate the output rows back before the store. Returns -2 when the shape is
// not one it runs (hd != 64, T not a multiple of 64, misaligned operands): the
// caller then uses the general contraction.
bool attn_av_fits(int64_t T, int64_t hd, int64_t batch, int64_t H, const float* P, int64_t ldp, int64_t sPb,
                  int64_t sPh, const float* B, int64_t ldb, int64_t sBb, int64_t sBh);
int attn_av(int kr, int64_t T, int64_t hd, int64_t batch, int64_t H, const float* P, int64_t ldp, int64_t sPb,
            int64_t sPh, const float* B, int64_t ldb, int64_t sBb, int64_t sBh, float* C, int64_t ldc, int64_t sCb,
            int64_t sCh, const float* rope_cos, const float* rope_sin, hipStream_t s);

// Row and elementwise kernels (mlb_ops.hip). All return 0 or a negative value
// on invalid sizes; they launch on stream s and never synchronise.
int gather_rows(const int32_t* ids, const float* table, int64_t V, int64_t d, int64_t N, float* out,
                int* err, hipStream_t s);
int rmsnorm_fwd(const float* x, const float* w, int64_t rows, int64_t d, float eps, float* y, float* r,
                hipStream_t s);
// dx = rmsnorm backward; written as out = base + dx (base may be out itself),
// or out = dx when base is null.
int rmsnorm_bwd_dx(const float* dy, const float* x, const float* w, const float* r, int64_t rows,
                   int64_t d, const float* base, float* out, hipStream_t s);
// Gain gradient: per column the contraction over rows of dy * (x * r), chunks of
// 1024 rows. part must hold ceil(rows/1024)*d floats. mode 0 dw = t, 1 dw = dw + t.
int rmsnorm_bwd_dw(const float* dy, const float* x, const float* r, int64_t rows, int64_t d, float* part,
                   float* dw, int mode, hipStream_t s);
// The gain gradient in two parts: the per-chunk column partials of one RMSNorm
// (ceil(rows/1024) * d floats at part), and later, in one launch for nprob
// of them, their folds in chunk order added to base + offs[p] (offs in device
// memory, the partials of problem p at part + p * ceil(rows/1024) * d).
int rmsnorm_bwd_dw_parts(const float* dy, const float* x, const float* r, int64_t rows, int64_t d, float* part,
                         hipStream_t s);
int fold_cols_batched(const float* part, int64_t rows, int64_t d, int64_t nprob, const int64_t* offs, float* base,
                      hipStream_t s);
int rope(float* x, int64_t B, int64_t T, int64_t H, int64_t hd, int64_t ld, const float* cosv,
         const float* sinv, int backward, hipStream_t s);
// In-place causal softmax of rows i of [nbh, T, T] over j <= i (blk: tiled
// layout, T a multiple of 32).
int softmax_causal(float* P, int64_t nbh, int64_t T, int blk, hipStream_t s);
// D[z*T + i] = DOT64 over hd of dO and O rows (head layout as q).
int attn_rowdot(const float* dO, const float* O, int64_t B, int64_t H, int64_t T, int64_t hd, int64_t ld,
                float* D, hipStream_t s);
// dS = (P * (dP - D_i)) * scale in place over dP, j <= i.
int softmax_bwd(const float* P, float* dP, const float* D, int64_t nbh, int64_t T, float scale, int blk,
                hipStream_t s);
int swiglu_fwd(const float* gu, int64_t rows, int64_t F, float* a, hipStream_t s);
int swiglu_bwd(const float* dA, const float* gu, int64_t rows, int64_t F, float* dgu, hipStream_t s);
// Cross-entropy rows (row stride ld >= V): loss_rows written, dl written
// (may alias logits).
int cross_entropy(const float* logits, const int32_t* tg, int64_t N, int64_t V, int64_t ld, float* loss_rows,
                  float* dl, int* err, hipStream_t s);
// out[0] = SUM64(v[0..n)) * mul.
// out[r] = index of the largest of the first V entries of row r * row_step +
// row_off (NaN lowest, ties to the lowest index, 0 if all NaN), r < nsel.
int argmax_rows(const float* x, int64_t nsel, int64_t row_step, int64_t row_off, int64_t ld, int64_t V,
                int32_t* out, hipStream_t s);
int sum64_scaled(const float* v, int64_t n, float mul, float* out, hipStream_t s);
// Embedding-gradient scatter. For every row v that appears in ids, in order of
// increasing position n: acc = init(v); acc = acc + dh[n]; then
// dst[v] = acc (mode 0) or dst[v] = dst[v] + acc (mode 1). init(v) is +0 when
// src_init is null, else src_init[v]. keys must hold embed_key_slots(N)
// uint64 values; N is at most EMBED_MAX_POSITIONS.
constexpr int64_t EMBED_MAX_POSITIONS = 65536;
int64_t embed_key_slots(int64_t N);
int embed_scatter(const int32_t* ids, const float* dh, int64_t N, int64_t d, int64_t V,
                  const float* src_init, float* dst, int mode, uint64_t* keys, hipStream_t s);
// The two halves of embed_scatter: the key sort (which depends on the ids
// only, so it can run early, on another stream) and the segment walk over
// keys that embed_sort wrote for the same ids, N and V.
int embed_sort(const int32_t* ids, int64_t N, int64_t V, uint64_t* keys, hipStream_t s);
int embed_scatter_sorted(const uint64_t* keys, const float* dh, int64_t N, int64_t d, int64_t V,
                         const float* src_init, float* dst, int mode, hipStream_t s);
// out = out + x elementwise (n floats).
int add_inplace(float* out, const float* x, int64_t n, hipStream_t s);
int adamw(float* p, float* g, float* m, float* v, int64_t n, float lr, float b1, float b2, float eps,
          float wd, float bc1, float bc2, hipStream_t s);
int exp_array(const float* x, float* y, int64_t n, int which, hipStream_t s);
int fill_zero(float* x, int64_t n, hipStream_t s);
int mfma_probe(int variant, const float* A, const float* B, const float* C, float* D, int64_t nwaves,
               hipStream_t s);

}  // namespace mlb
