/*
 * mlb.h - C ABI of the bitwise-reproducible FP32 training step (MI355X, gfx950).
 *
 * One training step of a Llama-style decoder - embedding lookup, pre-norm
 * RMSNorm, rotary causal attention, SwiGLU, untied (or tied) output table,
 * cross-entropy, backward, fixed-order accumulation of micro-batch gradients
 * and AdamW - computed under the frozen numerical profile MLB-P1, so that every
 * output bit depends only on the inputs. The model and optimiser follow the
 * MojoLearn 162M model card ("Compared with GPT-3 Small" and "Training"
 * tables); the bit-identity contract follows the mojolearn PyPI page ("What
 * bitwise identity means": reduction order, partitioning, FMA policy, flush
 * seams, transcendental spellings and tie rules are fixed, and a request that
 * cannot be met is refused by name instead of falling back).
 *
 * Memory: the caller owns one device arena (mlb_workspace_bytes) and the HIP
 * stream; the library owns the handle, a 64-byte pinned host staging buffer and
 * one side stream (see mlb_set_overlap). Every call is ordered on the caller's
 * stream. mlb_forward_loss, mlb_save,
 * mlb_load and mlb_read synchronise that stream; the others do not.
 * A handle is not thread-safe. Errors are returned as negative mlb_status
 * values; mlb_last_error_message() (thread-local) gives the detail.
 * NaN and Inf are not checked: they are deterministic bit patterns too, but
 * NaN payload bits are not part of the contract.
 */
#ifndef MLB_H
#define MLB_H
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

#define MLB_ABI_VERSION 1u
#define MLB_PROFILE_VERSION 1u /* MLB-P1 */

typedef int32_t mlb_status;
#define MLB_OK 0
#define MLB_E_INVALID_ARG (-1)      /* null pointer, bad size, bad enum */
#define MLB_E_UNSUPPORTED (-2)      /* named refusal: device or config outside the profile */
#define MLB_E_DEVICE (-3)           /* a HIP runtime call or kernel launch failed */
#define MLB_E_ARENA_TOO_SMALL (-4)
#define MLB_E_BAD_TOKEN (-5)        /* an input or target id outside [0, vocab) */
#define MLB_E_STATE (-6)            /* call order violated */
#define MLB_E_CORRUPT (-7)          /* checkpoint bytes fail a digest or size check */
#define MLB_E_PROFILE_MISMATCH (-8) /* checkpoint written under another format or profile */
#define MLB_E_CONFIG_MISMATCH (-9)  /* checkpoint written for another model config */
#define MLB_E_IO (-10)              /* host buffer too small */

/* Model shape and optimiser constants. abi_version must be MLB_ABI_VERSION.
 * d_model = n_heads * head_dim; head_dim even; d_model and ffn_hidden multiples
 * of 32; batch * seq_len <= 65,536 tokens per micro-batch. */
typedef struct mlb_config {
    uint32_t abi_version;
    uint32_t vocab, d_model, n_layers, n_heads, head_dim, ffn_hidden, tied, batch, seq_len;
    float rope_theta, rms_eps, beta1, beta2, adam_eps, weight_decay;
} mlb_config;

typedef struct mlb_model mlb_model;

typedef enum mlb_which { MLB_PARAMS = 0, MLB_GRAD = 1, MLB_ADAM_M = 2, MLB_ADAM_V = 3 } mlb_which;

/* Parameter count in canonical order: E_in [V,d]; per layer attn_norm [d],
 * Wq, Wk, Wv, Wo [d,d], mlp_norm [d], Wg, Wu [F,d], Wd [d,F]; W_out [V,d] when
 * untied. Linear weights are [out_features, in_features] (model card, "Anywhere
 * else: safetensors + PyTorch"). Returns -1 for an invalid config. */
int64_t mlb_param_count(const mlb_config* cfg);

/* Device bytes the arena must hold for cfg (params, gradient accumulator,
 * both moments, stored activations and scratch of one micro-batch of
 * batch x seq_len tokens; the model card's "Training" table runs 4 x 2,048).
 * MLB_E_INVALID_ARG for an invalid config, MLB_E_UNSUPPORTED for a shape the
 * kernels are not built for. Touches no device. */
mlb_status mlb_workspace_bytes(const mlb_config* cfg, size_t* bytes);

/* Creates a model on the current HIP device. init_params_host: host float32
 * array of mlb_param_count(cfg) values (step-0 parameters, canonical order),
 * read during the call; or NULL, and the step-0 parameters are drawn from seed
 * (model card "Training" table: N(0, 0.02) weights, norm gains 1 + N(0, 0.02))
 * by the profile's own generator: parameter k takes SplitMix64 outputs 2k and
 * 2k+1 of the stream started at seed (Steele, Lea and Flood 2014), u1 =
 * (first >> 11 plus 1) * 2^-53, u2 = (second >> 11) * 2^-53, z = sqrt(-2 log u1)
 * * cos(2 pi u2) in binary64 (Box-Muller), value 0.02 z (gains 1 + 0.02 z)
 * rounded once to binary32. dev_arena: caller-owned device memory of
 * arena_bytes, 256-byte aligned, untouched by anything else while the model
 * lives. hip_stream: a hipStream_t (may be null). Moments and the gradient
 * accumulator start at +0, step 0. Refuses a device that is not gfx950
 * (MLB_E_UNSUPPORTED). */
mlb_status mlb_init(const mlb_config* cfg, uint64_t seed, const float* init_params_host, void* dev_arena,
                    size_t arena_bytes, void* hip_stream, mlb_model** out);

/* Forward pass and loss of one micro-batch (model card, "Training" table: the
 * loss is the mean cross-entropy over the 4 x 2,048 tokens of a shard; the
 * mojolearn project page counts cross-entropy in the verified chain):
 * d_inputs and d_targets are device int32 arrays of batch*seq_len ids
 * (row-major [batch, seq_len]; targets are the next ids), read before the call
 * returns. Writes the shard loss to *out_loss_host and keeps the activations
 * for mlb_backward. Synchronises the stream. An id outside [0, vocab) gives
 * MLB_E_BAD_TOKEN (kernels read no table row for it) and no usable forward;
 * the state is unchanged. */
mlb_status mlb_forward_loss(mlb_model* m, const int32_t* d_inputs, const int32_t* d_targets, float* out_loss_host);

/* Inference forward of one batch of [batch, seq_len] device int32 ids (model
 * card, "Using the model": forward-only logits and loss). d_logits (device,
 * may be NULL) receives the logits [batch*seq_len, vocab] row-major; with
 * d_targets (device, may be NULL) the mean loss goes to *out_loss_host (both
 * or neither). The same arithmetic as the training forward: the loss equals
 * mlb_forward_loss's bit for bit. Keeps nothing for a backward; MLB_E_STATE
 * while a training forward awaits its backward. Synchronises the stream. */
mlb_status mlb_infer(mlb_model* m, const int32_t* d_inputs, const int32_t* d_targets, float* d_logits,
                     float* out_loss_host);
/* Greedy next token of every sequence of the batch after `position`
 * (0 <= position < seq_len): the index of the largest logit at that position,
 * NaN ranking below every number and ties going to the lowest index (0 when
 * every logit is NaN). Causality makes the ids after `position` irrelevant, so
 * a prompt of p ids continues with position p - 1. next_host receives batch
 * int32 values. Synchronises the stream. */
mlb_status mlb_greedy_next(mlb_model* m, const int32_t* d_inputs, int position, int32_t* next_host);

/* Backward of the last forward; folds its gradient g into the accumulator,
 * G = G + g (call order = micro-batch order). The model card's "Training"
 * table sums the 64 shard gradients of a step in a fixed order; this call is
 * one term of that sum, and the order of calls is the order of the sum.
 * MLB_E_STATE without a successful forward since the last backward (a second
 * backward of one forward adds nothing and is refused). */
mlb_status mlb_backward(mlb_model* m);

/* One AdamW step with learning rate lr on the accumulated G, then G = +0
 * (model card, "Training" table: AdamW with beta (0.9, 0.95), eps 1e-8,
 * weight decay 0.1; the learning rate of each step comes from the caller,
 * who follows the table's warmup and cosine schedule). Step t = previous + 1;
 * the bias corrections are RN(1 - beta^t) from a binary64 product. MLB_E_STATE
 * when no backward ran since the last step; the state is then unchanged. */
mlb_status mlb_adamw_step(mlb_model* m, float lr);

/* Exact state bytes (MLBC v1; model card, "Using the model": a checkpoint
 * that a trainer is restored from and whose load verifies every array digest):
 * 256-byte header (magic "MLBCKPT1", format, profile, config, step, parameter
 * count, SHA-256 of params, m, v and of the header itself) followed by params,
 * m and v as little-endian float32. The bytes are a pure function of the
 * state. host_buf NULL: *len = size only. MLB_E_STATE while gradients are
 * pending (between a backward and its AdamW step); MLB_E_IO if cap is too
 * small (*len still receives the size). The caller owns host_buf. */
mlb_status mlb_save(const mlb_model* m, void* host_buf, size_t cap, size_t* len);

/* Restores params, moments and step from mlb_save bytes (model card, "Using
 * the model": restore from checkpoint bytes, verifying every array digest).
 * Verifies magic, format and profile (MLB_E_PROFILE_MISMATCH), the header
 * digest, padding, size and every array digest (MLB_E_CORRUPT) and the config
 * (MLB_E_CONFIG_MISMATCH) before touching the state; a refused load leaves
 * the state as it was. A successful load clears G and any pending forward.
 * Synchronises the stream; host_buf is only read. */
mlb_status mlb_load(mlb_model* m, const void* host_buf, size_t len);

/* Copies a state array (mlb_param_count floats, canonical order) to host
 * memory, for the bit-for-bit comparisons the mojolearn PyPI page ("What
 * bitwise identity means") makes the test of the identity claim.
 * MLB_E_IO if bytes is smaller than the array; MLB_E_INVALID_ARG for an
 * unknown array. Synchronises the stream. */
mlb_status mlb_read(const mlb_model* m, mlb_which which, void* host_dst, size_t bytes);

/* The parameters as a safetensors file image, for running the weights in
 * other frameworks (model card, "Anywhere else: safetensors + PyTorch": the
 * file holds the checkpoint's parameter array byte for byte, linear weights
 * [out_features, in_features]). Layout: u64 little-endian header length, a
 * JSON header (padded with spaces to a multiple of 8 bytes) naming each tensor
 * of the canonical order (E_in, l<i>.attn_norm, l<i>.Wq, Wk, Wv, Wo,
 * l<i>.mlp_norm, l<i>.Wg, Wu, Wd, W_out) as F32 with its shape and byte range,
 * with the shape constants under "__metadata__"; then params_host's
 * mlb_param_count(cfg) floats unchanged. Host-only: no device is touched.
 * buf == NULL: *len receives the size. Errors: MLB_E_INVALID_ARG (config,
 * null params), MLB_E_IO (cap too small). */
mlb_status mlb_safetensors(const mlb_config* cfg, const float* params_host, void* buf, size_t cap, size_t* len);

/* Copies an activation of the last forward to host memory (stage ids: 0 layer
 * input, 1 attention-norm output, 2 its 1/rms, 3 q|k|v after rotation, 4 P,
 * 5 attention output, 6 mid-layer residual, 7 MLP-norm output, 8 its 1/rms,
 * 9 g|u, 10 SwiGLU output, 11 final hidden, 12 d-logits, 13 per-row losses;
 * 14 and 15 the rotary cos and sin tables [seq_len, head_dim/2] the model
 * uploaded at mlb_init, available before any forward).
 * Layouts are row-major; P is dense [batch*heads, T, T] with +0 above the
 * diagonal; d-logits are [tokens, vocab]. *count receives the element count;
 * host_dst may be NULL to query it. */
mlb_status mlb_read_stage(const mlb_model* m, int stage, int layer, void* host_dst, size_t bytes, size_t* count);

/* Stage identity card (mojolearn PyPI page, "What bitwise identity means":
 * per-stage hashes as a check of the identity claim): a tag ("L<layer>.<name>" for
 * per-layer stages, else the name), the dtype and element count, and the
 * SHA-256 of the exact bytes mlb_read_stage returns (little-endian float32).
 * Two runs agree on a stage exactly when their cards agree, so comparing cards
 * in computation order names the first stage where two runs diverge. */
typedef struct mlb_card {
    char tag[32];
    char dtype[8];
    uint64_t count;
    uint8_t sha256[32];
} mlb_card;
mlb_status mlb_stage_card(const mlb_model* m, int stage, int layer, mlb_card* out);
/* Card of a state array (params, accumulated gradient, AdamW moments). */
mlb_status mlb_state_card(const mlb_model* m, mlb_which which, mlb_card* out);

/* Stream overlap of the backward pass (default off). When on, the work that
 * only feeds the gradient accumulator (weight-gradient contractions, norm-gain
 * gradients, the embedding scatter) runs on a library-owned second stream of
 * default priority, concurrently with the input-gradient chain on the caller's
 * stream, and joins the caller's stream before mlb_backward returns; off runs
 * everything on the caller's stream. The bits are the same either way (each
 * accumulator entry receives one addition per micro-batch, in call order).
 * Per-launch statistics of overlapping kernels include each other's time.
 * MLB_E_STATE between a forward and its backward. Synchronises the stream. */
mlb_status mlb_set_overlap(mlb_model* m, int on);

/* Launch statistics (this library's own tracing). When enabled, every kernel
 * launch of the step is bracketed by HIP events on the model's stream and
 * aggregated per call site: launch count, total milliseconds, algorithmic
 * FLOPs (2 per valid multiply-add of a contraction) and algorithmic HBM bytes
 * (minimal reads + writes of a row or elementwise kernel). Enabling clears
 * the aggregates. mlb_stats_read synchronises the stream and copies up to cap
 * entries; *n receives the number of sites. */
typedef struct mlb_stat {
    char site[48];
    char kernel[96];
    int64_t launches;
    double ms, flops, bytes;
} mlb_stat;
mlb_status mlb_stats_enable(mlb_model* m, int on);
mlb_status mlb_stats_read(mlb_model* m, mlb_stat* out, int cap, int* n);
/* Restricts the statistics to the call sites named in sites (comma-separated
 * site names as mlb_stats_read reports them); NULL or "" times every site.
 * Each timed dispatch costs two event records on the stream, so timing a few
 * sites disturbs the step far less than timing all of them. */
mlb_status mlb_stats_sites(mlb_model* m, const char* sites);

uint64_t mlb_step(const mlb_model* m);
mlb_status mlb_destroy(mlb_model* m);
const char* mlb_status_name(mlb_status s);
const char* mlb_last_error_message(void);
uint32_t mlb_profile_version(void);

#ifdef __cplusplus
}
#endif
#endif
