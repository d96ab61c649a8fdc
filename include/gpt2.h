/*
 * gpt2.h -- C ABI of the MI355X (gfx950) GPT-2 training-step library.
 *
 * One call sequence is one training step ("Karpathy's four-hour GPT-2
 * reproduction in one post", parts 1 and 3; "Reproducing GPT-2 (124M) cheaply
 * with llm.c", training run):
 *
 *     for k in 0..K-1:  gpt2_forward(h, ids_k, targets_k, ...);  gpt2_backward(h, k, K);
 *     gpt2_adamw_step(h, step, lr, ...);
 *
 * Ownership.  The caller owns every device buffer (parameters, their bf16
 * copy, gradients, Adam moments, workspace) and the stream; the library keeps
 * raw pointers and a small host handle, never allocates or frees device
 * memory, and enqueues all work on the caller's stream.  Nothing synchronises
 * except gpt2_sync_status.  Device pointers must be 256-byte aligned.
 *
 * Errors.  Every int-returning call returns GPT2_OK (0) or a negative
 * GPT2_ERR_* code and never aborts or throws.  Errors found on the device
 * (token ids out of range, a non-finite gradient norm) are deferred: they are
 * recorded in device flags and reported by the next gpt2_sync_status.
 * gpt2_last_error(h) gives a message for the last host-side failure.
 *
 * Shapes.  n_embd % n_head == 0, head_dim = n_embd / n_head in {32, 64},
 * n_embd / 128 in {1, 2, 3, 4, 6, 8, 12, 16} (the LayerNorm row widths the
 * library is built for), padded_vocab_size % 128 == 0, vocab_size <=
 * padded_vocab_size <= 65536 (the cross-entropy row held by one block),
 * T % 64 == 0 and T <= max_seq_len, B*T % 128 == 0.  A config outside these
 * is refused by every call that takes one (GPT2_ERR_CONFIG), B or T outside
 * them with GPT2_ERR_SHAPE, before any device work.
 */
#ifndef GPT2_MI355X_H
#define GPT2_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Model shape, after GPTConfig(vocab_size, block_size, n_layer, n_head,
 * n_embd) of "A small GPT that writes fairy tales" (lm-book, code excerpt);
 * block_size is max_seq_len.  padded_vocab_size rounds the tied matrix up for
 * speed ("Karpathy's four-hour GPT-2 reproduction in one post", part 2, the
 * last speed-up); padded rows never enter the softmax. */
typedef struct gpt2_config {
  int32_t vocab_size;
  int32_t padded_vocab_size;
  int32_t n_layer;
  int32_t n_head;
  int32_t n_embd;
  int32_t max_seq_len;
} gpt2_config_t;

/* Precision of activations and matmul operands.  GPT2_FP32: everything fp32
 * (parity mode).  GPT2_BF16: bf16 matmul/attention operands and saved
 * activations with fp32 accumulation; fp32 master weights, gradients, Adam
 * moments, residual stream, LayerNorm statistics, softmax and loss
 * ("Reproducing GPT-2 (124M) cheaply with llm.c", setup: mixed precision). */
typedef enum { GPT2_FP32 = 0, GPT2_BF16 = 1 } gpt2_precision_t;

/* Flag OR'd into the precision argument of gpt2_workspace_bytes and gpt2_init:
 * activation recompute for the MLP (llm.c's -r option, "Reproducing GPT-2
 * (124M) cheaply with llm.c", training command flags).  Each layer keeps only
 * the MLP pre-activation (in the activation type) instead of GELU' and the
 * GELU output; two GELU-output buffers serve all layers (by layer parity) and
 * gpt2_backward rebuilds a layer's from the pre-activation before its MLP
 * weight gradient.  The workspace shrinks by (n_layer - 2) * B * T * 4 *
 * n_embd activation elements (n_layer >= 2); the step costs one extra
 * elementwise pass per layer.
 * The activation is taken from the rounded pre-activation in this mode, so
 * bf16 results differ from the default mode within rounding (fp32 results
 * are identical). */
#define GPT2_RECOMPUTE_GELU 0x100

/* Flag OR'd into the precision (GPT2_BF16 only): the forward's matmuls (qkv,
 * attention projection, MLP up and down, tied head) take FP8 E4M3 operands on
 * gfx950's FP8 matrix cores ("Reproducing GPT-2 (124M) cheaply with llm.c",
 * where FP8 training is announced as the next step), accumulating in fp32.
 * Scaling is per row: each activation row (token) and each weight row
 * (output channel) is stored as E4M3 values times one fp32 scale,
 * scale = max |row| / 448.  The backward stays bf16 (on the bf16 activations
 * and weights).  The workspace grows by the FP8 weight copy (one byte per
 * parameter), its row scales and one FP8 activation buffer of B*T*4*n_embd
 * bytes.  Needs n_embd % 256 == 0 and n_embd <= 1024 (rows of at most 4096
 * values are quantized); otherwise gpt2_workspace_bytes and gpt2_init return
 * GPT2_ERR_ARG. */
#define GPT2_FP8_FWD 0x200

enum {
  GPT2_OK = 0,
  GPT2_ERR_CONFIG = -1,      /* shape constraints above violated */
  GPT2_ERR_SHAPE = -2,       /* B or T outside what the handle was planned for */
  GPT2_ERR_ARG = -3,         /* null / misaligned pointer, bad step or micro-step index */
  GPT2_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  GPT2_ERR_TOKEN_RANGE = -5, /* deferred: an input id or target outside [0, vocab_size) */
  GPT2_ERR_NONFINITE = -6,   /* deferred: gradient norm was NaN/Inf; the update was skipped */
  GPT2_ERR_WORKSPACE = -7    /* workspace smaller than gpt2_workspace_bytes */
};

/* One tensor of the flat parameter layout.  The token embedding is also the
 * output layer ("Karpathy's four-hour GPT-2 reproduction in one post",
 * part 1); linear weights are stored [out, in].  decay = 1 for 2-D tensors
 * (matmul weights and embeddings take weight decay, part 3), 0 for biases and
 * LayerNorm gains/biases.  The decayed tensors form one prefix of the layout. */
typedef struct gpt2_tensor_desc {
  char name[32];
  int64_t offset; /* in elements from the start of the flat buffer */
  int32_t rows;
  int32_t cols; /* 0 for 1-D tensors */
  int32_t decay;
} gpt2_tensor_desc_t;

typedef struct gpt2_handle gpt2_t;

/* ---- host-only queries (no device needed) ---------------------------------- */

/* Stored parameter count Vp*C + Tmax*C + L*(12C^2 + 13C) + 2C, or a negative
 * error code when the config is invalid. */
int64_t gpt2_num_params(const gpt2_config_t* cfg);

/* Number of parameters that take weight decay (the decayed prefix). */
int64_t gpt2_num_decay_params(const gpt2_config_t* cfg);

/* Writes up to cap descriptors into out; returns the number of tensors
 * (2 + 12*n_layer + 2) or a negative error code. */
int gpt2_param_layout(const gpt2_config_t* cfg, gpt2_tensor_desc_t* out, int cap);

/* Device workspace (bytes) gpt2_init needs for micro-batch B x T in the given
 * precision: saved activations, logits, backward scratch and reduction
 * partials.  Negative error code on invalid arguments. */
int64_t gpt2_workspace_bytes(const gpt2_config_t* cfg, int B, int T, int precision);

/* Checks cfg/B/T against the shape constraints; GPT2_OK or an error code. */
int gpt2_check_shapes(const gpt2_config_t* cfg, int B, int T);

/* ---- lifecycle ----------------------------------------------------------------- */

/* Creates a handle for micro-batches of exactly B x T tokens.
 *   params    fp32 [N] master parameters (layout above), read and updated
 *   params_lp bf16 [N] copy used as matmul operand in GPT2_BF16, NULL in GPT2_FP32
 *   grads     fp32 [N] gradient accumulator, written by gpt2_backward
 *   adam_m, adam_v  fp32 [N] first/second moments, updated by gpt2_adamw_step
 *   workspace at least gpt2_workspace_bytes(cfg, B, T, precision) bytes
 *   stream    hipStream_t to enqueue on (NULL = the null stream)
 * Enqueues only the clearing of the deferred status flags (16 bytes of the
 * workspace).  After writing params, call gpt2_refresh_params. */
int gpt2_init(gpt2_t** out, const gpt2_config_t* cfg, int precision, int B, int T, float* params, void* params_lp,
              float* grads, float* adam_m, float* adam_v, void* workspace, int64_t workspace_bytes, void* stream);

/* Frees the host handle (no device memory is touched). */
void gpt2_destroy(gpt2_t* h);

/* Re-derives the bf16 parameter copy from the fp32 master parameters
 * (needed once after the caller fills params; AdamW keeps it current). */
int gpt2_refresh_params(gpt2_t* h);

/* Replaces the stream later calls enqueue on.
 *
 * Graph capture: gpt2_forward, gpt2_eval and gpt2_backward enqueue kernels
 * and event records/waits only (no allocation, memset, copy or host
 * synchronisation), so a caller may capture one micro-step into a HIP graph
 * by setting its capturing stream here first: the handle's second stream
 * joins the capture through an event recorded on that stream and is joined
 * back before each call returns.  A graph freezes the call's arguments (the
 * input and loss pointers, micro_step > 0 or not); replays read whatever the
 * caller's input buffers hold then.  gpt2_adamw_step takes the step and
 * learning rate by value, so it stays outside a graph replayed over steps.
 * Set the stream back to the one replays and later calls use afterwards. */
int gpt2_set_stream(gpt2_t* h, void* stream);

/* Overlap (default on): gpt2_backward runs the tied head's and each layer's
 * four weight-gradient products and the layers' partial-sum reductions, and
 * gpt2_forward the sort of the token ids for the embedding backward, on a
 * second stream owned by the handle (created by gpt2_init, default priority),
 * ordered by events after their inputs and before anything that overwrites
 * those inputs; both calls return with all of their work ordered before later
 * work on the caller's stream, so the caller sees one stream either way.
 * enable = 0 runs everything on the caller's stream (same results, bit for
 * bit; used to time kernels in isolation).  GPT2_ERR_ARG on a null handle. */
int gpt2_set_overlap(gpt2_t* h, int enable);

/* ---- the step ---------------------------------------------------------------------- */

/* Forward pass and loss of one micro-batch (the GPT-2 forward of
 * "Karpathy's four-hour GPT-2 reproduction in one post", part 1: token +
 * position embedding, pre-LN blocks of causal multi-head attention and a
 * tanh-GELU MLP, final LN, tied head, softmax cross-entropy over the real
 * vocabulary; loss in nats per token, "A small GPT that writes fairy tales",
 * Problem 3).
 *   d_idx, d_targets  int32 [B*T] device, row-major [B][T]; targets may be NULL
 *                     (then no loss is computed and gpt2_backward is not allowed)
 *   d_loss            fp32 [1] device or NULL: mean loss over the B*T positions
 *   d_loss_rows       fp32 [B*T] device or NULL: per-position loss
 * Ids outside [0, vocab_size) raise GPT2_ERR_TOKEN_RANGE at the next
 * gpt2_sync_status (the gather reads row 0 instead). */
int gpt2_forward(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, float* d_loss, float* d_loss_rows);

/* Forward-only evaluation of one micro-batch: the same forward and loss as
 * gpt2_forward (bit for bit), without what only the backward needs (gelu' of
 * the MLP pre-activation, the embedding sort, dlogits), so gpt2_backward may
 * not follow it.  The validation readouts of "A small GPT that writes fairy
 * tales" (training log and Problem 3) are host arithmetic on its mean loss:
 * perplexity = exp(loss), bits per byte = loss / ln 2 / (bytes per token).
 *   d_idx, d_targets  int32 [B*T] device; targets required (GPT2_ERR_ARG if NULL)
 *   d_loss, d_loss_rows  as for gpt2_forward
 * Token-range errors as for gpt2_forward. */
int gpt2_eval(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, float* d_loss, float* d_loss_rows);

/* Device pointer to the fp32 residual stream [B*T, n_embd] (row-major, rows
 * in [B][T] order) that the last gpt2_forward or gpt2_eval saved at the input
 * of block `layer`: for 0 <= layer < n_layer the input of that block's first
 * LayerNorm, for layer == n_layer the input of the final LayerNorm.  Layer 0
 * is the embedding output x0[b, t] = wte[id[b, t]] + wpe[t] ("Karpathy's
 * four-hour GPT-2 reproduction in one post", part 1: token plus position
 * embedding), one fp32 addition per element.  The memory is part of the
 * workspace: read-only for the caller, valid until the next forward on the
 * handle, ordered on the handle's stream.  GPT2_ERR_ARG for a null handle or
 * out pointer, or a layer outside [0, n_layer]. */
int gpt2_residual(gpt2_t* h, int layer, const float** out);

/* Backward pass of the last forward.  Adds (1/grad_accum_steps) times the
 * gradient of that micro-batch's mean loss into grads; micro_step == 0
 * overwrites grads instead ("Karpathy's four-hour GPT-2 reproduction in one
 * post", part 3: each micro-batch loss is divided by the number of
 * micro-batches).  0 <= micro_step < grad_accum_steps. */
int gpt2_backward(gpt2_t* h, int micro_step, int grad_accum_steps);

/* Global gradient-norm clipping and AdamW ("Karpathy's four-hour GPT-2
 * reproduction in one post", part 3: betas (0.9, 0.95), eps 1e-8, clip 1.0,
 * weight decay on 2-D tensors only).  With n = ||grads||_2, grads are scaled
 * by clip/n when n > clip; then for step t >= 1:
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   p -= lr * ((m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps) + wd*[2-D]*p)
 * and the bf16 copy is rewritten.  d_grad_norm (fp32 [1] device, or NULL)
 * receives n before clipping.  A non-finite n skips the update and raises
 * GPT2_ERR_NONFINITE at the next gpt2_sync_status.  grads are not modified
 * (the clip factor is applied on the fly). */
int gpt2_adamw_step(gpt2_t* h, int step, float lr, float beta1, float beta2, float eps, float weight_decay,
                    float grad_clip, float* d_grad_norm);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight training loops, harnesses that forbid hipMalloc): the same
 * clip + AdamW update as gpt2_adamw_step, on flat buffers the caller passes,
 * with no handle, no workspace and no allocation.  Its scratch (the global
 * norm's 1024 fp64 partial sums, the clip factor and the skip flag: 8448
 * bytes) is a fixed file-scope device array of the library, one copy per GPU,
 * held until the process ends.
 *   params    fp32 [n], updated in place; params_lp bf16 [n] copy rewritten
 *             from the updated params, or NULL
 *   grads     fp32 [n], read only (the clip factor is applied on the fly)
 *   adam_m, adam_v  fp32 [n] moments, updated in place
 *   n         multiple of 4, 4 <= n <= 2^36; the first n_decay elements
 *             (a multiple of 4, <= n) take weight decay
 *   d_grad_norm  fp32 [1] device, required: receives the pre-clip norm; a
 *             non-finite value there means the update was skipped
 *   stream    hipStream_t (NULL = the null stream); nothing synchronises
 * Pointers must be 16-byte aligned (params_lp 8-byte).  GPT2_ERR_ARG for bad
 * arguments or sizes beyond the limit, before any device work; GPT2_ERR_HIP
 * if a launch fails.  Every call on one GPU uses that GPU's scratch array, so
 * calls that overlap on one GPU (concurrent streams or threads) race; calls
 * ordered on one stream do not. */
int gpt2_adamw_step_noalloc(float* params, void* params_lp, const float* grads, float* adam_m, float* adam_v,
                            int64_t n, int64_t n_decay, int step, float lr, float beta1, float beta2, float eps,
                            float weight_decay, float grad_clip, float* d_grad_norm, void* stream);

/* Synchronises the stream and returns (then clears) the deferred device error
 * flags: GPT2_OK, GPT2_ERR_TOKEN_RANGE, GPT2_ERR_NONFINITE or GPT2_ERR_HIP. */
int gpt2_sync_status(gpt2_t* h);

/* Message for the last host-side error on h (never NULL). */
const char* gpt2_last_error(gpt2_t* h);

/* Static description of an error code. */
const char* gpt2_strerror(int code);

/* ---- kernel timing (for measurement) ----------------------------------------------- */

/* Number of timeable kernels, and the name of kernel id in [0, count):
 * gemm_nt_store, gemm_nt_gelu, gemm_nt_resid, gemm_nn_store, gemm_nn_gelu_bwd,
 * gemm_tn_f32 (per-layer weight gradients), gemm_tn_lmhead (weight gradient of
 * the tied output layer), attn_fwd, attn_bwd_dkv, attn_bwd_dq, cross_entropy,
 * layernorm_fwd, layernorm_bwd, adamw.  NULL for an invalid id. */
int gpt2_kernel_count(void);
const char* gpt2_kernel_name(int kernel_id);

/* Enables (1) or disables (0) event timing of one kernel: while enabled, each
 * launch of that kernel is bracketed by hipEventRecord on the library's
 * stream.  Enabling another id replaces the previous one. */
int gpt2_timing_enable(gpt2_t* h, int kernel_id, int enable);

/* Synchronises the stream, then returns the summed milliseconds, the number of
 * timed launches and their summed algorithmic FLOPs (2*M*N*K per matmul;
 * 4*hd per causal query-key pair and head for the attention passes; 0 for
 * memory-bound kernels) since the last read, and resets the counters. */
int gpt2_timing_read(gpt2_t* h, double* total_ms, int64_t* launches, double* flops);

#ifdef __cplusplus
}
#endif

#endif /* GPT2_MI355X_H */
