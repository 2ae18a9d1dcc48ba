/*
 * nc.h -- C ABI of the MI355X (gfx950) forward/backward library for the
 * nanochat-style decoder-only Transformer (the "d20" model).
 *
 * What the library computes is one training step's forward pass, loss and
 * backward pass of the model the nanochat speedrun walkthrough pretrains
 * (lyylswood.com page "100 dollars, 8000 lines of code: a hand-built ChatGPT
 * clone"): a Llama-like pre-norm decoder-only Transformer (introduction:
 * the author's note on the architecture), trained on next-token prediction
 * over packed rows (section Pretraining), 20 layers of 1280 channels and
 * 10 heads of dimension 128 at d20 (Pretraining, the printed model summary),
 * with no biases and no RMSNorm parameters and separate embedding and
 * unembedding tensors (Pretraining, optimiser paragraph), reporting the loss
 * also as bits per byte (Pretraining, bits-per-byte paragraph).
 *
 * Model, per row of T tokens (d = n_head * head_dim, F = d_ff, V = vocab):
 *   x = E[idx]
 *   per layer:  a = rms(x);  q,k,v = a Wq^T, a Wk^T, a Wv^T
 *               q,k = rotary(q,k)   (pairs (2i,2i+1), angle t*base^(-2i/Q))
 *               o = causal_softmax(q k^T / sqrt(Q)) v
 *               x = x + o Wo^T
 *               m = rms(x);  h = m W1^T;  x = x + relu(h)^2 W2^T
 *   xf = rms(x);  z = xf U^T;  ce[t] = logsumexp(z[t]) - z[t, target[t]]
 *   rms(x) = x / sqrt(mean(x^2) + eps)
 *   loss = sum(ce) / n_valid;  bpb = sum(ce) / (ln 2 * sum(bytes[target]))
 * A target of -1 is ignored (no loss, no bytes, no gradient).  With no
 * valid target at all, loss and bpb are 0 and every gradient is 0.
 *
 * Conventions
 *  - Every pointer argument named as device memory must point to memory of
 *    the GPU that is current when nc_init is called.  The caller owns every
 *    buffer, the workspace and the stream; the library allocates no device
 *    memory and frees nothing it did not create (nc_ctx is a host object).
 *  - Parameters (and their gradients) are one flat buffer each, in this
 *    order: E [V,d]; for each layer Wq, Wk, Wv, Wo [d,d], W1 [F,d], W2 [d,F];
 *    U [V,d].  Each matrix is row-major [out, in] and used as y = x W^T.
 *    Wq, Wk, Wv are adjacent, forming one [3d, d] matrix.  In block-only mode
 *    the buffer holds one layer's six tensors.
 *  - Parameters and activations are stored in the configuration's dtype
 *    (fp32 or bf16); every accumulation inside a kernel is fp32; row
 *    statistics are fp32; gradients of parameters are always fp32.
 *  - Activations are row-major [batch, seq_len, features] (token-major).
 *  - Every call enqueues its work on the context's stream and returns
 *    before the GPU finishes.  Outputs are valid once the stream is
 *    synchronised.  Host-only queries make no HIP call.
 *  - Host-side validation happens first; on failure nothing is enqueued.
 *  - A context is not thread-safe: use one context per stream.
 */
#ifndef NC_H
#define NC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NC_OK = 0,
  NC_ERR_INVALID_ARG = -1,   /* null pointer, bad enum value, bad flag */
  NC_ERR_SHAPE = -2,         /* dims not positive / not multiples of 64 / d != H*Q */
  NC_ERR_WORKSPACE = -3,     /* workspace too small or misaligned */
  NC_ERR_STATE = -4,         /* call out of order (e.g. backward before forward) */
  NC_ERR_HIP = -5,           /* a HIP call or kernel launch failed; see nc_last_error */
  NC_ERR_UNSUPPORTED = -6    /* valid but not supported by this library */
} nc_status;

typedef enum { NC_DTYPE_F32 = 0, NC_DTYPE_BF16 = 1 } nc_dtype;

enum {
  NC_FLAG_BLOCK_ONLY = 1,     /* one layer: no embedding, no head, no loss */
  NC_FLAG_PORTABLE_KERNELS = 2 /* bf16 only: use the plain (non-MFMA) GEMM and
                                 attention kernels, for cross-checking */
};

typedef struct {
  int32_t n_layer;    /* L */
  int32_t d_model;    /* d = n_head * head_dim */
  int32_t n_head;     /* H */
  int32_t head_dim;   /* Q, even */
  int32_t d_ff;       /* F (4d in the reference model) */
  int32_t vocab;      /* V (0 in block-only mode) */
  int32_t batch;      /* B rows per step */
  int32_t seq_len;    /* T tokens per row */
  float rope_base;    /* 10000 */
  float rms_eps;      /* 1e-6 */
  int32_t dtype;      /* nc_dtype */
  int32_t flags;      /* NC_FLAG_* */
} nc_config;

typedef struct nc_ctx nc_ctx;

/* Tensor ids for nc_param_offset. */
enum { NC_T_E = 0, NC_T_WQ, NC_T_WK, NC_T_WV, NC_T_WO, NC_T_W1, NC_T_W2, NC_T_U };

/* ---- host-only queries (no HIP calls) --------------------------------- */

/* Number of parameters: 12*L*d^2 + 2*V*d (560,988,160 at d20), or the six
 * layer tensors in block-only mode.  Negative nc_status on a bad config. */
int64_t nc_param_count(const nc_config* cfg);

/* Offset (in elements) and shape of one tensor in the flat parameter /
 * gradient buffer.  layer is ignored for E and U.  Returns nc_status. */
int nc_param_offset(const nc_config* cfg, int32_t tensor, int32_t layer,
                    int64_t* offset, int64_t* rows, int64_t* cols);

/* Bytes of device workspace nc_init needs for this config (saved
 * activations, the rotary table, loss partials, backward scratch).  The
 * workspace must be 256-byte aligned.  Negative nc_status on a bad config. */
int64_t nc_workspace_bytes(const nc_config* cfg);

/* Static text for a status code. */
const char* nc_status_string(int status);

/* ---- context ------------------------------------------------------------ */

/* Validate cfg, bind the workspace (device, >= nc_workspace_bytes(cfg)) and
 * the HIP stream (hipStream_t; NULL = the default stream), and enqueue the
 * fill of the rotary table.  *out receives a host object owned by the
 * caller (release with nc_destroy).  Returns nc_status. */
int nc_init(const nc_config* cfg, void* workspace, size_t ws_bytes,
            void* hip_stream, nc_ctx** out);

/* Switch the stream later calls enqueue on. */
int nc_set_stream(nc_ctx* ctx, void* hip_stream);

void nc_destroy(nc_ctx* ctx);

/* Text of the last error on this context ("" if none). */
const char* nc_last_error(const nc_ctx* ctx);

/* In bf16 mode without NC_FLAG_PORTABLE_KERNELS every product and attention
 * call runs on the matrix-core kernels when its shape allows (products:
 * B*T and the widths multiples of 128; attention: head dim 128 with T a
 * multiple of 64); any other shape runs the portable (non-MFMA) kernel instead, with
 * the same results to rounding but far slower.  *count receives how many
 * launches on this context took that fallback since it was created or last
 * reset (reset = 1 zeroes it after reading).  Host-only; fp32 contexts and
 * NC_FLAG_PORTABLE_KERNELS contexts always count 0. */
int nc_fallback_count(nc_ctx* ctx, int64_t* count, int32_t reset);

/* ---- full model ------------------------------------------------------------ */

/* Forward pass over B x T tokens.
 *   params  device, dtype, [nc_param_count]
 *   idx     device int32 [B*T], token ids in [0, V)
 *   targets device int32 [B*T], next-token ids in [0, V) or -1 (ignored)
 *   ce_out  device fp32 [B*T] per-token cross-entropy in nats (0 where the
 *           target is ignored), or NULL
 * idx and targets are copied into the workspace, and every activation the
 * backward pass needs is saved there.  An id outside [0, V) (or a target
 * >= V) is an error the library does not check on the host (the ids are in
 * device memory): nothing is read out of bounds for it, and NaN is written
 * into what depends on it -- the embedding row of a bad id (and from it the
 * activations of its row: attention products may carry it to other
 * positions of the row), the ce of a bad target, so also the loss, bits per
 * byte and gradients -- which shows after the stream is synchronised.  Not available in block-only mode
 * (NC_ERR_STATE). */
int nc_forward(nc_ctx* ctx, const void* params, const int32_t* idx,
               const int32_t* targets, float* ce_out);

/* nc_forward for evaluation (validation loss and bits per byte, section
 * Pretraining's bpb evaluation): the same results, bit for bit, without the
 * bf16 copy of the logits that nc_forward keeps in the workspace for the
 * backward when the batch is at most 65,536 tokens (writing it costs about
 * 2 % of a d20 training step).  A backward after it is still valid and
 * recomputes the unembedding product instead. */
int nc_forward_eval(nc_ctx* ctx, const void* params, const int32_t* idx,
                    const int32_t* targets, float* ce_out);

/* Loss and bits per byte of the last nc_forward.
 *   token_bytes device int32 [V], UTF-8 bytes of each vocabulary id
 *   out         device double [5]: mean ce in nats, bits per byte,
 *               sum of ce, sum of target bytes, number of valid targets.
 * Sums run in fp64 over the per-token fp32 ce (deterministic order).
 * NC_ERR_STATE without a prior nc_forward. */
int nc_loss_bpb(nc_ctx* ctx, const int32_t* token_bytes, double* out);

/* Gradient of the mean cross-entropy of the last nc_forward with respect to
 * every parameter, fp32, written to grads (device fp32 [nc_param_count]),
 * overwriting it (accumulate = 0) or adding to it (accumulate = 1).
 * params must be the buffer passed to nc_forward, unchanged.  NC_ERR_STATE
 * without a prior nc_forward.  Deterministic: every sum (embedding rows
 * included: the positions of each token id are summed in increasing order)
 * runs in a fixed order, so repeated calls give identical bits. */
int nc_backward(nc_ctx* ctx, const void* params, float* grads, int32_t accumulate);

/* Token-weighted variant (the simplified GRPO of section Reinforcement
 * learning: per-token advantage weights, normalised over tokens, no
 * reference model, no ratio clipping): the gradient of
 *   sum over valid targets t of w_t ce[t] / n_valid
 * with token_weights w device fp32 [B*T] (any sign; ignored targets still
 * contribute nothing).  w = 1 everywhere gives nc_backward's result bit for
 * bit.  Otherwise as nc_backward. */
int nc_backward_weighted(nc_ctx* ctx, const void* params, float* grads, int32_t accumulate,
                         const float* token_weights);

/* The weighted objective of the last nc_forward: out device double [2] =
 * {sum over valid targets of w_t ce[t], that sum / n_valid} (fp64, fixed
 * order; 0 / 0 gives 0).  NC_ERR_STATE without a prior nc_forward. */
int nc_loss_weighted(nc_ctx* ctx, const float* token_weights, double* out);

/* ---- KV-cache inference: prefill and decode ------------------------------ */
/* The Engine of the walkthrough (section Pretraining, the paragraph after
 * the sampled completions): generation with a KV cache in two phases,
 * prefill over the prompt and decode one token at a time, several samples
 * of one prompt decoded together.  The cache holds, per layer, K (rotated)
 * and V as [max_batch][max_len][d] in the model dtype, layer l's K at
 * element 2 l max_batch max_len d and its V right after.  Decode handles
 * at most 16 sequences and head_dim 32, 64, 96 or 128 (else
 * NC_ERR_UNSUPPORTED). */
int64_t nc_kv_cache_bytes(const nc_config* cfg, int32_t max_batch, int32_t max_len);

/* Bytes of the scratch nc_decode needs (256-byte aligned device memory). */
int64_t nc_decode_scratch_bytes(const nc_config* cfg, int32_t max_batch, int32_t max_len);

/* Prefill: the model over one prompt.  The context must have batch 1;
 * idx device int32 [seq_len] holds the prompt in its first prompt_len
 * entries and any valid ids after (causal attention keeps them from
 * affecting the prompt).  Writes K, V of positions 0 .. prompt_len-1 into
 * sequences 0 .. nseq-1 of the cache (the same prompt for each) and the
 * fp32 logits of the last prompt position to logits device [V].  Leaves the
 * context's forward state as nc_forward would. */
int nc_prefill(nc_ctx* ctx, const void* params, const int32_t* idx, int32_t prompt_len, int32_t nseq,
               void* kv_cache, int32_t max_batch, int32_t max_len, float* logits);

/* Decode: one new token per sequence, tokens device int32 [nseq], all at
 * position pos (the sequences' common length so far; 0 <= pos < max_len).
 * Appends each token's K, V at pos and writes fp32 logits [nseq][V] of the
 * next token.  Uses only the scratch (not the context's workspace).  A
 * token outside [0, V) reads nothing and makes its sequence's logits (and
 * the K, V it appends) NaN. */
int nc_decode(nc_ctx* ctx, const void* params, const int32_t* tokens, int32_t nseq, int32_t pos, void* kv_cache,
              int32_t max_batch, int32_t max_len, void* scratch, float* logits);

/* nc_decode for callers that cannot allocate device memory or pass a
 * scratch buffer (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and results, bit for
 * bit, with the scratch taken from a static device array of
 * nc_decode_static_max_bytes() bytes (16 MiB) that every GPU the library
 * runs on holds until the process ends.  The call allocates nothing.  Its
 * scratch is laid out for this call's size, (nseq, pos + 1), so it serves,
 * e.g., d20 with 16 sequences up to ~12k cached positions; a call needing
 * more returns NC_ERR_WORKSPACE (message in nc_last_error) before any
 * launch.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (several streams, several contexts) race and must be
 * serialised by the caller.  No part of the array needs to start at zero:
 * every call writes what it reads.  Otherwise as nc_decode. */
int64_t nc_decode_static_max_bytes(void);
int nc_decode_static(nc_ctx* ctx, const void* params, const int32_t* tokens, int32_t nseq, int32_t pos,
                     void* kv_cache, int32_t max_batch, int32_t max_len, float* logits);

/* Next token of each row of logits device fp32 [n][V], as the Engine
 * samples: the largest logit (first id on ties) when temperature == 0;
 * otherwise p_i proportional to exp((z_i - max z) / temperature) over the
 * top_k largest logits (all when top_k == 0; ties with the k-th largest are
 * kept), drawn by inverse CDF in id order: the first kept id whose running
 * sum exceeds u[row] * sum p (fp32 exponentials, fp64 sums in a fixed
 * order).  u device fp32 [n] in [0, 1) are the caller's uniforms; out
 * device int32 [n].  No context: enqueued on hip_stream.
 * NC_ERR_INVALID_ARG on a negative temperature or top_k, NC_ERR_SHAPE on
 * n < 1, V < 1 or V > 65536. */
int nc_sample(const float* logits, int32_t n, int32_t V, float temperature, int32_t top_k, const float* u,
              int32_t* out, void* hip_stream);

/* nc_sample with each row spread over ceil(V / 1024) workgroups instead of
 * one, for rows that would otherwise leave the chip idle (a decode step's
 * few sequences).  Same rule and inputs; the fp64 sums run in another fixed
 * order, so a draw can differ from nc_sample's only where u * sum lies
 * within rounding of a boundary of the inverse CDF.  top_k above 256 (and
 * below V) takes nc_sample's single-workgroup kernel.
 *   scratch  device, nc_sample_scratch_bytes(n, V) bytes, 256-byte aligned
 *            (NC_ERR_WORKSPACE otherwise), owned by the caller; calls that
 *            share it must not overlap.
 * NC_ERR_SHAPE on n < 1, n > 65535, V < 1 or V > 65536. */
int64_t nc_sample_scratch_bytes(int32_t n, int32_t V);
int nc_sample_parallel(const float* logits, int32_t n, int32_t V, float temperature, int32_t top_k,
                       const float* u, int32_t* out, void* scratch, void* hip_stream);

/* ---- single block (NC_FLAG_BLOCK_ONLY) ------------------------------------ */

/* y = block(x) for x, y device dtype [B*T, d] (may not alias).  Saves what
 * nc_block_backward needs.  NC_ERR_STATE unless the config is block-only. */
int nc_block_forward(nc_ctx* ctx, const void* block_params, const void* x, void* y);

/* Vector-Jacobian product of the last nc_block_forward with dy (device dtype
 * [B*T, d]): dx (device dtype [B*T, d]) and the six weight gradients
 * (device fp32, flat, block layout), overwritten or accumulated. */
int nc_block_backward(nc_ctx* ctx, const void* block_params, const void* dy,
                      void* dx, float* dparams, int32_t accumulate);

/* ---- optimiser step ------------------------------------------------------- */
/* The step after the backward pass (section Pretraining, optimiser
 * paragraph: Muon on every matrix, AdamW on the embedding E and the
 * unembedding U, nothing else trainable; learning-rate paragraph: rates
 * scale as 1/sqrt(width); the paragraph after the training log: lrm, a
 * multiplier falling linearly to 0 at the end).  The pages do not define
 * Muon; it is taken as published (K. Jordan et al., 2024):
 *   buf = momentum buf + g;  u = g + momentum buf (Nesterov) or buf;
 *   X = u / (||u||_F + 1e-7), transposed when rows > cols;
 *   ns_steps times:  A = X X^T;  B = ns_b A + ns_c A A;  X = ns_a X + B X;
 *   W -= lr_matrix sqrt(max(1, rows/cols)) X (transposed back).
 * Wq, Wk and Wv are three matrices here.  AdamW is the decoupled-decay
 * form with bias-corrected moments:
 *   p = p (1 - lr wd);  m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   p -= lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
 * Every g is first multiplied by grad_scale (1/n averages n micro-batch
 * gradients accumulated with nc_backward(..., accumulate = 1)).
 * The learning rates given here are the effective ones. */
typedef struct {
  float grad_scale;
  float lr_embed;        /* AdamW on E */
  float lr_unembed;      /* AdamW on U */
  float beta1, beta2, eps, weight_decay;
  int32_t adam_step;     /* t >= 1: AdamW steps taken, this one included */
  float lr_matrix;       /* Muon on every block matrix */
  float momentum;        /* in [0, 1) */
  int32_t nesterov;      /* 0 or 1 */
  int32_t ns_steps;      /* 0 .. 100 */
  float ns_a, ns_b, ns_c;
} nc_optim_hparams;

/* Default hyperparameters for iteration it (0-based) of num_iters, with
 * gradients accumulated over n_micro micro-batches.  These are readings, not
 * values from the pages: AdamW betas (0.8, 0.95), eps 1e-10, no decay,
 * rates 0.2 (E) and 0.004 (U) times (d/768)^-1/2; Muon rate 0.02, momentum
 * ramped 0.85 -> 0.95 over the first 300 iterations, Nesterov, 5 steps of
 * (3.4445, -4.7750, 2.0315); lrm = 1 until the last 20 % of the
 * iterations, then linear to 0; every rate is multiplied by lrm.
 * Host-only.  Returns nc_status. */
int nc_optim_default(const nc_config* cfg, int64_t it, int64_t num_iters, int32_t n_micro, nc_optim_hparams* out);

/* Bytes of optimiser state: fp32 [nc_param_count] holding, at each tensor's
 * parameter offset, Muon's momentum buffer (matrices) or AdamW's first
 * moment (E, U); then fp32 AdamW second moments of E [V*d] and U [V*d].
 * Zero it before the first step.  Negative nc_status on a bad config. */
int64_t nc_optim_state_bytes(const nc_config* cfg);

/* Bytes of device scratch nc_optimizer_step needs (256-byte aligned). */
int64_t nc_optim_scratch_bytes(const nc_config* cfg);

/* One optimiser step over every parameter.
 *   master  device fp32 [nc_param_count]: the parameters, updated in place
 *   params  device dtype [nc_param_count]: receives the updated parameters
 *           in the model dtype (the buffer nc_forward reads); may be master
 *           when the dtype is fp32
 *   grads   device fp32 [nc_param_count], read only
 *   state   device, nc_optim_state_bytes(cfg), updated in place
 *   scratch device, nc_optim_scratch_bytes(cfg)
 * The Newton-Schulz iteration runs in the model dtype (bf16 operands, fp32
 * accumulation, as published); everything else in fp32.  Deterministic:
 * repeated calls on the same inputs give identical bits.  Does not touch the
 * workspace, so a forward/backward state survives it.  NC_ERR_INVALID_ARG on
 * a null pointer or an out-of-range hyperparameter. */
int nc_optimizer_step(nc_ctx* ctx, float* master, void* params, const float* grads, void* state, void* scratch,
                      const nc_optim_hparams* hp);

/* ---- kernel timing (for roofline reports) --------------------------------- */

/* Kernel families of the step.  Each GEMM family is one matrix-core kernel
 * (one operand layout + epilogue); NC_TRACE_ATTN_FWD is one kernel and
 * NC_TRACE_ATTN_BWD the three backward kernels together. */
enum {
  NC_TRACE_GEMM_QKV_ROPE = 0, /* a Wqkv^T with the rotary epilogue           */
  NC_TRACE_GEMM_RESIDUAL,     /* x + o Wo^T and x + u W2^T                    */
  NC_TRACE_GEMM_RELU2,        /* u = relu(m W1^T)^2                           */
  NC_TRACE_GEMM_HEAD_LSE,     /* xf U^T with the log-sum-exp epilogue (which
                                 also keeps the logits when the head's
                                 backward runs as one token chunk)            */
  NC_TRACE_GEMM_HEAD_DZ,      /* dz = softmax - onehot: from the kept logits
                                 (an elementwise kernel, flops = 4 per logit),
                                 else xf U^T recomputed                       */
  NC_TRACE_GEMM_DGRAD,        /* activation gradients g W (dm, do, da, dxf)   */
  NC_TRACE_GEMM_DGRAD_RELU2,  /* dh = (g W2) * 2 relu(h)                      */
  NC_TRACE_GEMM_WGRAD,        /* weight gradients dWqkv, dWo, dW1, dW2, dU    */
  NC_TRACE_ATTN_FWD,
  NC_TRACE_ATTN_BWD,
  NC_TRACE_OPTIM_NS,          /* Muon's Newton-Schulz products (nc_optimizer_step) */
  NC_TRACE_OPTIM_ADAMW,       /* AdamW on E and U (nc_optimizer_step)         */
  NC_TRACE_COUNT
};

/* While enabled, every launch of `family` inside the model-level calls is
 * bracketed by HIP events recorded on the context's stream (host-side event
 * objects; no device memory).  family = -1 disables.  Enabling resets the
 * counters.  At most 65536 launches are recorded. */
int nc_trace_enable(nc_ctx* ctx, int32_t family);

/* Wait for the recorded events and report the family's launches: count,
 * summed duration (ms), summed algorithmic FLOPs (2*M*N*K per product; the
 * attention families count the causal products they compute) and summed
 * algorithmic HBM bytes (operands read once + result written once).  Any
 * pointer may be NULL. */
int nc_trace_read(nc_ctx* ctx, int64_t* launches, double* ms, double* flops, double* bytes);

#ifdef __cplusplus
}
#endif
#endif /* NC_H */
