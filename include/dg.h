/*
 * dg.h -- C ABI of the MI355X block-diffusion decoding library (libdg.so).
 *
 * One denoising step of a block-autoregressive text-diffusion decoder over
 * 256-token canvases, as described for DiffusionGemma:
 *   - "DiffusionGemma hits ~1,500 TPS on one H100", section "What DiffusionGemma
 *     is": fixed 256-token canvases of random tokens; each step runs a
 *     bidirectional decoder pass over all positions, accepts the confident
 *     tokens, re-randomizes the rest and repeats until the block converges;
 *     finished blocks are committed to the KV cache and the next canvas starts.
 *   - same page, section "How the sampler actually works": candidate per
 *     position, entropy-bound acceptance, re-randomization, step cap; nothing
 *     of a canvas enters the KV cache before the block is accepted.
 *   - "DiffusionGemma Hits 1,000 Tokens per Second", section "How diffusion
 *     text generation changes the bottleneck": the next canvas is conditioned
 *     on the committed block (block-autoregressive).
 *   - "Google open-sources DiffusionGemma", section "26B MoE Architecture, but
 *     Only 3.8B Activated": MoE, bidirectional attention.
 *
 * Rules the pages leave open and this library fixes (acceptance rule, random
 * draws, model details) are stated at each call below.
 *
 * Conventions for every call:
 *   - Every pointer named *_dev is device memory on the context's device; every
 *     other array pointer is host memory.  Host arrays are read or written
 *     before the call returns.
 *   - The caller owns all device memory (weights, KV cache, scratch) and the
 *     HIP stream; a context borrows them for its lifetime and never allocates
 *     device memory itself.
 *   - Every call returns a dg_status.  Arguments are validated before any work
 *     is queued, so a call that fails validation changes no state.  After any
 *     failure dg_last_error() gives a message.  Device faults surface as
 *     DG_ERR_HIP at the next call that synchronizes the stream.
 *   - Calls on one context must not overlap (not thread-safe per context).
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dg_status {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = -1, /* null pointer, bad size, shape the kernels do not support */
  DG_ERR_WORKSPACE = -2,   /* kv or scratch buffer smaller than dg_workspace_size() */
  DG_ERR_STATE = -3,       /* call not allowed in the request's current state */
  DG_ERR_CAPACITY = -4,    /* request index or context length beyond the configured maximum */
  DG_ERR_HIP = -5,         /* a HIP runtime call failed */
  DG_ERR_UNSUPPORTED = -6  /* configuration outside what the kernels implement */
} dg_status;

typedef enum dg_dtype { DG_F32 = 0, DG_BF16 = 1 } dg_dtype;

/*
 * Storage of the routed experts' weights.  The pages name FP8 checkpoints
 * ("DiffusionGemma hits ~1,500 TPS on one H100", section "Serve it with
 * vLLM") and a quantized model of about 18 GB ("Google open-sources
 * DiffusionGemma: H100 reaches 1000 TPS", section "26B MoE Architecture, but
 * Only 3.8B Activated") without their layout; the format taken:
 *   DG_EXPERTS_NATIVE: the model dtype, like every other weight;
 *   DG_EXPERTS_FP8: one byte per weight in the OCP FP8 E4M3 encoding (bias 7,
 *     subnormals at exponent 0, 0x7F / 0xFF NaN, largest finite 448) plus one
 *     float32 scale per output row (dg_layer_weights.w1_scale, ...):
 *     W[e][n][k] = scale[e][n] * e4m3(code[e][n][k]).  The kernels widen the
 *     codes to bf16 (exact) and apply the scale to the fp32 row sum.  bf16
 *     models only (DG_ERR_INVALID_ARG otherwise).  Code arrays must not hold
 *     NaN codes.
 *   DG_EXPERTS_MXFP4: the OCP Microscaling (MX) FP4 format: E2M1 codes (sign,
 *     two exponent bits with bias 1, one mantissa bit; magnitudes 0, 0.5, 1,
 *     1.5, 2, 3, 4, 6), two per byte with the lower reduction index k in the
 *     low nibble, plus one E8M0 scale byte per 32 consecutive weights of a row
 *     (dg_layer_weights.w1_mx_scale, ...):
 *     W[e][n][k] = 2^(s[e][n][k / 32] - 127) * e2m1(code of k).  The kernels
 *     widen the codes to bf16 times the block scale (exact).  bf16 models
 *     only; the reduction length of each matrix (d_model for w1 / w3,
 *     expert_hidden for w2) is a multiple of 64, as for every format.  Scale
 *     bytes must lie in 1 .. 252 (2^-126 .. 2^125, where every code times the
 *     scale is a bf16 value): byte 0 (2^-127) reads as a zero scale, 253 and
 *     254 overflow bf16 for the largest codes and 255 (NaN) is not implemented.
 *   The pages also name NVFP4 checkpoints; MXFP4 is CDNA4's native 4-bit
 *   format and the one built.
 */
typedef enum dg_expert_format {
  DG_EXPERTS_NATIVE = 0,
  DG_EXPERTS_FP8 = 1,
  DG_EXPERTS_MXFP4 = 2
} dg_expert_format;

/*
 * Model shape.  Pre-norm decoder blocks: RMSNorm (gain per channel, eps under
 * the root), grouped-query attention with rotate-half RoPE at absolute
 * positions (pairs j, j + head_dim/2; angle pos * rope_theta^(-2j/head_dim);
 * scores scaled by 1/sqrt(head_dim); q-head h reads kv-head
 * h / (n_q_heads / n_kv_heads)), then a mixture of experts: router logits
 * r = b . Wg^T in fp32, the top_k largest (ties to the lower expert id), gates
 * = softmax over those top_k logits, routed SwiGLU experts
 * W2 (silu(W1 b) * W3 b) weighted by the gates, plus one shared SwiGLU expert
 * with weight 1.  The embedding is not scaled and serves as the LM head (tied).
 *
 * Supported shapes: head_dim 16, 32, 64, 128 or 256 (bf16: at least 64);
 * d_model (at most 16384) and expert_hidden multiples of 64; n_q_heads*head_dim and
 * shared_hidden multiples of 64 (bf16) or 16 (f32); vocab a multiple of 128;
 * top_k <= 16; n_experts <= 256; max_requests <= 16; max_ctx a multiple of 64;
 * canvas_len == 256; prefill_chunk <= 32768.
 *
 * Self-conditioning ("DiffusionGemma hits ~1,500 TPS on one H100", section "How
 * the sampler actually works": the previous step's softmax is fed back through
 * a small gated MLP; the pages give no structure).  With self_cond_hidden m > 0
 * every canvas position keeps a state u in R^d: zero when the canvas starts,
 * and after each denoising step, at the positions that were open when the step
 * began, u = sum_v softmax(z)_v E[v] (the expectation of the tied embedding
 * under that step's logits z; softmax rounded to bf16 before the product).
 * Every forward over the canvas (denoising steps and the block commit) adds
 * sc_w2 (silu(sc_w1 u) * (sc_w3 u)) to the token embedding, u rounded to
 * bf16.  bf16 models only; m a multiple of 64 and at most 4096.
 */
typedef struct dg_model_config {
  int32_t vocab;
  int32_t d_model;
  int32_t n_layers;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t n_experts;
  int32_t top_k;
  int32_t expert_hidden;
  int32_t shared_hidden;
  int32_t canvas_len;    /* 256 */
  int32_t max_ctx;       /* per request: prompt + committed blocks + one canvas */
  int32_t max_requests;  /* canvases denoised together in one step */
  int32_t prefill_chunk; /* prompt rows per prefill pass; 0 selects 2048 */
  float rope_theta;      /* 10000 */
  float rms_eps;         /* 1e-6 */
  int32_t dtype;         /* dg_dtype of weights, KV cache and activations */
  int32_t expert_format; /* dg_expert_format of the routed experts' w1, w3, w2 */
  int32_t self_cond_hidden; /* width m of the self-conditioning MLP; 0 = none */
} dg_model_config;

/*
 * Entropy-bound sampler.  In both modes the candidate at every open position
 * is its argmax token (ties to the lower id), accepted positions never change,
 * every open position not accepted is re-drawn (see dg_denoise_step), and at
 * step max_steps of a block every position still open is set to its argmax and
 * accepted (the step cap; max_steps <= 0 selects canvas_len).
 *
 * DG_SAMPLER_THRESHOLD (0): "How the sampler actually works" leaves the rule
 * open; the reading taken accepts the open positions whose softmax entropy
 * (nats, fp32) is strictly below tau, plus always the single open position of
 * lowest entropy (ties to the lower position).
 *
 * DG_SAMPLER_BUDGET (1): the default sampler of "DiffusionGemma hits ~1,500 TPS
 * on one H100", section "How the sampler actually works" (budget 0.1, stop
 * threshold 0.005 there), described in words only.  Readings taken: open
 * positions are taken in order of rising entropy (ties to the lower position)
 * while the running sum of their entropies, the position's own included, is
 * at most `budget`, and the first of them always; the block ends early when
 * the argmax canvas (accepted positions at their token, open ones at this
 * step's argmax) equals that of the block's previous step and the mean
 * entropy of the open positions is below `stop_entropy`: every open position
 * not taken is then set to its argmax and accepted, as at the cap.  Sums and
 * the mean compare exactly in 64-bit fixed point: each fp32 entropy h counts
 * floor(clamp(h, 0, 64) * 2^40) (NaN as 64), budget and stop_entropy the same.
 * The previous argmax canvas is forgotten by dg_set_canvas.  tau is unused.
 */
#define DG_SAMPLER_THRESHOLD 0
#define DG_SAMPLER_BUDGET 1
typedef struct dg_sampler_config {
  float tau;
  int32_t max_steps;
  int32_t mode;        /* DG_SAMPLER_THRESHOLD or DG_SAMPLER_BUDGET */
  float budget;        /* >= 0, finite; DG_SAMPLER_BUDGET only */
  float stop_entropy;  /* >= 0, finite; DG_SAMPLER_BUDGET only */
} dg_sampler_config;

/*
 * Device weights of one layer, dtype of the model, row-major [out, in]:
 *   attn_norm, ffn_norm [d]; wq [Hq*hd, d]; wk, wv [Hkv*hd, d]; wo [d, Hq*hd];
 *   router [E, d]; w1, w3 [E, eh, d]; w2 [E, d, eh]; sw1, sw3 [sh, d]; sw2 [d, sh].
 * With expert_format DG_EXPERTS_FP8, w1, w3 and w2 hold E4M3 codes (uint8, same
 * shapes) and w1_scale, w3_scale [E, eh] and w2_scale [E, d] their float32 row
 * scales.  With DG_EXPERTS_MXFP4 they hold packed E2M1 codes (uint8 [E, eh, d/2]
 * and [E, d, eh/2]) and w1_mx_scale, w3_mx_scale [E, eh, d/32] and w2_mx_scale
 * [E, d, eh/32] their E8M0 block scales.  Scale pointers of the other formats
 * are ignored.
 */
typedef struct dg_layer_weights {
  const void *attn_norm, *wq, *wk, *wv, *wo;
  const void *ffn_norm, *router, *w1, *w3, *w2, *sw1, *sw3, *sw2;
  const float *w1_scale, *w3_scale, *w2_scale;
  const uint8_t *w1_mx_scale, *w3_mx_scale, *w2_mx_scale;
} dg_layer_weights;

typedef struct dg_weights {
  const void* embed;              /* [V, d] device; also the LM head */
  const void* final_norm;         /* [d] device */
  const dg_layer_weights* layers; /* host array of n_layers entries (copied by dg_create) */
  /* self-conditioning MLP (self_cond_hidden m > 0, else ignored), device, bf16:
   * sc_w1, sc_w3 [m, d]; sc_w2 [d, m] */
  const void *sc_w1, *sc_w3, *sc_w2;
} dg_weights;

/* Result of one denoising step for one request. */
typedef struct dg_step_info {
  int32_t active;      /* 1 if the request took part in this step */
  int32_t block;       /* canvas (block) index */
  int32_t step;        /* 1-based denoising step index within the block */
  int32_t n_accepted;  /* positions accepted by the entropy rule this step */
  int32_t n_forced;    /* positions forced at the step cap this step */
  int32_t n_open;      /* positions still open after the step */
  int32_t done;        /* 1 when every position of the canvas is accepted */
} dg_step_info;

typedef struct dg_stats {
  double prefill_ms;   /* wall time of all prefill calls in dg_generate */
  double decode_ms;    /* wall time of all denoising steps */
  double commit_ms;    /* wall time of all block commits */
  int64_t steps;       /* denoising steps run */
  int64_t tokens;      /* output tokens accepted (all requests, before truncation) */
} dg_stats;

typedef struct dg_ctx dg_ctx;

/*
 * Sizes of the two caller-owned device buffers for a configuration.
 * KV cache layout (elements of the model dtype), for request r, layer l:
 *   K at ((r * n_layers + l) * 2 + 0) * n_kv_heads * max_ctx * head_dim,
 *     as [n_kv_heads][max_ctx][head_dim] (post-RoPE keys, position-major);
 *   V at ((r * n_layers + l) * 2 + 1) * n_kv_heads * max_ctx * head_dim,
 *     as [n_kv_heads][head_dim][max_ctx] (transposed: position fastest).
 * Scratch holds activations, partial results and the canvas state.
 */
dg_status dg_workspace_size(const dg_model_config* cfg, size_t* kv_bytes, size_t* scratch_bytes);

/*
 * Create a context.  Validates the configuration, carves the scratch buffer and
 * records the weight pointers (not copied: they must outlive the context).
 * stream is a hipStream_t (NULL: the null stream).  The context also creates
 * one stream of its own (default priority) on which the bf16 model's shared
 * expert runs beside the routed experts; it is joined back into `stream` with
 * events inside every call, so each call's work is still ordered on `stream`.
 * On success *out receives the context; on failure *out is set to NULL and the
 * message is available from dg_last_error(NULL).
 */
dg_status dg_create(const dg_model_config* cfg, const dg_sampler_config* scfg,
                    const dg_weights* weights, void* kv_dev, size_t kv_bytes, void* scratch_dev,
                    size_t scratch_bytes, void* stream, dg_ctx** out);

/*
 * Prefill request `req` with n prompt token ids (host, each in [0, vocab)):
 * a causal forward over the prompt (the parent model is autoregressive; the
 * pages do not state the prompt mask) that writes the post-RoPE K and V of
 * every layer at positions [0, n).  Resets the request: committed length n,
 * block 0, no canvas.  `seed` keys the request's random draws.
 * Errors: DG_ERR_CAPACITY if req >= max_requests or n + canvas_len > max_ctx;
 * DG_ERR_INVALID_ARG for a null prompt, n < 0 or an id out of range.
 * Synchronizes the stream before returning.
 */
dg_status dg_prefill(dg_ctx* ctx, int32_t req, const int32_t* prompt_ids, int32_t n, uint64_t seed);

/*
 * One denoising step for every prefilled request that has room for a canvas.
 * A request without an active canvas first starts one: block index = blocks
 * committed so far, every position drawn at step index 0.  Then, over all
 * active canvases together: embed, n_layers blocks (canvas queries attend
 * without mask to the request's committed prefix and to the whole canvas),
 * final norm, LM head fused with per-position softmax entropy and argmax
 * (open positions only), and the sampler (see dg_sampler_config).  Positions
 * that stay open are re-drawn uniformly: token = floor(r0 * vocab / 2^64)
 * where r0 is the first word of Philox4x64-10 (Salmon et al., SC'11) with key
 * (seed, 0) and counter (position, step, block, 0).
 * info: host array of max_requests entries (entries of inactive requests get
 * active = 0).  A request whose canvas is done takes no further steps until
 * dg_commit_block.  Synchronizes the stream before returning.
 * Errors: DG_ERR_STATE if no request can step.
 */
dg_status dg_denoise_step(dg_ctx* ctx, dg_step_info* info);

/*
 * Commit request `req`'s finished canvas: one more forward over the final
 * canvas (all layers; the last layer's FFN and the LM head are not needed)
 * writes its post-RoPE K and V at positions [P, P + canvas_len), then the
 * committed length P grows by canvas_len and the block index by one.  out_ids
 * (host, canvas_len entries, may be NULL) receives the block's token ids.
 * Errors: DG_ERR_STATE if the request has no canvas or it is not done.
 */
dg_status dg_commit_block(dg_ctx* ctx, int32_t req, int32_t* out_ids);

/*
 * Whole generation for n_req requests (n_req <= max_requests), requests
 * 0..n_req-1: prefill each prompt, then block after block: denoise all
 * requests together until every canvas is done, commit each.  Output length
 * n_out is rounded up to whole canvases and truncated: out_ids[r] (host,
 * n_out entries each) receives request r's tokens.  stats may be NULL.
 */
dg_status dg_generate(dg_ctx* ctx, int32_t n_req, const int32_t* const* prompts,
                      const int32_t* n_prompt, int32_t n_out, const uint64_t* seeds,
                      int32_t* const* out_ids, dg_stats* stats);

void dg_destroy(dg_ctx* ctx);

/* Message of the last failure on ctx (or of the last failed dg_create if ctx is NULL). */
const char* dg_last_error(const dg_ctx* ctx);

/* ------------------------------------------------------------------------ */
/* Inspection and state injection, for tests and tools.                      */
/* ------------------------------------------------------------------------ */

typedef struct dg_request_state {
  int32_t prefilled;   /* 1 after dg_prefill */
  int32_t committed;   /* committed length P */
  int32_t block;       /* current / next block index */
  int32_t step;        /* steps taken on the current canvas */
  int32_t active;      /* 1 while a canvas exists */
  int32_t done;        /* 1 when the active canvas is fully accepted */
  uint64_t seed;
} dg_request_state;

dg_status dg_get_request(dg_ctx* ctx, int32_t req, dg_request_state* st);

/* Canvas ids (canvas_len int32) and accepted flags (canvas_len uint8, 0/1) of
 * an active request; either pointer may be NULL. */
dg_status dg_get_canvas(dg_ctx* ctx, int32_t req, int32_t* ids, uint8_t* accepted);

/*
 * Replace request req's canvas: ids and accepted flags (host, canvas_len each),
 * the number of steps already taken in the block, and the block index.  The
 * request must be prefilled; committed length is kept.  Makes the canvas
 * active.  Used to start both implementations of a step from the same state.
 * With self-conditioning, a request that had no active canvas gets a zero
 * state (as a canvas started by dg_denoise_step); an active request keeps its
 * state (dg_set_self_cond replaces it).
 */
dg_status dg_set_canvas(dg_ctx* ctx, int32_t req, const int32_t* ids, const uint8_t* accepted,
                        int32_t step, int32_t block);

/* Set the committed length of a prefilled request whose cache the caller has
 * filled directly (layout in dg_workspace_size); drops any canvas. */
dg_status dg_set_committed(dg_ctx* ctx, int32_t req, int32_t committed, uint64_t seed);

/*
 * Per-row results of the last dg_denoise_step, rows = active canvas rows in
 * request order (row = slot * canvas_len + position where slot counts the
 * requests that were active).  Any pointer may be NULL.  Entries for rows
 * that were accepted before the step are left untouched (not computed).
 * entropy, lse: fp32; argmax: int32.  router_ids (int32) and router_gates
 * (fp32): [n_layers][rows][top_k] routing decisions of every layer.
 */
dg_status dg_last_step_rows(dg_ctx* ctx, int32_t* n_rows, float* entropy, float* lse,
                            int32_t* argmax, int32_t* router_ids, float* router_gates);

/*
 * Router logits (fp32, before top-k) of every layer of the last
 * dg_denoise_step: logits (host) receives [n_layers][rows][n_experts], rows as
 * in dg_last_step_rows.  Errors: DG_ERR_STATE before the first step.
 */
dg_status dg_last_step_router_logits(dg_ctx* ctx, float* logits);

/*
 * Debug taps of the denoising step (tests and tools; outside the five-call
 * contract).  A caller that registers a device buffer of dg_debug_tap_size()
 * bytes gets, on every later dg_denoise_step, the fp32 hidden rows of the
 * step copied into it at three points of every layer; dg_debug_tap then reads
 * one of them back for the last step.  Rows as in dg_last_step_rows.
 *   DG_TAP_LAYER_INPUT     layer l's input rows x (layer = n_layers: the rows
 *                          after the last layer, before the final norm)
 *   DG_TAP_AFTER_ATTENTION x after layer l's attention half (residual added)
 *   DG_TAP_ROUTER_LOGITS   layer l's fp32 router logits [rows][n_experts]
 *                          (kept by every step, buffer or not)
 * The copies cost device bandwidth (2 n_layers + 1 row copies per step); a
 * NULL buffer turns them off.  The buffer is caller-owned and must outlive its
 * use.  dg_debug_tap errors: DG_ERR_STATE before a step (or when the last step
 * ran without a buffer), DG_ERR_INVALID_ARG for an unknown tap, a layer out of
 * range or a destination smaller than rows * d_model * 4 bytes (rows *
 * n_experts * 4 for the router logits).  dg_debug_set_tap_buffer:
 * DG_ERR_WORKSPACE if bytes < dg_debug_tap_size().
 */
#define DG_TAP_LAYER_INPUT 0
#define DG_TAP_AFTER_ATTENTION 1
#define DG_TAP_ROUTER_LOGITS 2
dg_status dg_debug_tap_size(const dg_model_config* cfg, size_t* bytes);
dg_status dg_debug_set_tap_buffer(dg_ctx* ctx, void* tap_dev, size_t bytes);
dg_status dg_debug_tap(dg_ctx* ctx, int32_t which, int32_t layer, float* host_dst, size_t bytes);

/*
 * Refusal self-test (host only; needs no GPU and makes no HIP call).  Every
 * launcher returns -1 and queues nothing for arguments its kernels do not
 * implement, and the entry point that called it then reports
 * DG_ERR_UNSUPPORTED ("launch refused: <launch>").  Creation-time validation
 * keeps a valid model from reaching these paths, so case i of
 * dg_debug_refusal_count() calls one launcher with such arguments on a stub
 * context and returns the status the entry point would return (the message,
 * NUL-terminated, to msg when msg_bytes > 0).  DG_ERR_INVALID_ARG for i out of
 * range.
 */
int32_t dg_debug_refusal_count(void);
dg_status dg_debug_refusal_case(int32_t i, char* msg, size_t msg_bytes);

/*
 * LM-head logits of the last step's final hidden rows: for each of the n
 * listed rows (indices as in dg_last_step_rows), vocab fp32 logits to
 * logits_dev (device, [n][vocab]).  Same normalisation and matrix-core path
 * as the fused head, but the logits are written out.
 */
dg_status dg_last_step_logits(dg_ctx* ctx, const int32_t* rows, int32_t n, float* logits_dev);

/*
 * Self-conditioning state of request req's canvas (see dg_model_config):
 * state (host, fp32 [canvas_len][d_model]) receives u of every position.
 * Errors: DG_ERR_UNSUPPORTED without self-conditioning, DG_ERR_STATE if the
 * request has no active canvas.
 */
dg_status dg_get_self_cond(dg_ctx* ctx, int32_t req, float* state);

/*
 * Replace request req's self-conditioning state (host, fp32
 * [canvas_len][d_model]); used with dg_set_canvas to start both
 * implementations of a step from the same state.  Same errors as
 * dg_get_self_cond.
 */
dg_status dg_set_self_cond(dg_ctx* ctx, int32_t req, const float* state);

/* ------------------------------------------------------------------------ */
/* Single operations of the step, on the context's weights and scratch.      */
/* Inputs and outputs are device pointers; each call runs on the context's   */
/* stream with the same kernels and launch shapes as the step and            */
/* synchronizes before returning.                                            */
/* ------------------------------------------------------------------------ */

/*
 * Attention half of layer `layer` for t rows x_dev (fp32 [t][d]) of request
 * req at absolute positions pos0 .. pos0+t-1: RMSNorm, q/k/v projection, RoPE,
 * K/V written to the request's cache at [pos0, pos0 + t), attention of the rows
 * over cache positions [0, pos0 + t) (causal != 0: key j visible to row i only
 * if j <= pos0 + i), output projection added to x_dev in place.
 * Requires pos0 + t <= max_ctx and t <= the context's row capacity.
 */
dg_status dg_op_attention(dg_ctx* ctx, int32_t req, int32_t layer, float* x_dev, int32_t t,
                          int32_t pos0, int32_t causal);

/*
 * FFN half of layer `layer` for t rows x_dev (fp32 [t][d]): RMSNorm, router,
 * top-k gates, token permutation, routed and shared experts, added to x_dev in
 * place.  ids_dev (int32 [t][top_k]) and gates_dev (fp32 [t][top_k]) receive
 * the routing (may be NULL).
 */
dg_status dg_op_moe(dg_ctx* ctx, int32_t layer, float* x_dev, int32_t t, int32_t* ids_dev,
                    float* gates_dev);

/*
 * Final RMSNorm and fused LM head over the n rows of h_dev (fp32 [n][d]):
 * per row fp32 entropy (nats), log-sum-exp and int32 argmax (ties to the lower
 * token id), without writing logits.  n <= max_requests * canvas_len.
 */
dg_status dg_op_lm_head(dg_ctx* ctx, const float* h_dev, int32_t n, float* entropy_dev,
                        float* lse_dev, int32_t* argmax_dev);

/*
 * dg_op_lm_head without allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops that forbid it): the
 * same kernels and results, but the normalised rows, the per-tile partial
 * statistics and the row count live in the library's static device scratch
 * (16 MiB, one copy per GPU, held until the process ends; its address on the
 * current device is resolved by dg_create) instead of the context's
 * workspace, and the call does not synchronise: the outputs are ready when
 * the context's stream reaches this point.  It calls no allocator and no
 * memset.  n may be any positive count whose buffers fit the 16 MiB (at most
 * about 256 rows at vocab 262144 and d_model 2816); a larger n is rejected
 * with DG_ERR_INVALID_ARG and a message giving the limit.  Every call on a GPU
 * shares that GPU's scratch: calls that overlap on one GPU (other streams,
 * other contexts, other threads) race.  DG_ERR_HIP if the scratch has no
 * device address.
 */
dg_status dg_op_lm_head_noalloc(dg_ctx* ctx, const float* h_dev, int32_t n, float* entropy_dev, float* lse_dev,
                                int32_t* argmax_dev);

/*
 * Sampler alone on request req's active canvas, given per-position entropy and
 * argmax (device, canvas_len each; entries of accepted positions are ignored)
 * as step `step` (1-based) of the current block.  Updates the canvas in place
 * and returns the step's counts in *info.
 */
dg_status dg_op_sample(dg_ctx* ctx, int32_t req, const float* entropy_dev,
                       const int32_t* argmax_dev, int32_t step, dg_step_info* info);

/*
 * Self-conditioning term of n rows: out_dev (fp32 [n][d]) = sc_w2 (silu(sc_w1 b)
 * * (sc_w3 b)) with b = bf16(u_dev) (u_dev fp32 [n][d]), by the kernels the
 * step runs on the canvas.  n <= max_requests * canvas_len.  Errors:
 * DG_ERR_UNSUPPORTED without self-conditioning.
 */
dg_status dg_op_self_cond(dg_ctx* ctx, const float* u_dev, int32_t n, float* out_dev);

/*
 * Context-free: n uniform tokens in [0, vocab) for positions 0..n-1 of
 * (seed, block, step), as drawn by the sampler, to out_dev (int32).  stream as
 * in dg_create.  Synchronizes.
 */
dg_status dg_philox_tokens(uint64_t seed, int32_t block, int32_t step, int32_t n, int32_t vocab,
                           int32_t* out_dev, void* stream);

/* ------------------------------------------------------------------------ */
/* Kernel timer, for measurement.                                            */
/* ------------------------------------------------------------------------ */

/*
 * Kernel families of a denoising step.  The timer brackets every launch of one
 * family with a pair of HIP events on the context's stream; a family made of
 * two launches (the LM head and its tile merge, attention and its split merge,
 * router logits and top-k in the fp32 model) is timed as one unit.
 */
typedef enum dg_kernel_family {
  DG_KF_NONE = 0,
  DG_KF_EMBED = 1,
  DG_KF_RMSNORM = 2,
  DG_KF_QKV = 3,          /* q/k/v projection + RoPE + K/V cache write */
  DG_KF_ATTENTION = 4,    /* split-KV attention + merge */
  DG_KF_OUT_PROJ = 5,     /* output projection + residual */
  DG_KF_ROUTER = 6,       /* router logits (+ top-k gates in the fp32 model) */
  DG_KF_PERMUTE = 7,      /* (top-k gates,) expert histogram, offsets, token
                             permutation, routed work lists */
  DG_KF_EXPERT_UP = 8,    /* routed experts, W1/W3 with SwiGLU */
  DG_KF_EXPERT_DOWN = 9,  /* routed experts, W2 */
  DG_KF_SHARED_UP = 10,   /* shared expert, W1/W3 with SwiGLU */
  DG_KF_SHARED_DOWN = 11, /* shared expert, W2 + residual */
  DG_KF_COMBINE = 12,     /* gate-weighted sum of the routed outputs + residual,
                             with the next layer's attention RMSNorm */
  DG_KF_LM_HEAD = 13,     /* fused LM head + softmax statistics + tile merge */
  DG_KF_SAMPLE = 14,      /* entropy-bound sampler */
  DG_KF_SELF_COND = 15,   /* self-conditioning: MLP term added to the embedding,
                             and the state update after the LM head */
  DG_KF_COUNT = 16
} dg_kernel_family;

/* Start timing `family` (DG_KF_NONE stops) on every later denoising step and
 * block commit; resets the totals.  Synchronizes the stream.
 * Errors: DG_ERR_INVALID_ARG for an unknown family. */
dg_status dg_kernel_timer(dg_ctx* ctx, int32_t family);

/* Total GPU time (ms, from the event pairs) and number of timed launches since
 * dg_kernel_timer.  Synchronizes the stream. */
dg_status dg_kernel_timer_read(dg_ctx* ctx, double* total_ms, int64_t* launches);

/* Bracket the timed family's launches only in every `every`-th denoising step or
 * block commit from now on (1, the default: all).  Each event pair costs a few
 * microseconds of stream time, so sampling keeps the timer from slowing the
 * steps it measures.  Errors: DG_ERR_INVALID_ARG if every < 1. */
dg_status dg_kernel_timer_every(dg_ctx* ctx, int32_t every);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
