/*
 * gpt2.h -- C ABI of the MI355X (gfx950) GPT-2 Pre-LN forward library.
 *
 * What the library computes (pages cited by title and section):
 *   x_0   = wte[id_t] + wpe[t]                       (pwwt.cn "逐行拆GPT-2源码", GPT2Model)
 *   H_l   = X_l + CausalMHA(LN_1(X_l))               (russellluo.com "Hidden State 如何流过
 *   X_l+1 = H_l + MLP(LN_2(H_l))                      GPT-2 Block", section GPT-2 Block)
 *   logits = LN_f(X_L) @ wte^T   (tied, no bias)     (pwwt.cn, GPT2LMHeadModel)
 * with LN(x) = gamma*(x-mu)/sqrt(var+eps)+beta (biased variance), attention
 * softmax(q k^T / sqrt(head_dim)) over keys j <= i, MLP = c_proj(gelu_new(c_fc(x)))
 * with gelu_new the tanh approximation (pwwt.cn, GPT2Attention and GPT2MLP).
 * Incremental decode with a key/value cache places the new token at position
 * past_len (pwwt.cn, GPT2Model position_ids and the KV-cache lines of
 * GPT2Attention).
 *
 * Conventions for every entry point:
 *   - Every pointer named d_* is DEVICE memory owned by the caller; the library
 *     never allocates or frees device memory and keeps only the pointers it is
 *     given at gpt2_create.  The gpt2_model handle owns host memory only.
 *   - Every call that launches work is asynchronous on `stream` (a hipStream_t,
 *     NULL = the default stream) and never synchronises.  Faults inside kernels
 *     surface at the caller's next synchronisation.
 *   - All argument checks happen on the host before anything is launched; on
 *     any error nothing is launched and nothing is written.
 *   - One handle must not be used concurrently from two streams: the forward
 *     and decode calls share its workspace.
 *   - Token ids must lie in [0, vocab_size).  The embedding clamps an id
 *     outside that range to the nearest valid one (0 or vocab_size - 1), so a
 *     bad id never makes the gather read outside wte, but the outputs of that
 *     position are then those of the clamped id; gpt2_set_id_check gives a
 *     device flag that reports it.
 */
#ifndef GPT2_H
#define GPT2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPT2_OK = 0,
  GPT2_ERR_INVALID_ARG = 1, /* null pointer, bad alignment, non-positive size */
  GPT2_ERR_SHAPE = 2,       /* T outside [1, n_positions], B < 1, blob size mismatch, ... */
  GPT2_ERR_CAPACITY = 3,    /* KV cache full or too small for the request */
  GPT2_ERR_WORKSPACE = 4,   /* workspace / parameter region smaller than required */
  GPT2_ERR_UNSUPPORTED = 5, /* configuration the kernels do not cover (see gpt2_config) */
  GPT2_ERR_HIP = 6          /* a HIP runtime call or kernel launch failed */
} gpt2_status;

typedef enum { GPT2_F32 = 0, GPT2_BF16 = 1 } gpt2_dtype;

/* Model hyper-parameters, the GPT2Config fields of pwwt.cn section GPT2Config.
 * Supported: d_model % 64 == 0, d_model <= 2048, d_model % n_head == 0,
 * head_dim = d_model/n_head in {16, 64} (16 with GPT2_F32 only),
 * d_ff % 64 == 0, n_positions <= 4096, vocab_size <= 2^24.
 * dtype GPT2_F32: every kernel computes and stores in fp32.
 * dtype GPT2_BF16: matrices, wte and wpe are held in bf16 (round to nearest
 * even from the fp32 blob), biases and LayerNorm parameters in fp32; matrix
 * products take bf16 operands with fp32 accumulation; the residual stream,
 * LayerNorm statistics, softmax and GELU are fp32.
 * logits_dtype: element type of the logits the forward and decode calls write
 * (GPT2_F32 or GPT2_BF16; the lm_head accumulates in fp32 either way and
 * GPT2_BF16 rounds each logit to nearest even on the store).
 * Variant switches (all 0 = GPT-2 as released):
 *   activation: 0 gelu_new, the tanh form (pwwt.cn GPT2MLP); 1 the erf GELU
 *     0.5x(1 + erf(x/sqrt 2)) the same section contrasts it with.
 *   scale_attn_by_inverse_layer_idx: 1 divides layer l's attention scores by
 *     l + 1 as well (pwwt.cn GPT2Config: on in the original TensorFlow code).
 *   post_ln: 1 wires each block as H = LN_1(X + Attn(X)), X' = LN_2(H + MLP(H))
 *     (the Post-Norm form, russellluo.com Pre-Norm section; dpshk.com 3.1);
 *     ln_f and the head are unchanged.
 *   separate_head: 1 gives the head its own weight lm_head.w [V, D]
 *     (nano-ai.tech Transformer Stack: an nn.Linear head), appended to the
 *     blob after ln_f; 0 ties it to wte. */
typedef struct {
  int32_t vocab_size;
  int32_t n_positions;
  int32_t d_model;
  int32_t n_head;
  int32_t n_layer;
  int32_t d_ff;
  float ln_eps;
  int32_t dtype;        /* gpt2_dtype of the arithmetic */
  int32_t logits_dtype; /* gpt2_dtype of d_logits */
  int32_t activation;   /* 0 gelu_new, 1 erf GELU */
  int32_t scale_attn_by_inverse_layer_idx;
  int32_t post_ln;
  int32_t separate_head;
} gpt2_config;

typedef struct gpt2_model gpt2_model;

/* A key/value cache in caller-owned device memory (gpt2_kv_cache_bytes bytes).
 * With S = gpt2_kv_stride(cfg, max_T) = max_T rounded up to a multiple of 64,
 * layer l occupies 2*B*S*d_model elements starting at element
 * l*2*B*S*d_model: K as [B][n_head][S][head_dim], then V transposed as
 * [B][n_head][head_dim][S]; position t of a sequence is slot t of its S, and
 * slots >= max_T are never read or written.  Element type as the model dtype.
 * past_len counts the cached positions; gpt2_forward with a view sets it to T
 * and gpt2_decode_step increments it. */
typedef struct {
  void* d_kv;
  int32_t B;
  int32_t max_T;
  int32_t past_len;
} gpt2_kv_view;

/* Number of floats in the host parameter blob: wte[V,D], wpe[P,D], per layer
 * ln_1.{w,b}, attn.c_attn.{w[D,3D],b}, attn.c_proj.{w[D,D],b}, ln_2.{w,b},
 * mlp.c_fc.{w[D,F],b}, mlp.c_proj.{w[F,D],b}, then ln_f.{w,b} -- the order of
 * the safetensors key list (pwwt.cn, section on weights and architecture),
 * matrices [in, out] as Conv1D stores them -- and, with separate_head, the
 * head lm_head.w [V, D]. */
gpt2_status gpt2_param_blob_floats(const gpt2_config* cfg, size_t* n_floats);

/* Bytes of the device parameter region (converted layout, see gpt2_init_params). */
gpt2_status gpt2_param_bytes(const gpt2_config* cfg, size_t* bytes);

/* One tensor of the parameter blob (the safetensors key list of pwwt.cn,
 * section on weights and architecture, in that order) and where
 * gpt2_init_params puts its converted copy.  Host-only queries, no HIP call.
 *   blob_offset:  first float of the tensor in the blob.
 *   rows, cols:   its blob shape [rows, cols]; vectors (biases, LayerNorm
 *                 gamma/beta) have rows = 1.
 *   dev_dtype:    element type in the device region: GPT2_BF16 for matrices,
 *                 wte, wpe (and lm_head.w) of a bf16 model, rounded to nearest
 *                 even; GPT2_F32 otherwise (all vectors, every fp32 model tensor).
 *   transposed:   1 when stored as [cols][rows] (element (r, c) of the blob
 *                 tensor at element c * dev_ld + r), 0 when stored as [rows][cols].
 *   dev_offset:   byte offset of the copy in the device region.
 *   dev_ld:       elements between consecutive stored rows.
 *   dev_rows:     stored rows, at least the blob's; the extra rows (wte and
 *                 lm_head.w, padded to a multiple of 256) hold zeros.
 * gpt2_param_tensor_count gives the number of tensors (4 + 12 * n_layer
 * with the tied head, one more with separate_head); gpt2_param_tensor returns
 * GPT2_ERR_SHAPE for an index outside [0, count). */
typedef struct {
  int64_t blob_offset;
  int32_t rows;
  int32_t cols;
  int32_t dev_dtype;
  int32_t transposed;
  int64_t dev_offset;
  int64_t dev_ld;
  int64_t dev_rows;
} gpt2_param_info;
gpt2_status gpt2_param_tensor_count(const gpt2_config* cfg, int32_t* n);
gpt2_status gpt2_param_tensor(const gpt2_config* cfg, int32_t index, gpt2_param_info* info);

/* Slot stride S of a KV cache for max_T positions (see gpt2_kv_view):
 * max_T rounded up to a multiple of 64.  GPT2_ERR_SHAPE unless
 * 1 <= max_T <= n_positions. */
gpt2_status gpt2_kv_stride(const gpt2_config* cfg, int32_t max_T, int32_t* stride);

/* Bytes of device workspace needed for gpt2_forward at batch B, length T, and
 * for gpt2_decode_step at batch B (T = 1). */
gpt2_status gpt2_workspace_bytes(const gpt2_config* cfg, int32_t B, int32_t T, size_t* bytes);

/* Bytes of a KV cache for B sequences of up to max_T positions (max_T <= n_positions). */
gpt2_status gpt2_kv_cache_bytes(const gpt2_config* cfg, int32_t B, int32_t max_T, size_t* bytes);

/* Create a handle.  d_params: gpt2_param_bytes bytes; d_workspace: ws_bytes
 * bytes (the largest forward the handle will run decides the size).  Both must
 * be 256-byte aligned and stay valid until gpt2_destroy.  No HIP call is made. */
gpt2_status gpt2_create(const gpt2_config* cfg, void* d_params, size_t param_bytes,
                        void* d_workspace, size_t ws_bytes, gpt2_model** out);

void gpt2_destroy(gpt2_model* model);

/* Convert the fp32 parameter blob (DEVICE memory, n_floats floats in the
 * gpt2_param_blob_floats order) into the device parameter region: matrices are
 * transposed to [out, in] and, for GPT2_BF16, rounded to bf16 (nearest even);
 * wte is zero-padded to a multiple of 256 rows.  The blob is only read and may
 * be freed once the stream has passed this call. */
gpt2_status gpt2_init_params(gpt2_model* model, const float* d_blob, size_t n_floats, void* stream);

/* Full forward of B sequences of T tokens (1 <= T <= n_positions).
 *   d_tokens: int32 [B, T] token ids.
 *   d_logits: [B, T, vocab_size] of cfg.logits_dtype, or NULL (skip the lm_head).
 *   d_hidden: fp32 [B, T, d_model] output of the final LayerNorm, or NULL.
 *   kv:       NULL, or a cache view with kv->B == B and kv->max_T >= T: keys and
 *             values of positions [0, T) are written into it and kv->past_len
 *             is set to T (prefill).
 * The workspace must hold gpt2_workspace_bytes(cfg, B, T). */
gpt2_status gpt2_forward(gpt2_model* model, const int32_t* d_tokens, int32_t B, int32_t T,
                         void* d_logits, float* d_hidden, gpt2_kv_view* kv, void* stream);

/* Row stride (elements) of the padded logits layout: vocab_size rounded up to
 * the device padding of the embedding matrix (a multiple of 256). */
gpt2_status gpt2_logits_padded_ld(const gpt2_config* cfg, int64_t* ld);

/* gpt2_forward with the logits rows logits_ld elements apart: row b*T + t
 * starts at d_logits + (b*T + t) * logits_ld, and the caller's buffer holds
 * (B*T - 1) * logits_ld + vocab_size elements (B*T * logits_ld when
 * logits_ld >= the padded stride).  Same computation as gpt2_forward (the
 * tied lm_head of pwwt.cn section GPT2LMHeadModel).
 *   logits_ld >= gpt2_logits_padded_ld: every row is written in whole; the
 *     columns [vocab_size, padded ld) receive 0 (the logits of the zero
 *     padding rows of the embedding) and columns past that are not written.
 *     This is the fast layout: no per-column test at the vocabulary edge, and
 *     rows aligned to the buffer's alignment.
 *   vocab_size <= logits_ld < padded ld: only columns [0, vocab_size) are written.
 * Errors: GPT2_ERR_SHAPE when d_logits is given and logits_ld < vocab_size or
 * logits_ld > INT32_MAX; the other checks are those of gpt2_forward. */
gpt2_status gpt2_forward_strided(gpt2_model* model, const int32_t* d_tokens, int32_t B, int32_t T,
                                 void* d_logits, int64_t logits_ld, float* d_hidden, gpt2_kv_view* kv,
                                 void* stream);

/* Next-token cross-entropy of B sequences of T tokens (2 <= T <= n_positions),
 * pwwt.cn section GPT2LMHeadModel (its second design): the logits of position
 * t are scored against the label of position t + 1 -- the shift happens here,
 * so labels are given per position like the tokens and NULL means "the tokens
 * themselves" -- and the mean is taken over the scored positions.
 *   d_labels:     int32 [B, T] or NULL.  A negative label marks a position
 *                 that is not scored (its loss is 0 and it is left out of the
 *                 mean); labels >= vocab_size are a caller error and give NaN.
 *   d_token_loss: fp32 [B, T-1] (position t of sequence b at b*(T-1) + t), or NULL.
 *   d_mean_loss:  fp32 [1], or NULL (at least one of the two outputs is required).
 *                 NaN when no position is scored.
 * Per position: log(sum_v exp(logit[v])) - logit[label], evaluated in fp32
 * from the lm_head's fp32 accumulators, which never leave the chip (no logits
 * are written).  Same workspace as gpt2_forward(B, T). */
gpt2_status gpt2_forward_loss(gpt2_model* model, const int32_t* d_tokens, const int32_t* d_labels, int32_t B,
                              int32_t T, float* d_token_loss, float* d_mean_loss, void* stream);

/* One decode step: one new token per sequence at position kv->past_len.
 *   d_new_tokens: int32 [kv->B]; d_logits: [kv->B, vocab_size] of cfg.logits_dtype.
 * Requires kv->past_len < kv->max_T (else GPT2_ERR_CAPACITY).  Appends the new
 * keys/values to the cache and increments kv->past_len (host side, at enqueue). */
gpt2_status gpt2_decode_step(gpt2_model* model, gpt2_kv_view* kv, const int32_t* d_new_tokens,
                             void* d_logits, void* stream);

/* gpt2_decode_step without the handle's workspace, for callers that cannot
 * allocate device memory or must not touch the workspace (code under HIP
 * graph capture, tight serving loops).  Same arguments, checks, kernels and
 * results as gpt2_decode_step; the step's activations and partial results live
 * in a scratch array of fixed size (gpt2_decode_scratch_bytes: `limit`, 16 MiB)
 * that the library holds on each GPU it runs on until the process ends.  The
 * call allocates nothing.  Every call on one GPU shares that GPU's array
 * (nothing in it needs to start at zero: each step writes what it later
 * reads), so calls that overlap on one GPU -- on two streams, or from two
 * threads -- race and must be serialised by the caller; the handle's
 * workspace is not touched.  The device is the current HIP device.
 * Errors: those of gpt2_decode_step, and GPT2_ERR_WORKSPACE when the step
 * needs more scratch than the limit (gpt2_decode_scratch_bytes: `bytes`;
 * GPT-2 small needs about 3.2 MB at B = 32). */
gpt2_status gpt2_decode_step_noalloc(gpt2_model* model, gpt2_kv_view* kv, const int32_t* d_new_tokens,
                                     void* d_logits, void* stream);

/* Scratch bytes gpt2_decode_step_noalloc needs at batch B (`bytes`, optional)
 * and the size of the library's per-device array (`limit`, optional). */
gpt2_status gpt2_decode_scratch_bytes(const gpt2_config* cfg, int32_t B, size_t* bytes, size_t* limit);

/* Greedy generation: n_steps decode steps in one call, each feeding the token
 * it chose to the next, with no host round trip (pwwt.cn closing section:
 * generation one token at a time over a KV cache; bbs.huaweicloud.com blog
 * 476445, architecture overview: LM head, softmax over the vocabulary, pick a
 * token).  The pick is the most probable token -- the largest logit, since
 * softmax is monotone -- the lowest id on ties, decided in fp32 from the
 * lm_head's accumulators, which are reduced on chip (no logits are written).
 *   d_tokens:     int32 [kv->B], the input of the first step, at position
 *                 kv->past_len (typically the prompt's last token after a
 *                 prefill of the others).
 *   d_out_tokens: int32 [kv->B, n_steps]; column i is the token chosen at
 *                 step i and the input of step i + 1.
 * Requires n_steps >= 1 and kv->past_len + n_steps <= kv->max_T (else
 * GPT2_ERR_CAPACITY); kv->past_len grows by n_steps (host side, at enqueue).
 * A row without any ordered logit (all NaN) yields token 0. */
gpt2_status gpt2_generate(gpt2_model* model, gpt2_kv_view* kv, const int32_t* d_tokens, int32_t n_steps,
                          int32_t* d_out_tokens, void* stream);

/* Generation that samples: like gpt2_generate, but each step draws its token
 * from softmax(logits / temperature) over the vocabulary -- the pages' last
 * step, a softmax over the vocabulary and a token picked from it
 * (bbs.huaweicloud.com blog 476445, architecture overview; nano-ai.tech
 * Transformer Stack: with random weights the pick is essentially a random
 * draw).  The draw uses the Gumbel-max form, argmax_v (logit_v / temperature
 * + G_v) with G_v = -ln(-ln U_v), evaluated in fp32 from the lm_head's
 * accumulators (no logits are written), and a counter-based generator, so
 * the tokens depend only on (seed, position, row) and are reproducible:
 *   s0  = splitmix64(seed)
 *   key = splitmix64(s0 ^ (position << 32) ^ row)      position: of the step's
 *                                                     input token (kv->past_len)
 *   U_v = ((splitmix64(key ^ v) >> 40) + 0.5) * 2^-24
 * with splitmix64(x) the SplitMix64 output function of x + 0x9E3779B97F4A7C15
 * (Steele, Lea and Flood, OOPSLA 2014).  temperature == 0 is the greedy
 * gpt2_generate; temperature < 0, NaN or infinite gives GPT2_ERR_INVALID_ARG.
 * Other arguments, checks and results as gpt2_generate. */
gpt2_status gpt2_generate_sample(gpt2_model* model, gpt2_kv_view* kv, const int32_t* d_tokens, int32_t n_steps,
                                 float temperature, uint64_t seed, int32_t* d_out_tokens, void* stream);

/* Bytes of the backward workspace for gpt2_block_backward at batch B, length T. */
gpt2_status gpt2_block_backward_workspace_bytes(const gpt2_config* cfg, int32_t B, int32_t T, size_t* bytes);

/* Backward of block `layer` (Pre-LN wiring; post_ln gives GPT2_ERR_UNSUPPORTED)
 * for B sequences of T tokens -- the gradients the llm.c notes of dpshk.com
 * (5.3) single out: LayerNorm with its coupled mean/variance terms, the
 * masked softmax (masked entries carry exactly zero gradient) and GELU.
 *   d_x:     fp32 [B, T, D], the block input X_l (the residual stream before
 *            the block, e.g. from gpt2_set_trace of the previous block).
 *   d_dy:    fp32 [B, T, D], gradient of the loss w.r.t. the block output.
 *   d_dx:    fp32 [B, T, D] out: gradient w.r.t. X_l (must not alias d_x, d_dy).
 *   d_grads: fp32 out, the layer's parameters in blob order (ln_1.w, ln_1.b,
 *            attn.c_attn.w [D, 3D], attn.c_attn.b, attn.c_proj.w [D, D],
 *            attn.c_proj.b, ln_2.w, ln_2.b, mlp.c_fc.w [D, F], mlp.c_fc.b,
 *            mlp.c_proj.w [F, D], mlp.c_proj.b), overwritten, summed over
 *            all B*T positions.
 *   d_ws / ws_bytes: caller-owned scratch of at least
 *            gpt2_block_backward_workspace_bytes(cfg, B, T) bytes, 256-byte
 *            aligned.  All data pointers 16-byte aligned.
 * The block's forward is recomputed from d_x (nothing from an earlier
 * forward call is reused).  bf16 models take bf16 matrix operands with fp32
 * accumulation; gradients are fp32.  The model workspace is not touched. */
gpt2_status gpt2_block_backward(gpt2_model* model, int32_t layer, int32_t B, int32_t T, const float* d_x,
                                const float* d_dy, float* d_dx, float* d_grads, void* d_ws, size_t ws_bytes,
                                void* stream);

/* Token-id check (pwwt.cn GPT2Config: ids index the vocab_size rows of wte):
 * when d_flag (DEVICE int32, caller-owned) is non-NULL, every later forward,
 * loss, decode or generation call of this handle stores 1 into *d_flag when
 * one of its input token ids lies outside [0, vocab_size) (that id was
 * clamped, see the conventions above).  The library never clears the flag:
 * the caller zeroes it and reads it after synchronising.  NULL turns the
 * check off (the clamp stays).  Labels of gpt2_forward_loss are not covered
 * (a label >= vocab_size gives a NaN loss). */
gpt2_status gpt2_set_id_check(gpt2_model* model, int32_t* d_flag);

/* Optional per-layer trace for debugging: when d_trace is non-NULL, the next
 * gpt2_forward calls copy the residual stream after every block (X_{l+1},
 * fp32 [n_layer][B*T][d_model]) into d_trace, which must hold that many floats.
 * NULL turns tracing off. */
gpt2_status gpt2_set_trace(gpt2_model* model, float* d_trace, size_t n_floats);

/* Kernel timing for measurement: when enabled, gpt2_forward records a pair of
 * HIP events (on the call's stream) around every launch of the kernel class
 * `which` (0 embed, 1 layernorm, 2 qkv gemm, 3 attention, 4 attn c_proj gemm,
 * 5 c_fc gemm, 6 mlp c_proj gemm, 7 lm_head gemm).  gpt2_timing_read waits for
 * the recorded events, returns the summed milliseconds and launch count since
 * the last read, and resets them.  At most 4096 launches are kept per read. */
gpt2_status gpt2_timing_enable(gpt2_model* model, int32_t which, int32_t on);
gpt2_status gpt2_timing_read(gpt2_model* model, double* total_ms, int32_t* launches);

const char* gpt2_status_string(gpt2_status s);

/* Text of the last HIP error seen by this thread inside the library ("" if none). */
const char* gpt2_last_error(void);

/* Digest of the sources this library was built from (16 hex digits of a
 * SHA-256 over the kernel sources, their headers, this header and the build
 * script; "unknown" when built without it), so that a loader can refuse a
 * binary that does not match the sources it ships with. */
const char* gpt2_source_hash(void);

#ifdef __cplusplus
}
#endif
#endif /* GPT2_H */
