/*
 * gpt.h — C ABI of the MI355X (gfx950) library that runs one pretraining step
 * (forward + backward) of nanochat's GPT.
 *
 * The model (page citations, by page title and section):
 *   - Depth dial: width = 64 * depth, heads = width / 128, head dim 128
 *     (aethryn.com "Nanochat: full-stack LLM training in 8,000 lines for $72",
 *     section "One dial controls everything"; atlas.blal.pro "nanochat —
 *     full-stack ChatGPT in ~8k lines", section "How it works", item 0).
 *   - Token embedding, parameter-free RMSNorm after the embedding, before every
 *     attention and MLP and before the head; RoPE with base 10,000 on q and k,
 *     then QK-RMSNorm; relu^2 MLP 4x wide; untied LM head with logits squashed
 *     to 15*tanh(z/15) in fp32 (aethryn.com, section "A Llama-class transformer
 *     with ten modern departures"; energyai.berlin "nanochat vs GPT-OSS",
 *     section "Architectural decisions").
 *   - Multi-query attention: every query head shares one K/V head
 *     (energyai.berlin, section "Architectural decisions", subsection MQA).
 *   - Bias-free linears (atlas.blal.pro, section "How it works", item 0).
 *   - bf16 compute with fp32 gradients; gradient accumulation on one GPU
 *     (aimarketly.com "nanochat-train" README, sections "Precision / dtype" and
 *     "Getting started").
 *
 * Conventions fixed where the pages are silent: RMSNorm eps = 2^-23 with no
 * gain; attention scale 1/sqrt(head_dim); RoPE pairs element i with i + D/2
 * and rotates by +t * theta^(-2i/D), positions restart at 0 in every batch
 * row; QK-norm is per (token, head) over D; plain causal mask; the loss is the
 * mean over all B*T positions.
 *
 * Memory ownership: the caller owns every device buffer (parameters,
 * gradients, workspace, token ids, outputs). The library never allocates or
 * frees device memory. The model handle is host memory owned by the library.
 *
 * Errors: every function returns a gpt_status; GPT_OK is 0, errors are
 * negative. Nothing is thrown across the ABI. gpt_last_error_message() gives a
 * thread-local detail string for the last failing call on that thread.
 *
 * Threading: a handle serves one stream at a time and is not re-entrant;
 * distinct handles are independent.
 *
 * Streams are passed as `void*` holding a hipStream_t (NULL = default stream).
 * All device work is enqueued asynchronously on that stream.
 */
#ifndef GPT_AMD_GPT_H
#define GPT_AMD_GPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gpt_status;
enum {
  GPT_OK = 0,
  GPT_E_INVALID_ARG = -1,  /* null pointer, non-positive size, B > max_B, T > max_T, ... */
  GPT_E_UNSUPPORTED = -2,  /* config outside what the kernels implement (n_kv_head != 1, head_dim != 128, ...) */
  GPT_E_WORKSPACE = -3,    /* workspace smaller than gpt_workspace_bytes() */
  GPT_E_STATE = -4,        /* gpt_backward without a preceding gpt_forward_loss(need_grad = 1) */
  GPT_E_HIP = -5,          /* a HIP runtime call failed (detail in gpt_last_error_message) */
  GPT_E_DEVICE = -6        /* sticky device-side flag, e.g. a token id outside [0, vocab_size) */
};

/* Compute/storage dtype of parameters and activations. Gradients are always fp32.
 * GPT_FP8_E4M3: bf16 parameters and activations as for GPT_BF16, but the QKV,
 * O and MLP products -- forward, input gradient and weight gradient -- take
 * e4m3 operands with one scale per tensor, s = 448 / max|tensor| (current
 * scaling), round to nearest even, saturating at +-448; the output gradient
 * is quantised too and the backward passes the quantisation straight through.
 * The LM head and attention stay bf16. (FP8 training: repo-explainer.com
 * "karpathy/nanochat: The $100 Full-Stack LLM", section "The Engine Room: Muon
 * and FP8"; optional FP8 matmuls: atlas.blal.pro "nanochat — full-stack
 * ChatGPT in ~8k lines", section "How it works", item "2. Pretrain". The
 * scaling recipe is this library's reading; the pages give none.) The layer
 * weights are quantised by gpt_forward_loss and reused by gpt_backward, so
 * parameters must not change in between. */
enum { GPT_F32 = 0, GPT_BF16 = 1, GPT_FP8_E4M3 = 2 };

typedef struct gpt_config {
  int32_t n_layer;      /* depth */
  int32_t model_dim;    /* C = 64 * depth; multiple of 128 */
  int32_t n_head;       /* H query heads, n_head * head_dim == model_dim */
  int32_t n_kv_head;    /* must be 1 (multi-query attention) */
  int32_t head_dim;     /* must be 128 */
  int32_t mlp_dim;      /* F = 4 * C; multiple of 128 */
  int32_t vocab_size;   /* V; multiple of 256 */
  int32_t max_seq_len;  /* longest T the model accepts */
  float rope_theta;     /* 10000 */
  float logit_softcap;  /* 15 */
  float norm_eps;       /* 2^-23 */
  int32_t dtype;        /* GPT_F32, GPT_BF16 or GPT_FP8_E4M3 */
  /* Sliding-window attention (aethryn.com "Nanochat: full-stack LLM training
   * in 8,000 lines for $72", section "A Llama-class transformer with ten
   * modern departures": the "SSSL" pattern, three short-window layers then one
   * full-context layer, the final layer always full). Layer l uses
   * window_pattern[l % strlen(window_pattern)]: 'S' admits key u for query t
   * iff 0 <= t - u < window_short, 'L' the full causal prefix. The last layer
   * is always full; "" makes every layer full (the default). */
  int32_t window_short;     /* W for 'S' layers; >= 1 when the pattern holds an 'S' */
  char window_pattern[8];   /* NUL-terminated, characters 'S' and 'L' only */
  /* Residual scalars and value embeddings (aethryn.com, section "A Llama-class
   * transformer with ten modern departures": per-layer resid_lambdas and
   * x0_lambdas mix each layer's residual stream with the normalised
   * embedding; gated value embeddings add to V at alternating layers;
   * atlas.blal.pro "nanochat — full-stack ChatGPT in ~8k lines", section "How
   * it works", item 0). Both off by default. */
  int32_t x0_lambdas;    /* 1: before layer l, x <- resid_lambdas[l] * x + x0_lambdas[l] * x0, with
                            x0 = rmsnorm(wte[idx]); parameters "resid_lambdas" and "x0_lambdas" [1, n_layer] */
  int32_t value_embeds;  /* 1: layers 0, 2, 4, ... add ve_gates[j] * ve_j[idx] to v right after the QKV
                            projection; parameters "h<l>.ve" [vocab_size, n_kv_head * head_dim] per such
                            layer and "ve_gates" [1, number of such layers] */
} gpt_config;

/* One parameter tensor inside the flat parameter (and gradient) buffer. */
typedef struct gpt_tensor_desc {
  char name[32];   /* "wte", "h<l>.w_qkv", "h<l>.w_o", "h<l>.w_1", "h<l>.w_2", "lm_head" */
  int64_t offset;  /* in elements from the start of the flat buffer */
  int64_t rows;    /* row-major [rows, cols] */
  int64_t cols;
} gpt_tensor_desc;

typedef struct gpt_model gpt_model;

/* Static name of a status code. Never NULL. */
const char* gpt_status_string(gpt_status s);

/* Thread-local detail of the last error raised on this thread ("" if none). */
const char* gpt_last_error_message(void);

/* The depth dial (aethryn.com "Nanochat: full-stack LLM training in 8,000
 * lines for $72", section "One dial controls everything": width = 64 x depth,
 * heads = width / 128; atlas.blal.pro "nanochat — full-stack ChatGPT in ~8k
 * lines", section "How it works": heads of dim 128, separate query and K/V
 * head counts (item 0), vocabulary 65,536 (item 1); energyai.berlin "nanochat
 * vs GPT-OSS", section "Context window and scaling": 2,048-token context).
 * Shapes from the depth dial: C = 64*depth, H = C/128, n_kv_head = 1, D = 128,
 * F = 4C, V = 65536, max_seq_len = 2048, theta = 1e4, softcap 15, eps = 2^-23,
 * every layer full causal attention (window_short 0, window_pattern "").
 * Host only. GPT_E_INVALID_ARG for depth < 2 (C must hold one 128-wide head
 * per 128 columns) or a null `out`. */
gpt_status gpt_config_from_depth(int32_t depth, int32_t dtype, gpt_config* out);

/* Checks a config against what the kernels implement. Host only. */
gpt_status gpt_config_validate(const gpt_config* cfg);

/* Number of parameters (elements). Host only; -1 if cfg is invalid.
 * Layout queries accept any n_kv_head >= 1 so that multi-head counts can be
 * checked; gpt_init accepts only n_kv_head == 1. */
int64_t gpt_param_count(const gpt_config* cfg);

/* Fills out[0..*n) with the canonical parameter order: wte [V, C]; per layer
 * w_qkv [(H + 2*n_kv_head)*D, C] (query heads, then K heads, then V heads),
 * w_o [C, H*D], w_1 [F, C], w_2 [C, F]; lm_head [V, C]; then, when enabled,
 * the value-embedding tables h<l>.ve [V, n_kv_head*D] (l = 0, 2, 4, ...),
 * resid_lambdas [1, n_layer], x0_lambdas [1, n_layer], ve_gates [1, n_ve].
 * On entry *n is the capacity of `out`; on return it is the number of
 * tensors (2 + 4*n_layer without the options). `out` may be NULL to query
 * the count. Host only. */
gpt_status gpt_param_layout(const gpt_config* cfg, gpt_tensor_desc* out, int32_t* n);

/* Bytes of device workspace gpt_init needs for batches up to max_B x max_T.
 * Host only. */
gpt_status gpt_workspace_bytes(const gpt_config* cfg, int32_t max_B, int32_t max_T, size_t* bytes);

/* Sets up one model for training steps on the caller's memory: fp32 gradients
 * beside parameters in the compute dtype (aimarketly.com "nanochat-train"
 * README, section "Precision / dtype": bf16 compute, fp32 master weights and
 * gradients), RoPE tables with base 10,000 (aethryn.com, section "A
 * Llama-class transformer with ten modern departures").
 * Creates a handle. `params` is the flat parameter buffer in the config dtype
 * (read only, never written); `grads` the flat fp32 gradient buffer with the
 * same offsets; `workspace` a device buffer of at least
 * gpt_workspace_bytes(cfg, max_B, max_T) bytes, 256-byte aligned. All three are
 * device pointers owned by the caller and must outlive the handle. Uploads
 * the RoPE cos/sin tables into the workspace on `stream`. */
gpt_status gpt_init(const gpt_config* cfg, const void* params, float* grads, void* workspace,
                    size_t ws_bytes, int32_t max_B, int32_t max_T, void* stream, gpt_model** out);

/* The forward pass of one pretraining step (aethryn.com "Nanochat: full-stack
 * LLM training in 8,000 lines for $72", section "A Llama-class transformer
 * with ten modern departures": embedding, RMSNorm before every block and the
 * head, RoPE then QK-norm, causal attention, relu^2 MLP, untied head with the
 * 15*tanh(z/15) softcap in fp32; energyai.berlin "nanochat vs GPT-OSS",
 * section "Architectural decisions": multi-query attention) and its loss,
 * the mean cross-entropy of the next token.
 * Forward pass and mean cross-entropy loss over all B*T positions.
 * idx, targets: device int32 [B, T] row-major; targets are the next tokens,
 * each in [0, V). loss: device fp32 scalar. row_loss: optional device fp32
 * [B*T] per-position losses (may be NULL). need_grad = 1 keeps the stash that
 * gpt_backward consumes; idx and targets must then stay valid until that
 * gpt_backward has run (it reads them again). An id outside [0, V) sets the
 * sticky device flag (read by gpt_sync_status) and makes the loss NaN.
 * Asynchronous. */
gpt_status gpt_forward_loss(gpt_model* m, const int32_t* idx, const int32_t* targets, int32_t B,
                            int32_t T, int32_t need_grad, float* loss, float* row_loss, void* stream);

/* The backward pass of the same step, written as dloss times the gradient so
 * that a caller can average micro-batches, and with `accumulate` for the
 * gradient accumulation a single GPU runs in place of eight (aimarketly.com
 * "nanochat-train" README, section "Getting started").
 * Backward of the last need_grad forward: grads = dloss * d(loss)/d(theta).
 * accumulate = 1 adds into the gradient buffer; 0 overwrites all of it
 * (including embedding rows no token touched). GPT_E_STATE if no forward is
 * pending. Asynchronous. */
gpt_status gpt_backward(gpt_model* m, float dloss, int32_t accumulate, void* stream);

/* Synchronises `stream` and reads the sticky device flag: GPT_E_DEVICE if a
 * kernel flagged bad input since gpt_init, else GPT_OK. */
gpt_status gpt_sync_status(gpt_model* m, void* stream);

/* Frees the handle (host memory only). */
gpt_status gpt_destroy(gpt_model* m);

/* Measurement support. gpt_profile_begin arms timing of every launch whose
 * kernel tag equals `tag` (see gpt_kernel_tag_name) with HIP events on the
 * stream the kernel runs on, or of every launch if tag < 0; gpt_profile_end
 * synchronises and returns the summed duration in milliseconds and the number
 * of timed launches, and disarms. At most 65536 launches are timed. */
gpt_status gpt_profile_begin(gpt_model* m, int32_t tag);
gpt_status gpt_profile_end(gpt_model* m, double* total_ms, int64_t* launches);

/* Options of a handle (take effect for the following calls).
 * GPT_OPT_GEMM_TILE: 0 (default) picks each GEMM's tile by its shape;
 * 1..3 force one tile variant for every GEMM, largest first (bf16
 * k-contiguous GEMMs: 256x256, 256x128 with two workgroups per CU, 128x128;
 * others: 256x256, 128x128, 64x64). Results are the same up to rounding
 * order; the option exists to measure and test every variant.
 * GPT_OPT_DKV_HSPLIT: bf16 attention backward, dK/dV kernel. 0 (default)
 * picks by grid size: each 128-key block of a batch row sums dK and dV over
 * all H query heads in one workgroup (1), or, when that grid would give
 * fewer than two rounds of workgroups per compute unit or the layer has a
 * sliding window, over two workgroups of H/2 heads each whose fp32 partial
 * rows a combine kernel adds in order (2). 1 or 2 force that form (2 needs
 * an even H, else 1 is used). Same result up to rounding order; the option
 * exists to test both forms at any size.
 * GPT_OPT_RESID_GRAD: where a bf16 model keeps the gradient of the residual
 * stream through the backward. 0 (default): in bf16, as for any gradient of
 * a bf16 activation (each kernel adds in fp32 and rounds once); 1: in fp32
 * (the bf16 copy the weight-gradient and dX products read is still made).
 * fp32 models, and models with the residual scalars (x0_lambdas), keep it in
 * fp32 either way. */
enum { GPT_OPT_GEMM_TILE = 1, GPT_OPT_DKV_HSPLIT = 2, GPT_OPT_RESID_GRAD = 3 };
gpt_status gpt_set_option(gpt_model* m, int32_t option, int32_t value);

/* Name of a kernel tag (NULL past the last tag); tags run 0..n-1. */
const char* gpt_kernel_tag_name(int32_t tag);

/* Debug access to a stashed activation of the last forward: device pointer and
 * byte size of the named buffer ("x", "h1", "qkv", "o", "lse", "h2", "a",
 * "hf", "logits", "rstd0"; FP8 models also "amax") for `layer` (ignored by
 * non-layer buffers). The pointer aliases the workspace and is valid until
 * the next call. "lse" holds the attention log-sum-exp per (batch row, head,
 * position) in base 2, i.e. ln(sum) * log2(e), fp32 [B, H, T]. "logits" holds
 * what the LM head stores for the backward, q = exp(z' - c) (1 - (z'/c)^2)
 * per row and vocabulary entry (z' = c tanh(z/c), c the softcap), activation
 * dtype [B*T, V]; a backward overwrites the target entries. "du" and "dqkv"
 * (no layer) hold the last backward's gradients at the MLP's hidden
 * activation [B*T, mlp_dim] and at the QKV projection's output
 * [B*T, (H+2)*128] of layer 0 (scratch reused layer by layer). "amax" holds
 * the layer's 16 fp32 |max| slots of the FP8 operands: h1, o, h2, a (forward
 * inputs of the QKV, O, W1, W2 products), the output gradients of W2 and W1
 * (d(out) of the MLP, du), of O and of QKV, then W_qkv, W_o, W_1, W_2, then 4
 * unused. */
gpt_status gpt_debug_buffer(gpt_model* m, const char* name, int32_t layer, void** ptr, size_t* bytes);

/* The per-tensor e4m3 quantisation FP8 models apply to every QKV / O / MLP
 * operand (see GPT_FP8_E4M3), exposed on its own. x: device bf16 [rows, cols]
 * row-major, cols a multiple of 16. Sets *amax (device fp32) to max|x|, then
 * writes codes e4m3(clamp(x * s, -448, 448)), s = 448 / amax computed in fp32
 * (1 if amax is 0), round to nearest even: q (device, may be NULL) [rows, cols]
 * row-major; qT (device, may be NULL) [cols, ldT] transposed, with columns
 * rows..ldT-1 set to code 0 (ldT >= rows, a multiple of 16). Codes: bit 7
 * sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa; 0x7f NaN. All
 * buffers are caller-owned, 16-byte aligned (amax 4-byte). GPT_E_INVALID_ARG
 * on bad sizes or pointers. Asynchronous on `stream`. */
gpt_status gpt_fp8_quantize(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* qT, int64_t ldT,
                            float* amax, void* stream);

/* The e4m3 matmul FP8 models run for their QKV / O / MLP products (see
 * GPT_FP8_E4M3), exposed on its own: out[m, n] = sum_k (a[m, k] / s_a) *
 * (b[n, k] / s_b), with a, b e4m3 codes as gpt_fp8_quantize writes them (a
 * [M, K] and b [N, K], both k-contiguous, row pitches lda, ldb >= K,
 * multiples of 16) and s = 448 / *amax (1 if *amax is 0) read from the device
 * fp32 slots amax_a, amax_b. The products accumulate in fp32. out: device
 * [M, N], row pitch ldo >= N (a multiple of 4), fp32 (out_dtype GPT_F32) or
 * bf16 rounded to nearest even (GPT_BF16). K must be a multiple of 128, N of
 * 4; all pointers 16-byte aligned. tile: 0 picks the tile by shape, 1..3
 * force 256x256, 256x128, 128x128. splits > 1 (fp32 output only) splits K
 * into that many slices whose partial sums go to `partials` (device fp32
 * [splits, M, N], caller-owned) and are added in slice order.
 * GPT_E_INVALID_ARG on bad sizes or pointers. Asynchronous on `stream`. */
gpt_status gpt_fp8_matmul(const uint8_t* a, int64_t lda, const float* amax_a, const uint8_t* b, int64_t ldb,
                          const float* amax_b, int32_t M, int32_t N, int32_t K, int32_t out_dtype, void* out,
                          int64_t ldo, int32_t tile, int32_t splits, float* partials, void* stream);

/* gpt_fp8_matmul for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and result, but split-K partials (splits > 1) go to a
 * fixed device array inside the library instead of a caller buffer. The array
 * holds 4,194,304 floats (16 MiB) on each GPU the library runs on, kept until
 * the process ends; splits * M * N above that is GPT_E_INVALID_ARG. Nothing
 * is allocated: the array's address on the current device is looked up on
 * the first call made on that device. Every call on one GPU shares that GPU's
 * array, so calls with splits > 1 that overlap on one GPU (other streams or
 * threads) race and must be serialised by the caller. */
gpt_status gpt_fp8_matmul_noalloc(const uint8_t* a, int64_t lda, const float* amax_a, const uint8_t* b,
                                  int64_t ldb, const float* amax_b, int32_t M, int32_t N, int32_t K,
                                  int32_t out_dtype, void* out, int64_t ldo, int32_t tile, int32_t splits,
                                  void* stream);

/* ---- The optimiser step after the backward ------------------------------
 * Muon for the blocks' matrix weights (w_qkv, w_o, w_1, w_2), AdamW for the
 * embeddings (wte and the value-embedding tables), the unembedding (lm_head)
 * and the scalars, on fp32 master weights whose cast to the config dtype
 * (round to nearest even) becomes the model's parameters (atlas.blal.pro
 * "nanochat — full-stack ChatGPT in ~8k lines", section "How it works", item
 * "2. Pretrain"; aethryn.com "Nanochat: full-stack LLM training in 8,000 lines
 * for $72", section "A Llama-class transformer with ten modern departures";
 * energyai.berlin "nanochat vs GPT-OSS", section "Muon optimizer").
 * AdamW: w <- w (1 - lr wd); m <- b1 m + (1 - b1) g; v <- b2 v + (1 - b2) g^2;
 * w <- w - lr / (1 - b1^t) * m / (sqrt(v) / sqrt(1 - b2^t) + eps).
 * Muon: u <- momentum u + g; X_0 = u / (||u||_F + 1e-7) in the orientation
 * with fewer rows; ns_steps times X <- a X + (b A + c A^2) X with A = X X^T
 * (products in the config dtype, fp32 accumulation); w <- w (1 - lr wd) -
 * lr sqrt(max(1, rows / cols)) X. (a, b, c) = (1.5, -0.5, 0) is the cubic
 * Newton-Schulz iteration towards the orthogonal polar factor of u. The
 * caller applies its own schedules through the per-step values. */
typedef struct gpt_optim_config {
  float lr_muon, lr_embed, lr_unembed, lr_scalar;
  float momentum;          /* Muon momentum of this step */
  float beta1, beta2, eps; /* AdamW */
  float wd_muon, wd_adamw; /* decoupled weight decay of each group */
  int32_t ns_steps;        /* 0..100 */
  float ns_a, ns_b, ns_c;
} gpt_optim_config;

/* fp32 elements of optimiser state: per parameter tensor in the canonical
 * order, Muon tensors hold u [rows, cols], AdamW tensors m then v [rows, cols]
 * each. Host only. */
gpt_status gpt_optimizer_state_elems(const gpt_config* cfg, int64_t* elems);

/* One optimiser step from the gradient buffer of the handle (as the last
 * gpt_backward left it). master: device fp32 [param_count] master weights,
 * updated in place; state: device fp32 [gpt_optimizer_state_elems], zero
 * before the first step; t: the 1-based step number (bias correction).
 * Writes the cast of the updated masters into the parameter buffer given to
 * gpt_init (the only call that writes it). Uses the handle's workspace as
 * scratch. Asynchronous on `stream`; GPT_E_INVALID_ARG on bad arguments. */
gpt_status gpt_optimizer_step(gpt_model* m, const gpt_optim_config* oc, float* master, float* state, int32_t t,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPT_AMD_GPT_H */
