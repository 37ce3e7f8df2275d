// Host side of the library: configuration, parameter layout, workspace
// planning and the forward/backward schedule of one pretraining step.
//
// Step structure (aethryn.com "Nanochat: full-stack LLM training in 8,000 lines
// for $72", section "A Llama-class transformer with ten modern departures";
// atlas.blal.pro "nanochat — full-stack ChatGPT in ~8k lines", section
// "How it works", item 0): x = rmsnorm(wte[idx]); per layer
// x += W_o attn(rope_qknorm(W_qkv rmsnorm(x))), x += W_2 relu(W_1 rmsnorm(x))^2;
// logits = softcap(W_lm rmsnorm(x)); loss = mean cross-entropy.
//
// The library owns no device memory: the caller hands in parameters,
// gradients and one workspace, which is carved up here.
//
// FP8 models (repo-explainer.com "karpathy/nanochat: The $100 Full-Stack
// LLM", section "The Engine Room: Muon and FP8"; atlas.blal.pro, section "How
// it works", item "2. Pretrain": optional FP8 matmuls) keep bf16 parameters
// and activations and run the QKV, O and MLP products -- forward, dX and dW --
// on per-tensor-scaled e4m3 operands: each operand tensor gets its |max|
// (amax pass), then its codes (quantise pass), row-major for the forward and
// dX products and token-major (transposed, tokens padded to 128 with zeros)
// for dW, so that every fp8 product is one k-contiguous GEMM. The layer
// weights are quantised once per forward and reused by the backward.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/gpt.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

gpt_status fail(gpt_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

#define HIP_TRY(expr)                                                                    \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess)                                                                \
      return fail(GPT_E_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, __LINE__); \
  } while (0)

constexpr int kHeadDim = 128;

// Kernel tags (measurement). Order fixes the tag numbers.
enum Tag : int {
  K_EMBED = 0, K_RMSNORM, K_GEMM_QKV, K_ROPE_QKNORM, K_ATTN_FWD_PREP, K_ATTN_FWD, K_GEMM_O, K_GEMM_W1, K_GEMM_W2,
  K_GEMM_LM, K_CE_LOSS, K_CE_BWD, K_GEMM_LM_DW, K_GEMM_LM_DX, K_RMSNORM_BWD, K_GEMM_W2_DW, K_GEMM_W2_DX,
  K_GEMM_W1_DW, K_GEMM_W1_DX, K_GEMM_O_DW, K_GEMM_O_DX, K_ATTN_BWD_PREP, K_ATTN_BWD_DQ, K_ATTN_BWD_DKV,
  K_ROPE_QKNORM_BWD, K_GEMM_QKV_DW, K_GEMM_QKV_DX, K_EMBED_BWD, K_WEIGHT_T, K_FP8_AMAX, K_FP8_QUANT,
  K_FP8_WEIGHTS, K_EMBED_SORT, K_X0_MIX, K_X0_MIX_BWD, K_VE_ADD, K_VE_BWD, K_OPT_ADAMW, K_OPT_MUON, K_NUM_TAGS
};

// |max| slots per layer of an FP8 model (fp32, zeroed at every forward)
enum AmaxSlot : int {
  A_H1 = 0, A_O, A_H2, A_A, A_DY_MLP, A_DU, A_DY_ATTN, A_DQKV, A_W_QKV, A_W_O, A_W_1, A_W_2, kAmaxSlots = 16
};
const char* kTagNames[K_NUM_TAGS] = {
  "embed_rmsnorm", "rmsnorm", "gemm_qkv", "rope_qknorm", "attn_fwd_transpose", "attn_fwd", "gemm_o",
  "gemm_w1_relu2", "gemm_w2", "gemm_lm_head_softcap", "ce_loss", "ce_bwd", "gemm_lm_head_dw", "gemm_lm_head_dx",
  "rmsnorm_bwd", "gemm_w2_dw", "gemm_w2_dx", "gemm_w1_dw", "gemm_w1_dx_relu2bwd", "gemm_o_dw", "gemm_o_dx",
  "attn_bwd_prep", "attn_bwd_dq", "attn_bwd_dkv", "rope_qknorm_bwd", "gemm_qkv_dw", "gemm_qkv_dx", "embed_bwd",
  "weight_transpose", "fp8_amax", "fp8_quantize", "fp8_weights", "embed_sort", "x0_mix", "x0_mix_bwd", "ve_add",
  "ve_bwd", "opt_adamw", "opt_muon"};

struct Layout {  // byte offsets inside the workspace
  size_t flag, loss_rows, rope_cos, rope_sin;
  size_t x, rstd0, hf, rstdf, logits, part, ztgt, lse_ce, ce_rscale;
  std::vector<size_t> h1, rstd1, qkv, rstd_qk, o, lse, h2, rstd2, a;
  size_t dres, dres_lp, dh, du, dqkv, dout, delta, dkv_part, split;
  size_t qT, kT, vT, doT;  // attention's transposed copies [B, heads, 128, Tp]
  size_t wT, tdesc;        // transposed weights (bf16 models) and their descriptor table
  // FP8 models: amax slots; e4m3 codes of the layer weights (row-major and
  // transposed, at each parameter's element offset) and their descriptor
  // table; row-major codes of the current forward operand; per-layer
  // token-major codes of the forward operands (kept for dW); codes of the
  // current output gradient, row-major and token-major
  size_t amax, wq, wqT, qdesc, xq, dyq, dyqT;
  std::vector<size_t> h1qT, oqT, h2qT, aqT;
  // residual scalars: x0 (the normalised embedding), the stream before each
  // layer's mix, the gradient reaching x0 through the mixes; partial sums of
  // the scalar gradients
  size_t x0, dx0acc, rpart;
  std::vector<size_t> xprev;
  // optimiser scratch: Newton-Schulz iterates and products, norm partials
  size_t ns_x, ns_xt, ns_a, ns_aa, ns_b, ns_part, ns_inv;
  int ns_batch;  // Muon matrices per batched launch
  size_t keys_a, vals_a, keys_b, vals_b, hist, carry;
  size_t total;
  size_t split_elems;
};

size_t esize(int dtype) { return dtype == GPT_F32 ? 4 : 2; }  // bf16 storage for GPT_BF16 and GPT_FP8_E4M3

// Padded token count of the token-major fp8 codes (the dW products' K).
int64_t pad_tokens(int64_t n) { return (n + 127) / 128 * 128; }

struct Planner {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  }
};

// Split-K slices for a dW GEMM [M, N] reduced over K tokens (256x256 tiles,
// one CTA per CU, 256 CUs). Candidates give at least one full round of CTAs
// (at least 1024 k per slice, at most 32 slices; requiring two rounds had
// cost the QKV and O dW 24 and 30 slices of partial traffic). Score of a
// slice count t: the busy fraction of the rounds. The fewest slices scoring
// at least 0.93 (each slice adds an M x N fp32 partial that is written and
// read back), else the best score. (A handicap for tiles * t not a multiple
// of 8, meant to keep whole slices on one XCD, doubled the MLP dW slices to
// 10 and cost each of them about 1 ms per d20 step.)
int dw_splits(int M, int N, int K) {
  const int64_t tiles = (int64_t)((M + 255) / 256) * ((N + 255) / 256);
  const int cap = std::min(32, std::max(1, K / 1024));
  int best = cap;
  double best_score = -1.0;
  for (int t = 1; t <= cap; ++t) {
    const int64_t blocks = tiles * t;
    if (blocks < 256 && t < cap) continue;
    const int64_t rounds = (blocks + 255) / 256;
    double score = (double)blocks / (double)(rounds * 256);
    if (score >= 0.93) return t;
    if (score > best_score + 1e-9) {
      best_score = score;
      best = t;
    }
  }
  return best;
}

// Sliding window of layer l (0 = full causal prefix): the pattern repeats over
// the layers, 'S' selects window_short, and the last layer is always full.
int layer_window(const gpt_config& c, int l) {
  const int n = (int)strnlen(c.window_pattern, sizeof(c.window_pattern));
  if (n == 0 || c.window_short <= 0 || l == c.n_layer - 1) return 0;
  return c.window_pattern[l % n] == 'S' ? c.window_short : 0;
}

// Value-embedding layers (0, 2, 4, ...) and their count.
bool ve_layer(const gpt_config& c, int l) { return c.value_embeds != 0 && l % 2 == 0; }
int n_ve_layers(const gpt_config& c) { return c.value_embeds != 0 ? (c.n_layer + 1) / 2 : 0; }

Layout plan(const gpt_config& c, int maxB, int maxT) {
  Layout L{};
  Planner p;
  const size_t N = (size_t)maxB * maxT, C = c.model_dim, H = c.n_head, F = c.mlp_dim, V = c.vocab_size;
  const size_t es = esize(c.dtype);
  const size_t QKV = (H + 2) * kHeadDim;
  L.flag = p.take(256);
  L.loss_rows = p.take(N * 4);
  L.rope_cos = p.take((size_t)maxT * 64 * 4);
  L.rope_sin = p.take((size_t)maxT * 64 * 4);
  L.x = p.take(N * C * es);
  L.rstd0 = p.take(N * 4);
  for (int l = 0; l < c.n_layer; ++l) {
    L.h1.push_back(p.take(N * C * es));
    L.rstd1.push_back(p.take(N * 4));
    L.qkv.push_back(p.take(N * QKV * es));
    L.rstd_qk.push_back(p.take(N * (H + 1) * 4));
    L.o.push_back(p.take(N * H * kHeadDim * es));
    L.lse.push_back(p.take(N * H * 4));
    L.h2.push_back(p.take(N * C * es));
    L.rstd2.push_back(p.take(N * 4));
    L.a.push_back(p.take(N * F * es));
  }
  L.hf = p.take(N * C * es);
  L.rstdf = p.take(N * 4);
  L.logits = p.take(N * V * es);
  L.part = p.take(N * (V / gk::kLMHeadPartCols) * 4);
  L.ztgt = p.take(N * 4);
  L.lse_ce = p.take(N * 4);
  L.ce_rscale = p.take(N * 4);
  L.dres = p.take(N * C * 4);
  L.dres_lp = p.take(N * C * es);
  L.dh = p.take(N * C * es);
  L.du = p.take(N * F * es);
  L.dqkv = p.take(N * QKV * es);
  L.dout = p.take(N * H * kHeadDim * es);
  L.delta = p.take(N * H * 4);
  L.dkv_part = p.take(2 * N * 2 * kHeadDim * 4);
  {
    const size_t Tp = (size_t)gk::attn_padded_len(maxT), BT = (size_t)maxB * Tp * kHeadDim;
    L.qT = p.take(BT * H * es);
    L.doT = p.take(BT * H * es);
    L.kT = p.take(BT * es);
    L.vT = p.take(BT * es);
  }
  // split-K partial buffer: largest splits*M*N over the per-layer dW GEMMs
  // (calls with fewer tokens clamp their slice count to this buffer)
  size_t se = 0;
  const int K = c.dtype == GPT_FP8_E4M3 ? (int)pad_tokens((int64_t)N) : (int)N;
  auto upd = [&](int M, int Nn) {
    int s = dw_splits(M, Nn, K);
    if (s > 1) se = std::max(se, (size_t)s * M * Nn);
  };
  upd((int)QKV, (int)C);
  upd((int)C, (int)(H * kHeadDim));
  upd((int)F, (int)C);
  upd((int)C, (int)F);
  upd((int)V, (int)C);
  L.split_elems = se;
  L.split = p.take(se * 4);
  {
    const int64_t np = gpt_param_count(&c);
    L.wT = c.dtype != GPT_F32 ? p.take((size_t)np * es) : p.take(0);
    L.tdesc = p.take((size_t)(2 + 4 * c.n_layer) * sizeof(gk::TransposeDesc));
  }
  if (c.dtype == GPT_FP8_E4M3) {
    const size_t np = (size_t)gpt_param_count(&c), Np = (size_t)pad_tokens((int64_t)N);
    const size_t widest = std::max(QKV, std::max(C, F));
    L.amax = p.take((size_t)c.n_layer * kAmaxSlots * 4);
    L.wq = p.take(np);
    L.wqT = p.take(np);
    L.qdesc = p.take((size_t)4 * c.n_layer * sizeof(gk::QuantDesc));
    L.xq = p.take(N * std::max(C, F));
    L.dyq = p.take(N * widest);
    L.dyqT = p.take(widest * Np);
    for (int l = 0; l < c.n_layer; ++l) {
      L.h1qT.push_back(p.take(C * Np));
      L.oqT.push_back(p.take(H * kHeadDim * Np));
      L.h2qT.push_back(p.take(C * Np));
      L.aqT.push_back(p.take(F * Np));
    }
  }
  if (c.x0_lambdas) {
    L.x0 = p.take(N * C * es);
    L.dx0acc = p.take(N * C * 4);
    for (int l = 0; l < c.n_layer; ++l) L.xprev.push_back(p.take(N * C * es));
  }
  L.rpart = (c.x0_lambdas || c.value_embeds) ? p.take(gk::resid_partials_elems() * 4) : p.take(0);
  {
    // the largest Muon matrix (elements) and its smaller side
    const size_t mats[4][2] = {{QKV, C}, {C, H * kHeadDim}, {F, C}, {C, F}};
    size_t big = 0, small2 = 0;
    for (auto& mm : mats) {
      big = std::max(big, mm[0] * mm[1]);
      const size_t sm = std::min(mm[0], mm[1]);
      small2 = std::max(small2, sm * sm);
    }
    // one matrix per layer has each shape: batches of up to kMuonBatch layers
    const size_t nb = (size_t)std::max(1, std::min(gk::kMuonBatch, c.n_layer));
    L.ns_batch = (int)nb;
    L.ns_x = p.take(nb * big * es);
    L.ns_xt = p.take(nb * big * es);
    L.ns_a = p.take(nb * small2 * es);
    L.ns_aa = p.take(nb * small2 * es);
    L.ns_b = p.take(nb * small2 * es);
    L.ns_part = p.take(nb * gk::muon_partials_elems() * 4);
    L.ns_inv = p.take(nb * 4);
  }
  L.keys_a = p.take(N * 4);
  L.vals_a = p.take(N * 4);
  L.keys_b = p.take(N * 4);
  L.vals_b = p.take(N * 4);
  L.hist = p.take(gk::embed_bwd_hist_elems((int)N) * 4);
  L.carry = p.take(gk::embed_bwd_carry_elems((int)N, (int)C) * 4);
  L.total = p.off;
  return L;
}

// Layout checks that do not depend on kernel support.
gpt_status check_shape(const gpt_config* c) {
  if (!c) return fail(GPT_E_INVALID_ARG, "config is NULL");
  if (c->n_layer < 1 || c->model_dim < 1 || c->n_head < 1 || c->n_kv_head < 1 || c->head_dim < 1 ||
      c->mlp_dim < 1 || c->vocab_size < 1 || c->max_seq_len < 1)
    return fail(GPT_E_INVALID_ARG, "config sizes must be positive");
  return GPT_OK;
}

struct Profiler {
  bool armed = false;
  int tag = -1;
  std::vector<hipEvent_t> ev;  // pairs
  size_t used = 0;             // pairs used
  static constexpr size_t kCap = 65536;
};

}  // namespace

struct gpt_model {
  gpt_config cfg;
  const void* params;
  float* grads;
  char* ws;
  size_t ws_bytes;
  int maxB, maxT;
  Layout L;
  // parameter offsets (elements)
  int64_t off_wte, off_lm;
  std::vector<int64_t> off_qkv, off_o, off_w1, off_w2;
  std::vector<int64_t> off_ve;                      // per layer, -1 without a value embedding
  int64_t off_resid = -1, off_x0lam = -1, off_gates = -1;
  int gemm_tile = 0;      // GPT_OPT_GEMM_TILE
  int dkv_hsplit = 0;     // GPT_OPT_DKV_HSPLIT
  int resid_grad_f32 = 0; // GPT_OPT_RESID_GRAD
  int ntdesc = 0;
  int64_t wt_tiles = 0;   // total 64x64 tiles of the batched weight transpose
  int nqdesc = 0;                         // FP8: layer-weight quantisation table
  int64_t wq_amax_blocks = 0, wq_blocks = 0;
  // state of the last forward
  bool pending = false;
  int B = 0, T = 0;
  const int32_t* idx = nullptr;
  const int32_t* targets = nullptr;
  Profiler prof;
};

namespace {

template <typename P>
P* wsp(gpt_model* m, size_t off) { return reinterpret_cast<P*>(m->ws + off); }

const char* pbase(gpt_model* m, int64_t elem_off) {
  return reinterpret_cast<const char*>(m->params) + elem_off * (int64_t)esize(m->cfg.dtype);
}

// Runs `fn` (which enqueues kernels and returns hipError_t) under the given tag.
template <typename Fn>
gpt_status run(gpt_model* m, int tag, hipStream_t s, Fn&& fn) {
  Profiler& P = m->prof;
  const bool timed = P.armed && (P.tag < 0 || P.tag == tag) && P.used < Profiler::kCap;
  if (timed) {
    if (P.ev.size() < 2 * (P.used + 1)) {
      hipEvent_t a, b;
      HIP_TRY(hipEventCreate(&a));
      HIP_TRY(hipEventCreate(&b));
      P.ev.push_back(a);
      P.ev.push_back(b);
    }
    HIP_TRY(hipEventRecord(P.ev[2 * P.used], s));
  }
  hipError_t e = fn();
  if (e != hipSuccess) return fail(GPT_E_HIP, "launch of %s failed: %s", kTagNames[tag], hipGetErrorString(e));
  if (timed) {
    HIP_TRY(hipEventRecord(P.ev[2 * P.used + 1], s));
    P.used++;
  }
  return GPT_OK;
}

#define RUN(tag, body)                                                       \
  do {                                                                       \
    gpt_status st_ = run(m, tag, stream, [&]() -> hipError_t { body });      \
    if (st_ != GPT_OK) return st_;                                           \
  } while (0)
#define TRY(x) do { gpt_status s_ = (x); if (s_ != GPT_OK) return s_; } while (0)

// FP8: amax pass then quantise pass of one bf16 operand [rows, cols]
// (contiguous) into row-major codes q and/or token-major codes qT [cols, ldT].
// amax_ready: the producer of src folded its |max| into amax as it wrote it
gpt_status quantize_operand(gpt_model* m, hipStream_t stream, const void* src, int rows, int cols, uint8_t* q,
                            uint8_t* qT, int64_t ldT, float* amax, bool amax_ready = false) {
  gk::QuantDesc d;
  d.src = src;
  d.ld = cols;
  d.rows = rows;
  d.cols = cols;
  d.q = q;
  d.qT = qT;
  d.ldT = (int32_t)ldT;
  d.amax = amax;
  if (!amax_ready) RUN(K_FP8_AMAX, return gk::launch_fp8_amax(d, stream););
  RUN(K_FP8_QUANT, return gk::launch_fp8_quantize(d, stream););
  return GPT_OK;
}

// dW split count, clamped to the partial buffer the workspace holds.
int dw_splits_ws(const gpt_model* m, int M, int N, int K) {
  int s = dw_splits(M, N, K);
  while (s > 1 && (size_t)s * M * N > m->L.split_elems) --s;
  return s;
}

}  // namespace

extern "C" {

const char* gpt_status_string(gpt_status s) {
  switch (s) {
    case GPT_OK: return "GPT_OK";
    case GPT_E_INVALID_ARG: return "GPT_E_INVALID_ARG";
    case GPT_E_UNSUPPORTED: return "GPT_E_UNSUPPORTED";
    case GPT_E_WORKSPACE: return "GPT_E_WORKSPACE";
    case GPT_E_STATE: return "GPT_E_STATE";
    case GPT_E_HIP: return "GPT_E_HIP";
    case GPT_E_DEVICE: return "GPT_E_DEVICE";
    default: return "GPT_E_UNKNOWN";
  }
}

const char* gpt_last_error_message(void) { return g_last_error.c_str(); }

gpt_status gpt_config_from_depth(int32_t depth, int32_t dtype, gpt_config* out) {
  if (!out) return fail(GPT_E_INVALID_ARG, "out is NULL");
  if (depth < 2) return fail(GPT_E_INVALID_ARG, "depth must be >= 2 (width 64*depth holds 128-wide heads)");
  if (dtype != GPT_F32 && dtype != GPT_BF16 && dtype != GPT_FP8_E4M3)
    return fail(GPT_E_INVALID_ARG, "dtype must be GPT_F32, GPT_BF16 or GPT_FP8_E4M3");
  gpt_config c;
  c.n_layer = depth;
  c.model_dim = 64 * depth;
  c.n_head = c.model_dim / kHeadDim;
  c.n_kv_head = 1;
  c.head_dim = kHeadDim;
  c.mlp_dim = 4 * c.model_dim;
  c.vocab_size = 65536;
  c.max_seq_len = 2048;
  c.rope_theta = 10000.f;
  c.logit_softcap = 15.f;
  c.norm_eps = 1.1920928955078125e-07f;  // 2^-23
  c.dtype = dtype;
  c.window_short = 0;
  std::memset(c.window_pattern, 0, sizeof(c.window_pattern));
  c.x0_lambdas = 0;
  c.value_embeds = 0;
  *out = c;
  return GPT_OK;
}

gpt_status gpt_config_validate(const gpt_config* c) {
  gpt_status s = check_shape(c);
  if (s != GPT_OK) return s;
  if (c->dtype != GPT_F32 && c->dtype != GPT_BF16 && c->dtype != GPT_FP8_E4M3)
    return fail(GPT_E_UNSUPPORTED, "dtype %d not supported", c->dtype);
  if (c->n_kv_head != 1) return fail(GPT_E_UNSUPPORTED, "n_kv_head must be 1 (multi-query attention)");
  if (c->head_dim != kHeadDim) return fail(GPT_E_UNSUPPORTED, "head_dim must be 128");
  if (c->n_head * c->head_dim != c->model_dim)
    return fail(GPT_E_UNSUPPORTED, "n_head * head_dim must equal model_dim");
  if (c->model_dim % 128 != 0 || c->model_dim > 4096)
    return fail(GPT_E_UNSUPPORTED, "model_dim must be a multiple of 128 and <= 4096");
  if (c->mlp_dim % 128 != 0) return fail(GPT_E_UNSUPPORTED, "mlp_dim must be a multiple of 128");
  if (c->vocab_size % 256 != 0 || c->vocab_size > 65536)
    return fail(GPT_E_UNSUPPORTED, "vocab_size must be a multiple of 256 and <= 65536");
  if (!(c->logit_softcap > 0.f) || !(c->norm_eps > 0.f) || !(c->rope_theta > 0.f))
    return fail(GPT_E_INVALID_ARG, "rope_theta, logit_softcap and norm_eps must be positive");
  bool nul = false, any_short = false;
  for (int i = 0; i < (int)sizeof(c->window_pattern); ++i) {
    const char ch = c->window_pattern[i];
    if (ch == 0) {
      nul = true;
      break;
    }
    if (ch != 'S' && ch != 'L') return fail(GPT_E_INVALID_ARG, "window_pattern may hold only 'S' and 'L'");
    any_short |= ch == 'S';
  }
  if (!nul) return fail(GPT_E_INVALID_ARG, "window_pattern must be NUL-terminated within 8 bytes");
  if (any_short && c->window_short < 1) return fail(GPT_E_INVALID_ARG, "window_short must be >= 1 for 'S' layers");
  if (c->window_short < 0) return fail(GPT_E_INVALID_ARG, "window_short must be >= 0");
  if ((c->x0_lambdas != 0 && c->x0_lambdas != 1) || (c->value_embeds != 0 && c->value_embeds != 1))
    return fail(GPT_E_INVALID_ARG, "x0_lambdas and value_embeds must be 0 or 1");
  return GPT_OK;
}

int64_t gpt_param_count(const gpt_config* c) {
  if (check_shape(c) != GPT_OK) return -1;
  const int64_t C = c->model_dim, H = c->n_head, Hkv = c->n_kv_head, D = c->head_dim, F = c->mlp_dim,
                V = c->vocab_size;
  const int64_t per_layer = (H + 2 * Hkv) * D * C + C * H * D + F * C + C * F;
  const int64_t nve = c->value_embeds ? (c->n_layer + 1) / 2 : 0;
  return 2 * V * C + c->n_layer * per_layer + nve * (V * Hkv * D + 1) + (c->x0_lambdas ? 2 * c->n_layer : 0);
}

gpt_status gpt_param_layout(const gpt_config* c, gpt_tensor_desc* out, int32_t* n) {
  gpt_status s = check_shape(c);
  if (s != GPT_OK) return s;
  if (!n) return fail(GPT_E_INVALID_ARG, "n is NULL");
  const int32_t nve = c->value_embeds ? (c->n_layer + 1) / 2 : 0;
  const int32_t count = 2 + 4 * c->n_layer + nve + (c->x0_lambdas ? 2 : 0) + (nve ? 1 : 0);
  if (!out) {
    *n = count;
    return GPT_OK;
  }
  if (*n < count) return fail(GPT_E_INVALID_ARG, "capacity %d < %d tensors", *n, count);
  const int64_t C = c->model_dim, H = c->n_head, Hkv = c->n_kv_head, D = c->head_dim, F = c->mlp_dim,
                V = c->vocab_size;
  int64_t off = 0;
  int k = 0;
  auto add = [&](const char* name, int64_t r, int64_t cc) {
    gpt_tensor_desc& d = out[k++];
    memset(d.name, 0, sizeof(d.name));
    snprintf(d.name, sizeof(d.name), "%s", name);
    d.offset = off;
    d.rows = r;
    d.cols = cc;
    off += r * cc;
  };
  add("wte", V, C);
  char nm[32];
  for (int l = 0; l < c->n_layer; ++l) {
    snprintf(nm, sizeof(nm), "h%d.w_qkv", l); add(nm, (H + 2 * Hkv) * D, C);
    snprintf(nm, sizeof(nm), "h%d.w_o", l); add(nm, C, H * D);
    snprintf(nm, sizeof(nm), "h%d.w_1", l); add(nm, F, C);
    snprintf(nm, sizeof(nm), "h%d.w_2", l); add(nm, C, F);
  }
  add("lm_head", V, C);
  for (int l = 0; l < c->n_layer; l += 2)
    if (c->value_embeds) {
      snprintf(nm, sizeof(nm), "h%d.ve", l);
      add(nm, V, Hkv * D);
    }
  if (c->x0_lambdas) {
    add("resid_lambdas", 1, c->n_layer);
    add("x0_lambdas", 1, c->n_layer);
  }
  if (nve) add("ve_gates", 1, nve);
  *n = count;
  return GPT_OK;
}

gpt_status gpt_workspace_bytes(const gpt_config* c, int32_t max_B, int32_t max_T, size_t* bytes) {
  gpt_status s = gpt_config_validate(c);
  if (s != GPT_OK) return s;
  if (!bytes) return fail(GPT_E_INVALID_ARG, "bytes is NULL");
  if (max_B < 1 || max_T < 1 || max_T > c->max_seq_len)
    return fail(GPT_E_INVALID_ARG, "need 1 <= max_B and 1 <= max_T <= max_seq_len");
  if ((int64_t)max_B * max_T > (int64_t)1 << 24) return fail(GPT_E_INVALID_ARG, "max_B * max_T too large");
  *bytes = plan(*c, max_B, max_T).total;
  return GPT_OK;
}

gpt_status gpt_init(const gpt_config* cfg, const void* params, float* grads, void* workspace, size_t ws_bytes,
                    int32_t max_B, int32_t max_T, void* stream_, gpt_model** out) {
  if (!out) return fail(GPT_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  gpt_status s = gpt_config_validate(cfg);
  if (s != GPT_OK) return s;
  if (!params || !grads || !workspace) return fail(GPT_E_INVALID_ARG, "params, grads and workspace must be non-NULL");
  if (((uintptr_t)workspace & 255) != 0) return fail(GPT_E_INVALID_ARG, "workspace must be 256-byte aligned");
  if (((uintptr_t)params & 15) != 0 || ((uintptr_t)grads & 15) != 0)
    return fail(GPT_E_INVALID_ARG, "params and grads must be 16-byte aligned");
  size_t need = 0;
  s = gpt_workspace_bytes(cfg, max_B, max_T, &need);
  if (s != GPT_OK) return s;
  if (ws_bytes < need) return fail(GPT_E_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  hipStream_t stream = (hipStream_t)stream_;

  gpt_model* m = new (std::nothrow) gpt_model();
  if (!m) return fail(GPT_E_INVALID_ARG, "out of host memory");
  m->cfg = *cfg;
  m->params = params;
  m->grads = grads;
  m->ws = reinterpret_cast<char*>(workspace);
  m->ws_bytes = ws_bytes;
  m->maxB = max_B;
  m->maxT = max_T;
  m->L = plan(*cfg, max_B, max_T);
  int32_t n = 0;
  gpt_param_layout(cfg, nullptr, &n);
  std::vector<gpt_tensor_desc> d(n);
  gpt_param_layout(cfg, d.data(), &n);
  const int i_lm = 1 + 4 * cfg->n_layer;  // lm_head's index; optional tensors follow it
  m->off_wte = d[0].offset;
  for (int l = 0; l < cfg->n_layer; ++l) {
    m->off_qkv.push_back(d[1 + 4 * l].offset);
    m->off_o.push_back(d[2 + 4 * l].offset);
    m->off_w1.push_back(d[3 + 4 * l].offset);
    m->off_w2.push_back(d[4 + 4 * l].offset);
  }
  m->off_lm = d[i_lm].offset;
  m->off_ve.assign(cfg->n_layer, -1);
  for (int i = i_lm + 1; i < n; ++i) {
    const std::string nm(d[i].name);
    if (nm == "resid_lambdas") m->off_resid = d[i].offset;
    else if (nm == "x0_lambdas") m->off_x0lam = d[i].offset;
    else if (nm == "ve_gates") m->off_gates = d[i].offset;
    else m->off_ve[std::atoi(nm.c_str() + 1)] = d[i].offset;  // "h<l>.ve"
  }

  // RoPE tables: angle = t * theta^(-2i/D) in double precision, stored as fp32.
  std::vector<float> ct((size_t)max_T * 64), st((size_t)max_T * 64);
  for (int t = 0; t < max_T; ++t)
    for (int i = 0; i < 64; ++i) {
      const double ang = (double)t * std::pow((double)cfg->rope_theta, -2.0 * i / (double)kHeadDim);
      ct[(size_t)t * 64 + i] = (float)std::cos(ang);
      st[(size_t)t * 64 + i] = (float)std::sin(ang);
    }
  // transposed-weight descriptors (all matrices except the embedding, which
  // is never multiplied)
  // (FP8 models: only the LM head; their layer weights get e4m3 copies)
  std::vector<gk::TransposeDesc> td;
  int64_t tiles = 0;
  for (int i = cfg->dtype == GPT_FP8_E4M3 ? i_lm : 1; i <= i_lm; ++i) {
    gk::TransposeDesc t;
    t.offset = d[i].offset;
    t.rows = (int32_t)d[i].rows;
    t.cols = (int32_t)d[i].cols;
    t.tile0 = tiles;
    tiles += ((d[i].rows + 63) / 64) * ((d[i].cols + 63) / 64);
    td.push_back(t);
  }
  m->ntdesc = (int)td.size();
  m->wt_tiles = tiles;
  // FP8 layer-weight quantisation table: codes at the parameter's offset in
  // wq (row-major) and wqT (transposed)
  std::vector<gk::QuantDesc> qd;
  if (cfg->dtype == GPT_FP8_E4M3) {
    int64_t ab = 0, qb = 0;
    for (int i = 1; i < i_lm; ++i) {
      const int l = (i - 1) / 4, w = (i - 1) % 4;
      gk::QuantDesc q;
      q.src = reinterpret_cast<const char*>(params) + d[i].offset * 2;
      q.ld = d[i].cols;
      q.rows = (int32_t)d[i].rows;
      q.cols = (int32_t)d[i].cols;
      q.q = reinterpret_cast<uint8_t*>(m->ws + m->L.wq) + d[i].offset;
      q.qT = reinterpret_cast<uint8_t*>(m->ws + m->L.wqT) + d[i].offset;
      q.ldT = q.rows;
      q.amax = reinterpret_cast<float*>(m->ws + m->L.amax) + l * kAmaxSlots + A_W_QKV + w;
      q.amax_block0 = ab;
      q.quant_block0 = qb;
      if (gk::check_quant_desc(q) != hipSuccess) {
        delete m;
        return fail(GPT_E_UNSUPPORTED, "weight %s cannot be quantised", d[i].name);
      }
      ab += gk::amax_blocks(q);
      qb += gk::quant_blocks(q);
      qd.push_back(q);
    }
    m->nqdesc = (int)qd.size();
    m->wq_amax_blocks = ab;
    m->wq_blocks = qb;
  }
  hipError_t e = hipMemcpyAsync(m->ws + m->L.rope_cos, ct.data(), ct.size() * 4, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess && !qd.empty())
    e = hipMemcpyAsync(m->ws + m->L.qdesc, qd.data(), qd.size() * sizeof(gk::QuantDesc), hipMemcpyHostToDevice,
                       stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(m->ws + m->L.tdesc, td.data(), td.size() * sizeof(gk::TransposeDesc), hipMemcpyHostToDevice,
                       stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(m->ws + m->L.rope_sin, st.data(), st.size() * 4, hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipMemsetAsync(m->ws + m->L.flag, 0, 256, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);  // host tables go out of scope
  if (e != hipSuccess) {
    delete m;
    return fail(GPT_E_HIP, "gpt_init upload failed: %s", hipGetErrorString(e));
  }
  *out = m;
  return GPT_OK;
}

gpt_status gpt_forward_loss(gpt_model* m, const int32_t* idx, const int32_t* targets, int32_t B, int32_t T,
                            int32_t need_grad, float* loss, float* row_loss, void* stream_) {
  if (!m || !idx || !targets || !loss) return fail(GPT_E_INVALID_ARG, "NULL argument");
  if (B < 1 || T < 1 || B > m->maxB || T > m->maxT)
    return fail(GPT_E_INVALID_ARG, "B=%d T=%d outside [1, %d] x [1, %d]", B, T, m->maxB, m->maxT);
  hipStream_t stream = (hipStream_t)stream_;
  const gpt_config& c = m->cfg;
  const bool fp8 = c.dtype == GPT_FP8_E4M3;
  const int dt = fp8 ? GPT_BF16 : c.dtype;  // activation storage
  const int gdt = fp8 ? 2 : dt;              // operands of the QKV / O / MLP products
  const int N = B * T, C = c.model_dim, H = c.n_head, F = c.mlp_dim, V = c.vocab_size;
  const int QKV = (H + 2) * kHeadDim, HD = H * kHeadDim;
  const Layout& L = m->L;
  int* flag = wsp<int>(m, L.flag);
  m->pending = false;
  const int64_t Np = pad_tokens(N);
  float* amax = fp8 ? wsp<float>(m, L.amax) : nullptr;
  auto slot = [&](int l, int k) { return amax + l * kAmaxSlots + k; };
  uint8_t* xq = fp8 ? wsp<uint8_t>(m, L.xq) : nullptr;
  const uint8_t* wq = fp8 ? wsp<uint8_t>(m, L.wq) : nullptr;
  // A = activation (or its codes), B = weight at element offset woff (or its codes)
  auto operands = [&](gk::GemmArgs& a, const void* act, int64_t woff, int l, int act_slot, int w_slot) {
    if (fp8) {
      a.A = xq;
      a.B = wq + woff;
      a.amax_a = slot(l, act_slot);
      a.amax_b = slot(l, w_slot);
    } else {
      a.A = act;
      a.B = pbase(m, woff);
    }
  };
  if (fp8) {
    RUN(K_FP8_WEIGHTS, return gk::launch_fill_f32(amax, 0.f, (int64_t)c.n_layer * kAmaxSlots, stream););
    RUN(K_FP8_WEIGHTS, return gk::launch_fp8_amax_batched(reinterpret_cast<const gk::QuantDesc*>(m->ws + L.qdesc),
                                                          m->nqdesc, m->wq_amax_blocks, stream););
    RUN(K_FP8_WEIGHTS, return gk::launch_fp8_quantize_batched(
                           reinterpret_cast<const gk::QuantDesc*>(m->ws + L.qdesc), m->nqdesc, m->wq_blocks, stream););
  }

  RUN(K_EMBED, return gk::launch_embed_rmsnorm(dt, pbase(m, m->off_wte), idx, N, C, V, c.norm_eps, m->ws + L.x,
                                               wsp<float>(m, L.rstd0), flag, stream););
  if (c.x0_lambdas)  // keep x0 = rmsnorm(wte[idx]) for the per-layer mixes
    RUN(K_X0_MIX, return hipMemcpyAsync(m->ws + L.x0, m->ws + L.x, (size_t)N * C * esize(dt), hipMemcpyDeviceToDevice,
                                        stream););
  for (int l = 0; l < c.n_layer; ++l) {
    if (c.x0_lambdas)
      RUN(K_X0_MIX, return gk::launch_x0_mix(dt, m->ws + L.x, m->ws + L.x0, m->ws + L.xprev[l],
                                             pbase(m, m->off_resid + l), pbase(m, m->off_x0lam + l), (int64_t)N * C,
                                             stream););
    RUN(K_RMSNORM, return gk::launch_rmsnorm(dt, m->ws + L.x, N, C, c.norm_eps, m->ws + L.h1[l],
                                             wsp<float>(m, L.rstd1[l]), stream););
    if (fp8) TRY(quantize_operand(m, stream, m->ws + L.h1[l], N, C, xq, wsp<uint8_t>(m, L.h1qT[l]), Np, slot(l, A_H1)));
    RUN(K_GEMM_QKV, {
      gk::GemmArgs a;
      a.tile = m->gemm_tile;
      operands(a, m->ws + L.h1[l], m->off_qkv[l], l, A_H1, A_W_QKV);
      a.lda = C; a.ldb = C;
      a.M = N; a.N = QKV; a.K = C;
      a.C = m->ws + L.qkv[l]; a.ldc = QKV;
      return gk::launch_gemm(gdt, gk::Epi::Store, a, stream);
    });
    if (ve_layer(c, l))
      RUN(K_VE_ADD, return gk::launch_ve_add(dt, m->ws + L.qkv[l], QKV, (H + 1) * kHeadDim, idx, pbase(m, m->off_ve[l]),
                                             pbase(m, m->off_gates + l / 2), N, V, stream););
    RUN(K_ROPE_QKNORM, return gk::launch_rope_qknorm(dt, m->ws + L.qkv[l], B, T, H, c.norm_eps,
                                                     wsp<float>(m, L.rope_cos), wsp<float>(m, L.rope_sin),
                                                     wsp<float>(m, L.rstd_qk[l]), stream););
    const int win = layer_window(c, l);
    RUN(K_ATTN_FWD_PREP, return gk::launch_attn_fwd(dt, m->ws + L.qkv[l], B, T, H, win, m->ws + L.o[l],
                                                    wsp<float>(m, L.lse[l]), m->ws + L.vT, 0, stream););
    // FP8: the attention forward and the W1 / W2-dX epilogues (few long
    // blocks) fold the |max| of what they store, so those operands skip the
    // separate |max| pass; the row kernels' operands keep it
    RUN(K_ATTN_FWD, return gk::launch_attn_fwd(dt, m->ws + L.qkv[l], B, T, H, win, m->ws + L.o[l],
                                               wsp<float>(m, L.lse[l]), m->ws + L.vT, 1, stream,
                                               fp8 ? slot(l, A_O) : nullptr););
    if (fp8)
      TRY(quantize_operand(m, stream, m->ws + L.o[l], N, HD, xq, wsp<uint8_t>(m, L.oqT[l]), Np, slot(l, A_O), true));
    RUN(K_GEMM_O, {
      gk::GemmArgs a;
      a.tile = m->gemm_tile;
      operands(a, m->ws + L.o[l], m->off_o[l], l, A_O, A_W_O);
      a.lda = HD; a.ldb = HD;
      a.M = N; a.N = C; a.K = HD;
      a.C = m->ws + L.x; a.ldc = C;
      return gk::launch_gemm(gdt, gk::Epi::Residual, a, stream);
    });
    RUN(K_RMSNORM, return gk::launch_rmsnorm(dt, m->ws + L.x, N, C, c.norm_eps, m->ws + L.h2[l],
                                             wsp<float>(m, L.rstd2[l]), stream););
    if (fp8) TRY(quantize_operand(m, stream, m->ws + L.h2[l], N, C, xq, wsp<uint8_t>(m, L.h2qT[l]), Np, slot(l, A_H2)));
    RUN(K_GEMM_W1, {
      gk::GemmArgs a;
      a.tile = m->gemm_tile;
      operands(a, m->ws + L.h2[l], m->off_w1[l], l, A_H2, A_W_1);
      a.lda = C; a.ldb = C;
      a.M = N; a.N = F; a.K = C;
      a.C = m->ws + L.a[l]; a.ldc = F;
      if (fp8) a.amax_out = slot(l, A_A);
      return gk::launch_gemm(gdt, gk::Epi::Relu2, a, stream);
    });
    if (fp8)
      TRY(quantize_operand(m, stream, m->ws + L.a[l], N, F, xq, wsp<uint8_t>(m, L.aqT[l]), Np, slot(l, A_A), true));
    RUN(K_GEMM_W2, {
      gk::GemmArgs a;
      a.tile = m->gemm_tile;
      operands(a, m->ws + L.a[l], m->off_w2[l], l, A_A, A_W_2);
      a.lda = F; a.ldb = F;
      a.M = N; a.N = C; a.K = F;
      a.C = m->ws + L.x; a.ldc = C;
      return gk::launch_gemm(gdt, gk::Epi::Residual, a, stream);
    });
  }
  RUN(K_RMSNORM, return gk::launch_rmsnorm(dt, m->ws + L.x, N, C, c.norm_eps, m->ws + L.hf,
                                           wsp<float>(m, L.rstdf), stream););
  RUN(K_GEMM_LM, {
    gk::GemmArgs a;
      a.tile = m->gemm_tile;
    a.A = m->ws + L.hf; a.lda = C;
    a.B = pbase(m, m->off_lm); a.ldb = C;
    a.M = N; a.N = V; a.K = C;
    a.C = m->ws + L.logits; a.ldc = V;
    a.part = wsp<float>(m, L.part);
    a.targets = targets;
    a.ztgt = wsp<float>(m, L.ztgt);
    a.softcap = c.logit_softcap;
    return gk::launch_gemm(dt, gk::Epi::LMHead, a, stream);
  });
  RUN(K_CE_LOSS, return gk::launch_ce_loss(wsp<float>(m, L.part), V / gk::kLMHeadPartCols, wsp<float>(m, L.ztgt),
                                           targets, N, V, c.logit_softcap, wsp<float>(m, L.lse_ce),
                                           wsp<float>(m, L.loss_rows), row_loss, loss, flag, stream););
  m->B = B;
  m->T = T;
  m->idx = idx;
  m->targets = targets;
  m->pending = need_grad != 0;
  return GPT_OK;
}

gpt_status gpt_backward(gpt_model* m, float dloss, int32_t accumulate, void* stream_) {
  if (!m) return fail(GPT_E_INVALID_ARG, "NULL model");
  if (!m->pending) return fail(GPT_E_STATE, "gpt_backward needs a preceding gpt_forward_loss with need_grad = 1");
  hipStream_t stream = (hipStream_t)stream_;
  const gpt_config& c = m->cfg;
  const bool fp8 = c.dtype == GPT_FP8_E4M3;
  const int dt = fp8 ? GPT_BF16 : c.dtype;  // activation storage
  const int B = m->B, T = m->T, N = B * T, C = c.model_dim, H = c.n_head, F = c.mlp_dim, V = c.vocab_size;
  const int QKV = (H + 2) * kHeadDim, HD = H * kHeadDim;
  const Layout& L = m->L;
  float* G = m->grads;
  const int acc = accumulate ? 1 : 0;
  m->pending = false;

  auto dw = [&](int tag, const void* dy, int ldy, const void* x, int ldx, int M, int Nn, int64_t goff) -> gpt_status {
    RUN(tag, {
      gk::GemmArgs a;
      a.tile = m->gemm_tile;
      a.A = dy; a.lda = ldy; a.a_kcontig = false;
      a.B = x; a.ldb = ldx; a.b_kcontig = false;
      a.M = M; a.N = Nn; a.K = N;
      a.splits = dw_splits_ws(m, M, Nn, N);
      a.C = G + goff; a.ldc = Nn;
      a.accumulate = acc;
      a.split_buf = wsp<float>(m, L.split);
      return gk::launch_gemm(dt, gk::Epi::GradF32, a, stream);
    });
    return GPT_OK;
  };
  // dX = dY W for W [K, Nn] (row-major, w at element offset woff). bf16
  // models multiply by the transposed copy W^T [Nn, K] (both operands
  // k-contiguous, the direct-to-LDS kernel); fp32 reads W as is.
  const bool use_wt = dt == GPT_BF16;
  auto dx = [&](int tag, gk::Epi epi, const void* dy, int ldy, int64_t woff, int Nn, int K, void* out,
                const void* aux) -> gpt_status {
    RUN(tag, {
      gk::GemmArgs a;
      a.tile = m->gemm_tile;
      a.A = dy; a.lda = ldy;
      if (use_wt) {
        a.B = m->ws + L.wT + woff * (int64_t)esize(dt); a.ldb = K; a.b_kcontig = true;
      } else {
        a.B = pbase(m, woff); a.ldb = Nn; a.b_kcontig = false;
      }
      a.M = N; a.N = Nn; a.K = K;
      a.C = out; a.ldc = Nn;
      a.C2 = const_cast<void*>(aux); a.ldc2 = Nn;
      return gk::launch_gemm(dt, epi, a, stream);
    });
    return GPT_OK;
  };
  if (use_wt)
    RUN(K_WEIGHT_T, return gk::launch_transpose_batched(dt, m->params, m->ws + L.wT,
                                                        reinterpret_cast<const gk::TransposeDesc*>(m->ws + L.tdesc),
                                                        m->ntdesc, m->wt_tiles, stream););
  // FP8 products. Output-gradient codes: row-major dyq [N, K] and token-major
  // dyqT [K, Np]; forward operands' token-major codes from the stash; weight
  // codes (transposed) from the forward's quantisation.
  const int64_t Np = pad_tokens(N);
  float* amax = fp8 ? wsp<float>(m, L.amax) : nullptr;
  auto slot = [&](int l, int k) { return amax + l * kAmaxSlots + k; };
  uint8_t* dyq = fp8 ? wsp<uint8_t>(m, L.dyq) : nullptr;
  uint8_t* dyqT = fp8 ? wsp<uint8_t>(m, L.dyqT) : nullptr;
  const uint8_t* wqT = fp8 ? wsp<uint8_t>(m, L.wqT) : nullptr;
  auto dw8 = [&](int tag, size_t xT, int l, int dy_slot, int x_slot, int M, int Nn, int64_t goff) -> gpt_status {
    RUN(tag, {
      gk::GemmArgs a;
      a.tile = m->gemm_tile;
      a.A = dyqT; a.lda = Np;
      a.B = m->ws + xT; a.ldb = Np;
      a.M = M; a.N = Nn; a.K = (int)Np;
      a.splits = dw_splits_ws(m, M, Nn, (int)Np);
      a.C = G + goff; a.ldc = Nn;
      a.accumulate = acc;
      a.split_buf = wsp<float>(m, L.split);
      a.amax_a = slot(l, dy_slot);
      a.amax_b = slot(l, x_slot);
      return gk::launch_gemm(2, gk::Epi::GradF32, a, stream);
    });
    return GPT_OK;
  };
  auto dx8 = [&](int tag, gk::Epi epi, int l, int dy_slot, int w_slot, int64_t woff, int Nn, int K, void* out,
                 const void* aux, float* amax_out = nullptr) -> gpt_status {
    RUN(tag, {
      gk::GemmArgs a;
      a.tile = m->gemm_tile;
      a.A = dyq; a.lda = K;
      a.B = wqT + woff; a.ldb = K;
      a.M = N; a.N = Nn; a.K = K;
      a.C = out; a.ldc = Nn;
      a.C2 = const_cast<void*>(aux); a.ldc2 = Nn;
      a.amax_a = slot(l, dy_slot);
      a.amax_b = slot(l, w_slot);
      a.amax_out = amax_out;
      return gk::launch_gemm(2, epi, a, stream);
    });
    return GPT_OK;
  };

  // the ids sorted once: the embedding and value-embedding gradients sum over them
  RUN(K_EMBED_SORT, return gk::launch_embed_sort(m->idx, N, V, wsp<int32_t>(m, L.keys_a), wsp<int32_t>(m, L.vals_a),
                                                 wsp<int32_t>(m, L.keys_b), wsp<int32_t>(m, L.vals_b),
                                                 wsp<int32_t>(m, L.hist), stream););
  if (c.x0_lambdas) RUN(K_X0_MIX_BWD, return gk::launch_fill_f32(wsp<float>(m, L.dx0acc), 0.f, (int64_t)N * C, stream););
  // dz = r_n q (target entries fixed in place), never formed: dW_lm = q^T (r h)
  // with the scaled copy of h in dh's buffer (read before dX overwrites it),
  // dX_lm = q W_lm with rows scaled by r in the final norm's backward
  // the residual-stream gradient: fp32 in dres for fp32 models, by option, and
  // with residual scalars (their gradients are dot products of this gradient
  // with the stream, which its bf16 rounding moves measurably); else in the
  // activation dtype in dres_lp alone
  float* const dres32 = (dt == GPT_F32 || m->resid_grad_f32 || c.x0_lambdas) ? wsp<float>(m, L.dres) : nullptr;
  RUN(K_CE_BWD, return gk::launch_ce_grad_prep(dt, m->ws + L.logits, wsp<float>(m, L.lse_ce), wsp<float>(m, L.ztgt),
                                               m->targets, N, V, c.logit_softcap, dloss / (float)N, m->ws + L.hf, C,
                                               m->ws + L.dh, wsp<float>(m, L.ce_rscale), stream););
  // The embedding gradient is zeroed here, ahead of the LM-head products,
  // rather than just before its segment sums: the zeros (4VC bytes) land in
  // the caches, and their write-back to HBM then drains under these
  // MFMA-bound GEMMs instead of under the segment sums' reads.
  if (!acc)
    RUN(K_EMBED_BWD, return gk::launch_fill_f32(G + m->off_wte, 0.f, (int64_t)V * C, stream););
  TRY(dw(K_GEMM_LM_DW, m->ws + L.logits, V, m->ws + L.dh, C, V, C, m->off_lm));
  TRY(dx(K_GEMM_LM_DX, gk::Epi::Store, m->ws + L.logits, V, m->off_lm, C, V, m->ws + L.dh, nullptr));
  RUN(K_RMSNORM_BWD, return gk::launch_rmsnorm_bwd(dt, m->ws + L.dh, m->ws + L.hf, wsp<float>(m, L.rstdf), N, C, 0,
                                                   dres32, m->ws + L.dres_lp, stream,
                                                   wsp<float>(m, L.ce_rscale)););
  for (int l = c.n_layer - 1; l >= 0; --l) {
    // MLP
    if (fp8) {
      TRY(quantize_operand(m, stream, m->ws + L.dres_lp, N, C, dyq, dyqT, Np, slot(l, A_DY_MLP)));
      TRY(dw8(K_GEMM_W2_DW, L.aqT[l], l, A_DY_MLP, A_A, C, F, m->off_w2[l]));
      TRY(dx8(K_GEMM_W2_DX, gk::Epi::Relu2Bwd, l, A_DY_MLP, A_W_2, m->off_w2[l], F, C, m->ws + L.du, m->ws + L.a[l],
              slot(l, A_DU)));
      TRY(quantize_operand(m, stream, m->ws + L.du, N, F, dyq, dyqT, Np, slot(l, A_DU), true));
      TRY(dw8(K_GEMM_W1_DW, L.h2qT[l], l, A_DU, A_H2, F, C, m->off_w1[l]));
      TRY(dx8(K_GEMM_W1_DX, gk::Epi::Store, l, A_DU, A_W_1, m->off_w1[l], C, F, m->ws + L.dh, nullptr));
    } else {
      TRY(dw(K_GEMM_W2_DW, m->ws + L.dres_lp, C, m->ws + L.a[l], F, C, F, m->off_w2[l]));
      TRY(dx(K_GEMM_W2_DX, gk::Epi::Relu2Bwd, m->ws + L.dres_lp, C, m->off_w2[l], F, C, m->ws + L.du,
             m->ws + L.a[l]));
      TRY(dw(K_GEMM_W1_DW, m->ws + L.du, F, m->ws + L.h2[l], C, F, C, m->off_w1[l]));
      TRY(dx(K_GEMM_W1_DX, gk::Epi::Store, m->ws + L.du, F, m->off_w1[l], C, F, m->ws + L.dh, nullptr));
    }
    RUN(K_RMSNORM_BWD, return gk::launch_rmsnorm_bwd(dt, m->ws + L.dh, m->ws + L.h2[l], wsp<float>(m, L.rstd2[l]),
                                                     N, C, 1, dres32, m->ws + L.dres_lp, stream););
    // attention
    if (fp8) {
      TRY(quantize_operand(m, stream, m->ws + L.dres_lp, N, C, dyq, dyqT, Np, slot(l, A_DY_ATTN)));
      TRY(dw8(K_GEMM_O_DW, L.oqT[l], l, A_DY_ATTN, A_O, C, HD, m->off_o[l]));
      TRY(dx8(K_GEMM_O_DX, gk::Epi::Store, l, A_DY_ATTN, A_W_O, m->off_o[l], HD, C, m->ws + L.dout, nullptr));
    } else {
      TRY(dw(K_GEMM_O_DW, m->ws + L.dres_lp, C, m->ws + L.o[l], HD, C, HD, m->off_o[l]));
      TRY(dx(K_GEMM_O_DX, gk::Epi::Store, m->ws + L.dres_lp, C, m->off_o[l], HD, C, m->ws + L.dout, nullptr));
    }
    gk::AttnBwdArgs ab;
    ab.qkv = m->ws + L.qkv[l];
    ab.o = m->ws + L.o[l];
    ab.dout = m->ws + L.dout;
    ab.lse = wsp<float>(m, L.lse[l]);
    ab.B = B; ab.T = T; ab.H = H;
    ab.window = layer_window(m->cfg, l);
    ab.delta = wsp<float>(m, L.delta);
    ab.qT = m->ws + L.qT;
    ab.kT = m->ws + L.kT;
    ab.doT = m->ws + L.doT;
    ab.dqkv = m->ws + L.dqkv;
    ab.dkv_part = wsp<float>(m, L.dkv_part);
    ab.hsplit = m->dkv_hsplit;
    // fp32: transposed copies and delta (the bf16 dQ kernel forms delta itself)
    if (dt == GPT_F32) RUN(K_ATTN_BWD_PREP, return gk::launch_attn_bwd(dt, ab, 0, stream););
    RUN(K_ATTN_BWD_DQ, return gk::launch_attn_bwd(dt, ab, 1, stream););
    RUN(K_ATTN_BWD_DKV, return gk::launch_attn_bwd(dt, ab, 2, stream););
    RUN(K_ROPE_QKNORM_BWD, return gk::launch_rope_qknorm_bwd(dt, m->ws + L.dqkv, m->ws + L.qkv[l],
                                                             wsp<float>(m, L.rstd_qk[l]), B, T, H,
                                                             wsp<float>(m, L.rope_cos), wsp<float>(m, L.rope_sin),
                                                             stream););
    if (ve_layer(c, l)) {  // v = h1 W_v^T + gate * ve[idx]: dv reaches the gate and the table
      const int vcol = (H + 1) * kHeadDim;
      RUN(K_VE_BWD, return gk::launch_ve_gate_grad(dt, m->ws + L.dqkv, QKV, vcol, m->idx, pbase(m, m->off_ve[l]), N, V,
                                                   wsp<float>(m, L.rpart), G + m->off_gates + l / 2, acc, stream););
      RUN(K_VE_BWD, return gk::launch_ve_scatter(dt, wsp<int32_t>(m, L.keys_a), wsp<int32_t>(m, L.vals_a),
                                                 m->ws + L.dqkv, QKV, vcol, pbase(m, m->off_gates + l / 2), N, V, acc,
                                                 G + m->off_ve[l], wsp<float>(m, L.carry), stream););
    }
    if (fp8) {
      TRY(quantize_operand(m, stream, m->ws + L.dqkv, N, QKV, dyq, dyqT, Np, slot(l, A_DQKV)));
      TRY(dw8(K_GEMM_QKV_DW, L.h1qT[l], l, A_DQKV, A_H1, QKV, C, m->off_qkv[l]));
      TRY(dx8(K_GEMM_QKV_DX, gk::Epi::Store, l, A_DQKV, A_W_QKV, m->off_qkv[l], C, QKV, m->ws + L.dh, nullptr));
    } else {
      TRY(dw(K_GEMM_QKV_DW, m->ws + L.dqkv, QKV, m->ws + L.h1[l], C, QKV, C, m->off_qkv[l]));
      TRY(dx(K_GEMM_QKV_DX, gk::Epi::Store, m->ws + L.dqkv, QKV, m->off_qkv[l], C, QKV, m->ws + L.dh, nullptr));
    }
    RUN(K_RMSNORM_BWD, return gk::launch_rmsnorm_bwd(dt, m->ws + L.dh, m->ws + L.h1[l], wsp<float>(m, L.rstd1[l]),
                                                     N, C, 1, dres32, m->ws + L.dres_lp, stream););
    if (c.x0_lambdas)  // x_in = resid_lambdas[l] x_prev + x0_lambdas[l] x0
      RUN(K_X0_MIX_BWD, return gk::launch_x0_mix_bwd(dt, dres32, m->ws + L.dres_lp, m->ws + L.xprev[l],
                                                     m->ws + L.x0, wsp<float>(m, L.dx0acc),
                                                     pbase(m, m->off_resid + l), pbase(m, m->off_x0lam + l), l == 0,
                                                     (int64_t)N * C, wsp<float>(m, L.rpart), G + m->off_resid + l,
                                                     G + m->off_x0lam + l, acc, stream););
  }
  RUN(K_EMBED_BWD, {
    gk::EmbedBwdArgs a;
    a.dtype = dt;
    a.wte = pbase(m, m->off_wte);
    a.idx = m->idx;
    a.dres = dres32;
    a.dres_lp = m->ws + L.dres_lp;
    a.rstd0 = wsp<float>(m, L.rstd0);
    a.N = N; a.C = C; a.V = V;
    a.accumulate = acc;
    a.dwte_zeroed = 1;  // zeroed before the LM-head products (without accumulate)
    a.dwte = G + m->off_wte;
    a.keys_a = wsp<int32_t>(m, L.keys_a);
    a.vals_a = wsp<int32_t>(m, L.vals_a);
    a.keys_b = wsp<int32_t>(m, L.keys_b);
    a.vals_b = wsp<int32_t>(m, L.vals_b);
    a.hist = wsp<int32_t>(m, L.hist);
    a.carry = wsp<float>(m, L.carry);
    return gk::launch_embed_bwd(a, stream);
  });
  return GPT_OK;
}

gpt_status gpt_sync_status(gpt_model* m, void* stream_) {
  if (!m) return fail(GPT_E_INVALID_ARG, "NULL model");
  hipStream_t stream = (hipStream_t)stream_;
  int flag = 0;
  HIP_TRY(hipStreamSynchronize(stream));
  HIP_TRY(hipMemcpy(&flag, m->ws + m->L.flag, sizeof(int), hipMemcpyDeviceToHost));
  if (flag) return fail(GPT_E_DEVICE, "device flag 0x%x: token id outside [0, vocab_size)", flag);
  return GPT_OK;
}

gpt_status gpt_destroy(gpt_model* m) {
  if (!m) return GPT_OK;
  for (hipEvent_t e : m->prof.ev) (void)hipEventDestroy(e);
  delete m;
  return GPT_OK;
}

gpt_status gpt_profile_begin(gpt_model* m, int32_t tag) {
  if (!m) return fail(GPT_E_INVALID_ARG, "NULL model");
  if (tag >= K_NUM_TAGS) return fail(GPT_E_INVALID_ARG, "unknown tag %d", tag);
  m->prof.armed = true;
  m->prof.tag = tag;
  m->prof.used = 0;
  return GPT_OK;
}

gpt_status gpt_profile_end(gpt_model* m, double* total_ms, int64_t* launches) {
  if (!m || !total_ms || !launches) return fail(GPT_E_INVALID_ARG, "NULL argument");
  Profiler& P = m->prof;
  double tot = 0.0;
  for (size_t i = 0; i < P.used; ++i) {
    HIP_TRY(hipEventSynchronize(P.ev[2 * i + 1]));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, P.ev[2 * i], P.ev[2 * i + 1]));
    tot += ms;
  }
  *total_ms = tot;
  *launches = (int64_t)P.used;
  P.armed = false;
  P.used = 0;
  return GPT_OK;
}

gpt_status gpt_set_option(gpt_model* m, int32_t option, int32_t value) {
  if (!m) return fail(GPT_E_INVALID_ARG, "NULL model");
  switch (option) {
    case GPT_OPT_GEMM_TILE:
      if (value < 0 || value > 3) return fail(GPT_E_INVALID_ARG, "GEMM tile option %d not in 0..3", value);
      m->gemm_tile = value;
      return GPT_OK;
    case GPT_OPT_DKV_HSPLIT:
      if (value < 0 || value > 2) return fail(GPT_E_INVALID_ARG, "dK/dV head-split option %d not in 0..2", value);
      m->dkv_hsplit = value;
      return GPT_OK;
    case GPT_OPT_RESID_GRAD:
      if (value < 0 || value > 1) return fail(GPT_E_INVALID_ARG, "residual-gradient option %d not in 0..1", value);
      m->resid_grad_f32 = value;
      return GPT_OK;
    default:
      return fail(GPT_E_INVALID_ARG, "unknown option %d", option);
  }
}

const char* gpt_kernel_tag_name(int32_t tag) {
  if (tag < 0 || tag >= K_NUM_TAGS) return nullptr;
  return kTagNames[tag];
}

gpt_status gpt_debug_buffer(gpt_model* m, const char* name, int32_t layer, void** ptr, size_t* bytes) {
  if (!m || !name || !ptr || !bytes) return fail(GPT_E_INVALID_ARG, "NULL argument");
  const gpt_config& c = m->cfg;
  const Layout& L = m->L;
  const size_t N = (size_t)m->B * m->T, es = esize(c.dtype), C = c.model_dim, H = c.n_head;
  const bool lv = layer >= 0 && layer < c.n_layer;
  auto set = [&](size_t off, size_t b) { *ptr = m->ws + off; *bytes = b; return GPT_OK; };
  const std::string s(name);
  if (s == "x") return set(L.x, N * C * es);
  if (s == "hf") return set(L.hf, N * C * es);
  if (s == "rstd0") return set(L.rstd0, N * 4);
  if (s == "logits") return set(L.logits, N * (size_t)c.vocab_size * es);
  if (s == "du") return set(L.du, N * (size_t)c.mlp_dim * es);
  if (s == "dqkv") return set(L.dqkv, N * (H + 2) * kHeadDim * es);
  if (!lv) return fail(GPT_E_INVALID_ARG, "unknown buffer '%s' or layer %d out of range", name, layer);
  if (s == "h1") return set(L.h1[layer], N * C * es);
  if (s == "qkv") return set(L.qkv[layer], N * (H + 2) * kHeadDim * es);
  if (s == "o") return set(L.o[layer], N * H * kHeadDim * es);
  if (s == "lse") return set(L.lse[layer], N * H * 4);
  if (s == "h2") return set(L.h2[layer], N * C * es);
  if (s == "a") return set(L.a[layer], N * (size_t)c.mlp_dim * es);
  if (s == "amax" && c.dtype == GPT_FP8_E4M3) return set(L.amax + (size_t)layer * kAmaxSlots * 4, kAmaxSlots * 4);
  return fail(GPT_E_INVALID_ARG, "unknown buffer '%s'", name);
}

}  // extern "C"

namespace {
// Optimiser group of a parameter tensor: 0 Muon (blocks' matrix weights),
// 1 embeddings (wte, value-embedding tables), 2 unembedding, 3 scalars.
int optim_group(const std::string& nm) {
  auto ends = [&](const char* suf) {
    const size_t n = strlen(suf);
    return nm.size() >= n && nm.compare(nm.size() - n, n, suf) == 0;
  };
  if (nm[0] == 'h' && (ends(".w_qkv") || ends(".w_o") || ends(".w_1") || ends(".w_2"))) return 0;
  if (nm == "lm_head") return 2;
  if (nm == "wte" || ends(".ve")) return 1;
  return 3;
}
}  // namespace

extern "C" {

gpt_status gpt_optimizer_state_elems(const gpt_config* c, int64_t* elems) {
  if (!elems) return fail(GPT_E_INVALID_ARG, "elems is NULL");
  gpt_status s = gpt_config_validate(c);
  if (s != GPT_OK) return s;
  int32_t n = 0;
  gpt_param_layout(c, nullptr, &n);
  std::vector<gpt_tensor_desc> d(n);
  gpt_param_layout(c, d.data(), &n);
  int64_t tot = 0;
  for (auto& t : d) tot += (optim_group(t.name) == 0 ? 1 : 2) * t.rows * t.cols;
  *elems = tot;
  return GPT_OK;
}

gpt_status gpt_optimizer_step(gpt_model* m, const gpt_optim_config* oc, float* master, float* state, int32_t t,
                              void* stream_) {
  if (!m || !oc || !master || !state) return fail(GPT_E_INVALID_ARG, "NULL argument");
  if (t < 1) return fail(GPT_E_INVALID_ARG, "the step number t must be >= 1");
  if (oc->ns_steps < 0 || oc->ns_steps > 100) return fail(GPT_E_INVALID_ARG, "ns_steps must be in [0, 100]");
  if (!(oc->beta1 >= 0.f && oc->beta1 < 1.f && oc->beta2 >= 0.f && oc->beta2 < 1.f && oc->eps > 0.f))
    return fail(GPT_E_INVALID_ARG, "need 0 <= beta1, beta2 < 1 and eps > 0");
  if (((uintptr_t)master & 15) || ((uintptr_t)state & 15))
    return fail(GPT_E_INVALID_ARG, "master and state must be 16-byte aligned");
  hipStream_t stream = (hipStream_t)stream_;
  const gpt_config& c = m->cfg;
  const int dt = c.dtype == GPT_F32 ? GPT_F32 : GPT_BF16;  // the parameters' storage dtype
  const Layout& L = m->L;
  int32_t n = 0;
  gpt_param_layout(&c, nullptr, &n);
  std::vector<gpt_tensor_desc> d(n);
  gpt_param_layout(&c, d.data(), &n);
  char* params = reinterpret_cast<char*>(const_cast<void*>(m->params));
  const double bc1 = 1.0 - std::pow((double)oc->beta1, (double)t);
  const double bc2 = 1.0 - std::pow((double)oc->beta2, (double)t);
  // state offsets in parameter order (Muon: momentum; AdamW: m then v)
  std::vector<int64_t> soff(d.size());
  int64_t so = 0;
  for (size_t i = 0; i < d.size(); ++i) {
    soff[i] = so;
    so += (optim_group(d[i].name) == 0 ? 1 : 2) * d[i].rows * d[i].cols;
  }
  std::vector<char> done(d.size(), 0);
  for (size_t i = 0; i < d.size(); ++i) {
    const auto& td = d[i];
    const int grp = optim_group(td.name);
    const int64_t ne = td.rows * td.cols;
    if (grp == 0) {
      if (done[i]) continue;
      // this matrix and the later ones of its shape, in batches
      std::vector<size_t> same;
      for (size_t k = i; k < d.size(); ++k)
        if (!done[k] && optim_group(d[k].name) == 0 && d[k].rows == td.rows && d[k].cols == td.cols) same.push_back(k);
      for (size_t b0 = 0; b0 < same.size(); b0 += (size_t)L.ns_batch) {
        const int cnt = (int)std::min(same.size() - b0, (size_t)L.ns_batch);
        RUN(K_OPT_MUON, {
          gk::MuonArgs a;
          a.count = cnt;
          for (int j = 0; j < cnt; ++j) {
            const auto& tj = d[same[b0 + j]];
            a.w[j] = master + tj.offset;
            a.g[j] = m->grads + tj.offset;
            a.u[j] = state + soff[same[b0 + j]];
            a.out[j] = params + tj.offset * (int64_t)esize(dt);
          }
          a.rows = (int)td.rows;
          a.cols = (int)td.cols;
          a.lr = oc->lr_muon;
          a.mu = oc->momentum;
          a.wd = oc->wd_muon;
          a.steps = oc->ns_steps;
          a.a = oc->ns_a; a.b = oc->ns_b; a.c = oc->ns_c;
          a.X = m->ws + L.ns_x; a.XT = m->ws + L.ns_xt;
          a.A = m->ws + L.ns_a; a.AA = m->ws + L.ns_aa; a.Bm = m->ws + L.ns_b;
          a.partials = wsp<float>(m, L.ns_part);
          a.inv = wsp<float>(m, L.ns_inv);
          return gk::launch_muon(dt, a, stream);
        });
      }
      for (size_t k : same) done[k] = 1;
    } else {
      const float lr = grp == 1 ? oc->lr_embed : grp == 2 ? oc->lr_unembed : oc->lr_scalar;
      RUN(K_OPT_ADAMW, {
        gk::AdamwArgs a;
        a.w = master + td.offset;
        a.g = m->grads + td.offset;
        a.m = state + soff[i];
        a.v = state + soff[i] + ne;
        a.out = params + td.offset * (int64_t)esize(dt);
        a.n = ne;
        a.lr = lr;
        a.beta1 = oc->beta1; a.beta2 = oc->beta2; a.eps = oc->eps; a.wd = oc->wd_adamw;
        a.step_size = (float)(lr / bc1);
        a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
        return gk::launch_adamw(dt, a, stream);
      });
    }
  }
  return GPT_OK;
}

gpt_status gpt_fp8_matmul(const uint8_t* a, int64_t lda, const float* amax_a, const uint8_t* b, int64_t ldb,
                          const float* amax_b, int32_t M, int32_t N, int32_t K, int32_t out_dtype, void* out,
                          int64_t ldo, int32_t tile, int32_t splits, float* partials, void* stream_) {
  if (!a || !b || !amax_a || !amax_b || !out) return fail(GPT_E_INVALID_ARG, "NULL argument");
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0 || N % 4 != 0)
    return fail(GPT_E_INVALID_ARG, "need M, N, K >= 0, K a multiple of 128 and N a multiple of 4");
  if (lda < K || ldb < K || ldo < N || lda % 16 != 0 || ldb % 16 != 0 || ldo % 4 != 0)
    return fail(GPT_E_INVALID_ARG, "need lda, ldb >= K (multiples of 16) and ldo >= N (a multiple of 4)");
  if (((uintptr_t)a & 15) || ((uintptr_t)b & 15) || ((uintptr_t)out & 15))
    return fail(GPT_E_INVALID_ARG, "a, b and out must be 16-byte aligned");
  if (tile < 0 || tile > 3) return fail(GPT_E_INVALID_ARG, "tile must be 0..3");
  if (out_dtype != GPT_F32 && out_dtype != GPT_BF16) return fail(GPT_E_INVALID_ARG, "out_dtype must be GPT_F32 or GPT_BF16");
  if (splits < 1 || splits > 64 || (splits > 1 && (out_dtype != GPT_F32 || !partials)))
    return fail(GPT_E_INVALID_ARG, "splits must be 1..64; more than one needs fp32 output and a partial buffer");
  hipStream_t stream = (hipStream_t)stream_;
  gk::GemmArgs g;
  g.tile = tile;
  g.A = a; g.lda = lda;
  g.B = b; g.ldb = ldb;
  g.M = M; g.N = N; g.K = K;
  g.C = out; g.ldc = ldo;
  g.amax_a = amax_a;
  g.amax_b = amax_b;
  g.splits = splits;
  g.split_buf = partials;
  g.accumulate = 0;
  if (M == 0 || N == 0) return GPT_OK;
  if (K == 0) return fail(GPT_E_INVALID_ARG, "K must be positive");
  HIP_TRY(gk::launch_gemm(2, out_dtype == GPT_F32 ? gk::Epi::GradF32 : gk::Epi::Store, g, stream));
  return GPT_OK;
}

gpt_status gpt_fp8_matmul_noalloc(const uint8_t* a, int64_t lda, const float* amax_a, const uint8_t* b,
                                  int64_t ldb, const float* amax_b, int32_t M, int32_t N, int32_t K,
                                  int32_t out_dtype, void* out, int64_t ldo, int32_t tile, int32_t splits,
                                  void* stream) {
  float* part = nullptr;
  if (splits > 1) {
    if (M < 0 || N < 0 || splits > 64)
      return fail(GPT_E_INVALID_ARG, "need M, N >= 0 and splits 1..64");
    const uint64_t need = (uint64_t)splits * (uint64_t)M * (uint64_t)N;
    if (need > gk::kNoAllocScratchFloats)
      return fail(GPT_E_INVALID_ARG, "splits * M * N = %llu exceeds the fixed partial buffer of %llu floats",
                  (unsigned long long)need, (unsigned long long)gk::kNoAllocScratchFloats);
    HIP_TRY(gk::noalloc_scratch(&part));
  }
  return gpt_fp8_matmul(a, lda, amax_a, b, ldb, amax_b, M, N, K, out_dtype, out, ldo, tile, splits, part, stream);
}

gpt_status gpt_fp8_quantize(const void* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* qT, int64_t ldT,
                            float* amax, void* stream_) {
  if (!x || !amax || (!q && !qT)) return fail(GPT_E_INVALID_ARG, "x, amax and one of q, qT must be non-NULL");
  if (rows < 0 || cols < 0 || rows > INT32_MAX || cols > INT32_MAX || cols % 16 != 0)
    return fail(GPT_E_INVALID_ARG, "need 0 <= rows, cols < 2^31 and cols a multiple of 16");
  if (qT && (ldT < rows || ldT % 16 != 0 || ldT > INT32_MAX))
    return fail(GPT_E_INVALID_ARG, "ldT must be >= rows and a multiple of 16");
  if (((uintptr_t)x & 15) || ((uintptr_t)q & 15) || ((uintptr_t)qT & 15) || ((uintptr_t)amax & 3))
    return fail(GPT_E_INVALID_ARG, "x, q and qT must be 16-byte aligned, amax 4-byte aligned");
  hipStream_t stream = (hipStream_t)stream_;
  gk::QuantDesc d;
  d.src = x;
  d.ld = cols;
  d.rows = (int32_t)rows;
  d.cols = (int32_t)cols;
  d.q = q;
  d.qT = qT;
  d.ldT = (int32_t)(qT ? ldT : 0);
  d.amax = amax;
  HIP_TRY(gk::launch_fill_f32(amax, 0.f, 1, stream));
  HIP_TRY(gk::launch_fp8_amax(d, stream));
  HIP_TRY(gk::launch_fp8_quantize(d, stream));
  return GPT_OK;
}

}  // extern "C"
