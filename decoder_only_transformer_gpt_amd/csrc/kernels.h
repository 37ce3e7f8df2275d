// Host-side launch interface of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gk {

enum class Epi : int {
  Store = 0,     // C = acc (activation dtype)
  Residual = 1,  // C += acc in place (the residual stream)
  Relu2 = 2,     // C = max(acc, 0)^2 (a); the backward recovers max(u, 0) = sqrt(a)
  LMHead = 3,    // C = c*tanh(acc/c) (logits), exp-sum partials, logit at target
  Relu2Bwd = 4,  // C = acc * 2*sqrt(a) with a = max(u, 0)^2 read from C2
  GradF32 = 5,   // fp32 gradient: C = acc or C += acc; split-K writes partials
};

struct GemmArgs {
  // C[m, n] = sum_k A(m, k) * B(n, k)
  const void* A = nullptr;
  int64_t lda = 0;
  bool a_kcontig = true;  // A(m,k) at A[m*lda + k] if true, else A[k*lda + m]
  const void* B = nullptr;
  int64_t ldb = 0;
  bool b_kcontig = true;  // B(n,k) at B[n*ldb + k] if true, else B[k*ldb + n]
  int M = 0, N = 0, K = 0;
  int splits = 1;          // split-K slices (GradF32 only)
  int tile = 0;            // 0: by shape; 1..3: force a tile variant (largest first)
  void* C = nullptr;
  int64_t ldc = 0;
  void* C2 = nullptr;
  int64_t ldc2 = 0;
  // LMHead
  float* part = nullptr;   // [M, N / 128] exp-sum partials
  const int32_t* targets = nullptr;
  float* ztgt = nullptr;   // [M] logit at the target, fp32
  float softcap = 15.f;
  // GradF32
  int accumulate = 0;
  float* split_buf = nullptr;  // [splits, M, N] partials when splits > 1
  int zslice = -1;             // split-K slice of the block; -1: blockIdx.z
  // fp8 operands (dtype 2): |max| slots of A and B; acc is scaled by 1/(s_a s_b)
  const float* amax_a = nullptr;
  const float* amax_b = nullptr;
  // Relu2 / Relu2Bwd on fp8 operands: optional slot for the |max| of the
  // stored output, one atomic max per block (the slot must start at 0)
  float* amax_out = nullptr;
  // batched products (Store / Residual epilogues, no split-K): product j reads
  // A + j*stride_a, B + j*stride_b and writes C + j*stride_c (bytes)
  int batch = 1;
  int64_t stride_a = 0, stride_b = 0, stride_c = 0;
};

// dtype: 0 = fp32, 1 = bf16 (gpt.h GPT_F32 / GPT_BF16), 2 = fp8 e4m3
// operands (k-contiguous, K a multiple of 128) with bf16 / fp32 outputs
hipError_t launch_gemm(int dtype, Epi epi, const GemmArgs& a, hipStream_t s);
// Fixed device array for split-K partials of gpt_fp8_matmul_noalloc (floats,
// 16 MiB per GPU), and the address of the current device's copy (looked up
// once per device with hipGetSymbolAddress).
constexpr size_t kNoAllocScratchFloats = (size_t)4 << 20;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(float** out);
// Partial-column width of the LMHead epilogue (exp-sum partials per row).
constexpr int kLMHeadPartCols = 64;

// Row-wise kernels ---------------------------------------------------------
hipError_t launch_embed_rmsnorm(int dtype, const void* wte, const int32_t* idx, int N, int C, int V,
                                float eps, void* x, float* rstd, int* flag, hipStream_t s);
hipError_t launch_rmsnorm(int dtype, const void* x, int N, int C, float eps, void* y, float* rstd,
                          hipStream_t s);
// dres = (accumulate ? dres : 0) + r * (dy - y * mean(dy*y)); dres_lp = dres in the activation dtype;
// with dres null the gradient is kept in dres_lp alone (read there when accumulating);
// dy_row_scale (optional, fp32 [N]): dy of row n is multiplied by dy_row_scale[n] first
hipError_t launch_rmsnorm_bwd(int dtype, const void* dy, const void* y, const float* rstd, int N, int C,
                              int accumulate, float* dres, void* dres_lp, hipStream_t s,
                              const float* dy_row_scale = nullptr);
hipError_t launch_rope_qknorm(int dtype, void* qkv, int B, int T, int H, float eps, const float* cos_t,
                              const float* sin_t, float* rstd_qk, hipStream_t s);
hipError_t launch_rope_qknorm_bwd(int dtype, void* dqkv, const void* qkv, const float* rstd_qk, int B,
                                  int T, int H, const float* cos_t, const float* sin_t, hipStream_t s);

// Attention (causal, multi-query, head_dim 128) ----------------------------
// Transposed copies use [B, heads, 128, Tp] with Tp = attn_padded_len(T).
int attn_padded_len(int T);
// vT: scratch of B * 128 * Tp elements. Stage 0 writes vT (the V transpose),
// stage 1 runs the attention kernel; they are separate so each can be timed.
// window: sliding-window length (keys u with 0 <= t - u < window); 0 or >= T
// means the full causal prefix.
hipError_t launch_attn_fwd(int dtype, const void* qkv, int B, int T, int H, int window, void* o, float* lse, void* vT,
                           int stage, hipStream_t s,
                           float* amax = nullptr);  // optional: |max| of o, one atomic max per block
struct AttnBwdArgs {
  const void* qkv;   // [N, (H+2)*128] normalised q, k and v
  const void* o;     // [N, H*128]
  const void* dout;  // [N, H*128]
  const float* lse;  // [B, H, T], base 2: lse * log2(e)
  int B, T, H;
  int window = 0;    // sliding-window length; 0 (or >= T) = full causal prefix
  float* delta;      // [B, H, T] scratch
  void* qT;          // [B, H, 128, Tp] scratch
  void* kT;          // [B, 1, 128, Tp] scratch
  void* doT;         // [B, H, 128, Tp] scratch
  void* dqkv;        // [N, (H+2)*128] output
  float* dkv_part;   // [2, N, 256] fp32 scratch (bf16 dK/dV split over two head halves), or null
  int hsplit = 0;    // bf16 dK/dV: 0 picks by grid size, 1 or 2 forces that many head groups per key block
};
// Stage 0: transposed copies + delta; stage 1: dQ; stage 2: dK and dV.
hipError_t launch_attn_bwd(int dtype, const AttnBwdArgs& a, int stage, hipStream_t s);

// Cross-entropy -------------------------------------------------------------
hipError_t launch_ce_loss(const float* part, int nparts, const float* ztgt, const int32_t* targets, int N,
                          int V, float softcap, float* lse, float* row_loss, float* row_loss_out,
                          float* loss, int* flag, hipStream_t s);
hipError_t launch_ce_grad_prep(int dtype, void* q, const float* lse, const float* ztgt, const int32_t* targets, int N,
                               int V, float softcap, float scale, const void* h, int C, void* hs, float* rscale,
                               hipStream_t s);

// Embedding backward ---------------------------------------------------------
struct EmbedBwdArgs {
  int dtype;
  const void* wte;       // [V, C]
  const int32_t* idx;    // [N]
  const float* dres;     // [N, C] gradient w.r.t. x0 (the normalised embedding), fp32; or null:
  const void* dres_lp = nullptr;  // then this one, [N, C] in the activation dtype
  const float* rstd0;    // [N]
  int N, C, V;
  int accumulate;
  int dwte_zeroed = 0;   // without accumulate: dwte was zeroed earlier by the caller (no fill here)
  float* dwte;           // [V, C] fp32
  // scratch (inside the workspace); keys_a / vals_a hold the ids sorted by launch_embed_sort
  int32_t* keys_a; int32_t* vals_a; int32_t* keys_b; int32_t* vals_b;  // [N] each
  int32_t* hist;         // embed_bwd_hist_elems(N)
  float* carry;          // embed_bwd_carry_elems(N, C)
};
// Stable sort of the token ids (key = id, value = position) into keys_a /
// vals_a (keys_b / vals_b scratch); launch_embed_bwd and launch_ve_scatter
// read the sorted arrays.
hipError_t launch_embed_sort(const int32_t* idx, int N, int V, int32_t* keys_a, int32_t* vals_a, int32_t* keys_b,
                             int32_t* vals_b, int32_t* hist, hipStream_t s);
hipError_t launch_embed_bwd(const EmbedBwdArgs& a, hipStream_t s);
// dve [V, 128] fp32 (+)= gate * sum over positions with that id of dv, dv at
// column col0 of dqkv (row pitch ld), in sorted-id order (deterministic).
hipError_t launch_ve_scatter(int dtype, const int32_t* keys, const int32_t* vals, const void* dqkv, int64_t ld,
                             int col0, const void* gate, int N, int V, int accumulate, float* dve, float* carry,
                             hipStream_t s);

// Residual scalars and value embeddings ----------------------------------------
size_t resid_partials_elems();
// xprev = x; x = lam_r * x + lam_0 * x0 over n elements (lam_* device scalars in the param dtype)
hipError_t launch_x0_mix(int dtype, void* x, const void* x0, void* xprev, const void* lam_r, const void* lam_0,
                         int64_t n, hipStream_t s);
// backward of the mix: scalar gradients (+)= <dres, xprev>, <dres, x0>; dres
// becomes the gradient of xprev (first: of x0, dx0acc included); dres_lp = dres
// (dres null: the gradient is read from and written to dres_lp alone)
hipError_t launch_x0_mix_bwd(int dtype, float* dres, void* dres_lp, const void* xprev, const void* x0, float* dx0acc,
                             const void* lam_r, const void* lam_0, int first, int64_t n, float* partials,
                             float* g_lam_r, float* g_lam_0, int accumulate, hipStream_t s);
// v[n] += gate * ve[idx[n]] (v = 128 values at column col0 of qkv, row pitch ld)
hipError_t launch_ve_add(int dtype, void* qkv, int64_t ld, int col0, const int32_t* idx, const void* ve,
                         const void* gate, int N, int V, hipStream_t s);
// g_gate (+)= sum_n <dv[n], ve[idx[n]]>
hipError_t launch_ve_gate_grad(int dtype, const void* dqkv, int64_t ld, int col0, const int32_t* idx, const void* ve,
                               int N, int V, float* partials, float* g_gate, int accumulate, hipStream_t s);
size_t embed_bwd_hist_elems(int N);
size_t embed_bwd_carry_elems(int N, int C);

hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t s);

// Batched transpose of row-major [rows, cols] tensors stored at `offset`
// (elements) in src into [cols, rows] at the same offset in dst.
struct TransposeDesc {
  int64_t offset;
  int32_t rows, cols;
  int64_t tile0;  // index of the tensor's first 64x64 tile
};
hipError_t launch_transpose_batched(int dtype, const void* src, void* dst, const TransposeDesc* desc, int ndesc,
                                    int64_t total_tiles, hipStream_t s);

// FP8 (e4m3) operands ---------------------------------------------------------
// One bf16 tensor [rows, cols] (row pitch ld elements) and where its codes go:
// q [rows, cols] row-major (pitch cols) and/or qT [cols, ldT] (its transpose,
// columns rows..ldT-1 written as code 0). amax: the tensor's fp32 |max| slot,
// to be zeroed before the amax pass (launch_fill_f32) and read by the
// quantise pass and the GEMM epilogue; s = 448 / amax (1 if amax == 0).
struct QuantDesc {
  const void* src = nullptr;    // bf16
  int64_t ld = 0;
  int32_t rows = 0, cols = 0;   // cols a multiple of 16
  uint8_t* q = nullptr;
  uint8_t* qT = nullptr;
  int32_t ldT = 0;              // >= rows, a multiple of 16
  float* amax = nullptr;
  int64_t amax_block0 = 0;      // first block of this tensor in a batched amax launch
  int64_t quant_block0 = 0;     // first block of this tensor in a batched quantise launch
};
hipError_t check_quant_desc(const QuantDesc& d);
int64_t amax_blocks(const QuantDesc& d);
int64_t quant_blocks(const QuantDesc& d);
hipError_t launch_fp8_amax(const QuantDesc& d, hipStream_t s);      // amax = max(amax, max |x|)
hipError_t launch_fp8_quantize(const QuantDesc& d, hipStream_t s);
// Batched over a device table of n descriptors (block offsets filled in).
hipError_t launch_fp8_amax_batched(const QuantDesc* table, int n, int64_t total_blocks, hipStream_t s);
hipError_t launch_fp8_quantize_batched(const QuantDesc* table, int n, int64_t total_blocks, hipStream_t s);

// Optimiser -------------------------------------------------------------------
struct AdamwArgs {
  float* w;            // fp32 master [n]
  const float* g;      // fp32 gradient [n]
  float* m;            // first moment [n]
  float* v;            // second moment [n]
  void* out;           // the model's copy (model dtype) [n]
  int64_t n;
  float lr, beta1, beta2, eps, wd;
  float step_size;     // lr / (1 - beta1^t)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
};
hipError_t launch_adamw(int dtype, const AdamwArgs& a, hipStream_t s);
// Muon on up to kMuonBatch matrices of one shape at once: every step of the
// iteration is one launch for the whole batch.
constexpr int kMuonBatch = 32;
struct MuonArgs {
  int count;                      // matrices in the batch, 1..kMuonBatch
  float* w[kMuonBatch];           // fp32 masters [rows, cols]
  const float* g[kMuonBatch];     // fp32 gradients
  float* u[kMuonBatch];           // momenta
  void* out[kMuonBatch];          // the model's copies (model dtype)
  int rows, cols;
  float lr, mu, wd;
  int steps;           // Newton-Schulz steps
  float a, b, c;       // X <- a X + (b A + c A^2) X
  // scratch (model dtype unless noted), count copies each, contiguous: X and
  // X^T [min*max], A, AA, Bm [min^2]; partials (fp32, count *
  // muon_partials_elems()), inv (fp32, count)
  void *X, *XT, *A, *AA, *Bm;
  float* partials;
  float* inv;
};
size_t muon_partials_elems();
hipError_t launch_muon(int dtype, const MuonArgs& a, hipStream_t s);

}  // namespace gk
