// The optimiser step after the backward: Muon for the blocks' matrix weights,
// AdamW for the embeddings, the unembedding and the scalars, on fp32 master
// weights whose cast to the compute dtype becomes the model's parameters
// (atlas.blal.pro "nanochat — full-stack ChatGPT in ~8k lines", section "How
// it works", item "2. Pretrain"; aethryn.com "Nanochat: full-stack LLM
// training in 8,000 lines for $72", section "A Llama-class transformer with
// ten modern departures"; energyai.berlin "nanochat vs GPT-OSS", section
// "Muon optimizer").
//
// AdamW is one elementwise pass (HBM-bound). Muon per matrix: the momentum
// update with a per-block partial sum of squares (one block adds them in
// order: the Frobenius norm), the normalised start of the Newton-Schulz
// iteration in the orientation with fewer rows, then per step
// A = X X^T, optionally A A, B = b A + c A A, X <- a X + B X on the library's
// k-contiguous GEMM (X^T kept as a second copy so that both products are
// k-contiguous), and finally w <- w (1 - lr wd) - lr s X with the cast.
// Matrices of one shape (the same projection of every layer) go through
// together: each kernel takes the batch on its grid's y axis, each product is
// one batched GEMM, so the small per-matrix products (25 to 100 tiles) fill
// the chip.

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int kNormBlocks = 1024;

template <typename T>
__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ w, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v, T* __restrict__ out,
                                                    int64_t n, float lr, float b1, float b2, float eps, float wd,
                                                    float step_size, float inv_sqrt_bc2) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float gi = g[i];
    float wi = w[i] * (1.f - lr * wd);
    const float mi = b1 * m[i] + (1.f - b1) * gi;
    const float vi = b2 * v[i] + (1.f - b2) * gi * gi;
    wi -= step_size * mi / (sqrtf(vi) * inv_sqrt_bc2 + eps);
    w[i] = wi;
    m[i] = mi;
    v[i] = vi;
    out[i] = from_f32<T>(wi);
  }
}

struct MuonPtrs {
  float* w[kMuonBatch];
  const float* g[kMuonBatch];
  float* u[kMuonBatch];
  void* out[kMuonBatch];
};

// matrix blockIdx.y: u = mu u + g, per-block partial sums of u^2
__global__ __launch_bounds__(256) void muon_momentum_kernel(MuonPtrs P, float mu, int64_t n,
                                                            float* __restrict__ partials_all) {
  __shared__ float red[4];
  float* __restrict__ u = P.u[blockIdx.y];
  const float* __restrict__ g = P.g[blockIdx.y];
  float* __restrict__ partials = partials_all + (size_t)blockIdx.y * (kNormBlocks + 16);
  float s = 0.f;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const float ui = mu * u[i] + g[i];
    u[i] = ui;
    s += ui * ui;
  }
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) partials[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// inv = 1 / (sqrt(sum of partials) + 1e-7), partials added in order; one
// block per matrix
__global__ __launch_bounds__(256) void inv_norm_kernel(const float* __restrict__ partials_all, int n,
                                                       float* inv_all) {
  __shared__ float red[4];
  const float* __restrict__ partials = partials_all + (size_t)blockIdx.x * (kNormBlocks + 16);
  float* inv = inv_all + blockIdx.x;
  float s = 0.f;
  for (int p = threadIdx.x; p < n; p += 256) s += partials[p];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) *inv = 1.f / (sqrtf(red[0] + red[1] + red[2] + red[3]) + 1e-7f);
}

// dst = (scale ? src * scale : src) in the dtype of dst, optionally
// transposed: src [rows, cols] -> dst [cols, rows]. 64x64 tiles through LDS.
// Matrix j = blockIdx.y: src = (src0 ? src0 + j*rows*cols : the momentum
// P.u[j]), dst = dst0 + j*rows*cols, scale = scales ? scales[j] : 1.
template <typename S, typename D>
__global__ __launch_bounds__(256) void copy_tile_kernel(const S* __restrict__ src0, MuonPtrs P,
                                                        D* __restrict__ dst0, int rows, int cols, int transpose,
                                                        const float* __restrict__ scales) {
  __shared__ float tile[64][65];
  const int j = blockIdx.y;
  const int64_t n = (int64_t)rows * cols;
  const S* __restrict__ src = src0 ? src0 + j * n : reinterpret_cast<const S*>(P.u[j]);
  D* __restrict__ dst = dst0 + j * n;
  const int tiles_c = (cols + 63) / 64;
  const int r0 = (blockIdx.x / tiles_c) * 64, c0 = (blockIdx.x % tiles_c) * 64;
  const float f = scales ? scales[j] : 1.f;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i / 64, c = i % 64;
    if (r0 + r < rows && c0 + c < cols) tile[r][c] = to_f32(src[(int64_t)(r0 + r) * cols + c0 + c]) * f;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    if (transpose) {
      const int c = i / 64, r = i % 64;
      if (r0 + r < rows && c0 + c < cols) dst[(int64_t)(c0 + c) * rows + r0 + r] = from_f32<D>(tile[r][c]);
    } else {
      const int r = i / 64, c = i % 64;
      if (r0 + r < rows && c0 + c < cols) dst[(int64_t)(r0 + r) * cols + c0 + c] = from_f32<D>(tile[r][c]);
    }
  }
}

// B = b A + c AA (AA may be null when c == 0); X scaled by a in the same pass
template <typename T>
__global__ __launch_bounds__(256) void ns_combine_kernel(const T* __restrict__ A, const T* __restrict__ AA,
                                                         T* __restrict__ Bm, int64_t nA, float b, float c,
                                                         T* __restrict__ X, int64_t nX, float a) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nA; i += (int64_t)gridDim.x * blockDim.x) {
    float v = b * to_f32(A[i]);
    if (AA) v += c * to_f32(AA[i]);
    Bm[i] = from_f32<T>(v);
  }
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nX; i += (int64_t)gridDim.x * blockDim.x)
    X[i] = from_f32<T>(a * to_f32(X[i]));
}

// w <- w (1 - lr wd) - lr s X(i, j), X stored [rows, cols] or transposed; out = cast(w);
// matrix blockIdx.y (its X at X0 + y*rows*cols)
template <typename T>
__global__ __launch_bounds__(256) void muon_apply_kernel(MuonPtrs P, const T* __restrict__ X0, int rows, int cols,
                                                         int transposed, float lr, float wd, float s) {
  const int64_t n = (int64_t)rows * cols;
  float* __restrict__ w = P.w[blockIdx.y];
  T* __restrict__ out = reinterpret_cast<T*>(P.out[blockIdx.y]);
  const T* __restrict__ X = X0 + blockIdx.y * n;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols, c = i % cols;
    const float x = to_f32(X[transposed ? c * rows + r : i]);
    const float wi = w[i] * (1.f - lr * wd) - lr * s * x;
    w[i] = wi;
    out[i] = from_f32<T>(wi);
  }
}

int grid_for(int64_t n) { return (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 8192)); }

template <typename T>
hipError_t adamw_typed(const AdamwArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(adamw_kernel<T>, dim3(grid_for(a.n)), dim3(256), 0, s, a.w, a.g, a.m, a.v, (T*)a.out, a.n, a.lr,
                     a.beta1, a.beta2, a.eps, a.wd, a.step_size, a.inv_sqrt_bc2);
  return hipGetLastError();
}

template <typename T>
hipError_t muon_typed(const MuonArgs& a, hipStream_t s) {
  const int rows = a.rows, cols = a.cols, G = a.count;
  const int64_t n = (int64_t)rows * cols;
  const bool tr = rows > cols;
  const int p = tr ? cols : rows, q = tr ? rows : cols;
  const int dtype = sizeof(T) == 2 ? 1 : 0;
  const int64_t es = sizeof(T);
  T* X = (T*)a.X;
  T* XT = (T*)a.XT;
  T* A = (T*)a.A;
  T* AA = (T*)a.AA;
  T* Bm = (T*)a.Bm;
  MuonPtrs P;
  for (int j = 0; j < G; ++j) {
    P.w[j] = a.w[j];
    P.g[j] = a.g[j];
    P.u[j] = a.u[j];
    P.out[j] = a.out[j];
  }
  hipError_t e;
  hipLaunchKernelGGL(muon_momentum_kernel, dim3(kNormBlocks, G), dim3(256), 0, s, P, a.mu, n, a.partials);
  hipLaunchKernelGGL(inv_norm_kernel, dim3(G), dim3(256), 0, s, (const float*)a.partials, kNormBlocks, a.inv);
  // X_j = u_j / |u_j|, transposed to [p, q] when rows > cols
  const int tiles = ((rows + 63) / 64) * ((cols + 63) / 64);
  hipLaunchKernelGGL((copy_tile_kernel<float, T>), dim3(tiles, G), dim3(256), 0, s, (const float*)nullptr, P, X, rows,
                     cols, (int)tr, (const float*)a.inv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int ptiles = ((p + 63) / 64) * ((q + 63) / 64);
  for (int it = 0; it < a.steps; ++it) {
    hipLaunchKernelGGL((copy_tile_kernel<T, T>), dim3(ptiles, G), dim3(256), 0, s, (const T*)X, P, XT, p, q, 1,
                       (const float*)nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GemmArgs g;
    g.A = X; g.lda = q; g.B = X; g.ldb = q;
    g.M = p; g.N = p; g.K = q;
    g.C = A; g.ldc = p;
    g.batch = G; g.stride_a = g.stride_b = (int64_t)p * q * es; g.stride_c = (int64_t)p * p * es;
    if ((e = launch_gemm(dtype, Epi::Store, g, s)) != hipSuccess) return e;
    const bool quintic = a.c != 0.f;
    if (quintic) {
      GemmArgs h;
      h.A = A; h.lda = p; h.B = A; h.ldb = p;  // A is symmetric: A A = A A^T
      h.M = p; h.N = p; h.K = p;
      h.C = AA; h.ldc = p;
      h.batch = G; h.stride_a = h.stride_b = h.stride_c = (int64_t)p * p * es;
      if ((e = launch_gemm(dtype, Epi::Store, h, s)) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(ns_combine_kernel<T>, dim3(grid_for((int64_t)G * p * q)), dim3(256), 0, s, (const T*)A,
                       quintic ? (const T*)AA : (const T*)nullptr, Bm, (int64_t)G * p * p, a.b, a.c, X,
                       (int64_t)G * p * q, a.a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GemmArgs k;  // X += B X, with X^T [q, p] as the k-contiguous second operand
    k.A = Bm; k.lda = p; k.B = XT; k.ldb = p;
    k.M = p; k.N = q; k.K = p;
    k.C = X; k.ldc = q;
    k.batch = G; k.stride_a = (int64_t)p * p * es; k.stride_b = k.stride_c = (int64_t)p * q * es;
    if ((e = launch_gemm(dtype, Epi::Residual, k, s)) != hipSuccess) return e;
  }
  const float scale = sqrtf(std::max(1.f, (float)rows / (float)cols));
  hipLaunchKernelGGL(muon_apply_kernel<T>, dim3(grid_for(n), G), dim3(256), 0, s, P, (const T*)X, rows, cols, (int)tr,
                     a.lr, a.wd, scale);
  return hipGetLastError();
}

}  // namespace

size_t muon_partials_elems() { return kNormBlocks + 16; }

hipError_t launch_adamw(int dtype, const AdamwArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  return dtype == 1 ? adamw_typed<bf16>(a, s) : adamw_typed<float>(a, s);
}

hipError_t launch_muon(int dtype, const MuonArgs& a, hipStream_t s) {
  if (a.count < 1 || a.count > kMuonBatch) return hipErrorInvalidValue;
  if (a.rows <= 0 || a.cols <= 0) return hipSuccess;
  return dtype == 1 ? muon_typed<bf16>(a, s) : muon_typed<float>(a, s);
}

}  // namespace gk
