// Softcapped cross-entropy over the vocabulary.
//
// The LM head GEMM epilogue has already squashed the logits to
// z' = c * tanh(z / c) (c = 15, in fp32; aethryn.com "Nanochat: full-stack LLM
// training in 8,000 lines for $72", section "A Llama-class transformer with
// ten modern departures") and emitted, per row and 128 columns, the partial
// sums of exp(z' - c). Because |z'| < c every term lies in (e^-2c, 1], so the
// log-sum-exp is c + log(sum of partials) with no running maximum.
//
//   row loss  l_n = lse_n - z'_{n, target}
//   loss      = mean over all B*T rows (fixed-order reduction: deterministic)
//   backward  dz_nv = (exp(z'_nv - lse_n) - [v == target]) * dloss / N * (1 - (z'_nv / c)^2)
//
// The backward overwrites the stored logits in place with dz, which is what
// the two LM-head backward GEMMs read.

#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

// One wave per row: sums the row's partials in a fixed order.
__global__ __launch_bounds__(256) void ce_rows_kernel(const float* __restrict__ part, int nparts,
                                                      const float* __restrict__ ztgt,
                                                      const int32_t* __restrict__ targets, int N, int V,
                                                      float c, float* __restrict__ lse,
                                                      float* __restrict__ row_loss, float* __restrict__ row_out,
                                                      int* flag) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= N) return;
  const float* p = part + (int64_t)row * nparts;
  float s = 0.f;
  for (int i = lane; i < nparts; i += 64) s += p[i];
  s = wave_sum(s);
  if (lane == 0) {
    const float l = c + logf(s);
    const int t = targets[row];
    float loss;
    if ((unsigned)t >= (unsigned)V) {
      loss = __builtin_nanf("");
      *flag = FLAG_BAD_TOKEN;
    } else {
      loss = l - ztgt[row];
    }
    lse[row] = l;
    row_loss[row] = loss;
    if (row_out) row_out[row] = loss;
  }
}

// Single block: mean of N row losses in a fixed order.
__global__ __launch_bounds__(1024) void mean_kernel(const float* __restrict__ x, int N, float* __restrict__ out) {
  __shared__ float red[16];
  float s = 0.f;
  for (int i = threadIdx.x; i < N; i += 1024) s += x[i];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x < 64) {
    float v = threadIdx.x < 16 ? red[threadIdx.x] : 0.f;
    v = wave_sum(v);
    if (threadIdx.x == 0) *out = v / (float)N;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void ce_bwd_kernel(T* __restrict__ z, const float* __restrict__ lse,
                                                     const int32_t* __restrict__ targets, int N, int V, float c,
                                                     float scale) {
  const int64_t nvec = (int64_t)N * V / 8;
  const float inv_c = 1.f / c;
  for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < nvec; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e0 = q * 8;
    const int row = (int)(e0 / V);
    const int col = (int)(e0 % V);
    const float l = lse[row];
    const int t = targets[row];
    float v[8];
    load8(z + e0, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float zc = v[e];
      float p = __expf(zc - l);
      if (col + e == t) p -= 1.f;
      const float u = zc * inv_c;
      v[e] = p * scale * (1.f - u * u);
    }
    store8(z + e0, v);
  }
}

}  // namespace

hipError_t launch_ce_loss(const float* part, int nparts, const float* ztgt, const int32_t* targets, int N, int V,
                          float softcap, float* lse, float* row_loss, float* row_loss_out, float* loss, int* flag,
                          hipStream_t s) {
  hipLaunchKernelGGL(ce_rows_kernel, dim3((N + 3) / 4), dim3(256), 0, s, part, nparts, ztgt, targets, N, V, softcap,
                     lse, row_loss, row_loss_out, flag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(1024), 0, s, row_loss, N, loss);
  return hipGetLastError();
}

hipError_t launch_ce_bwd(int dtype, void* logits, const float* lse, const int32_t* targets, int N, int V,
                         float softcap, float scale, hipStream_t s) {
  const int64_t nvec = (int64_t)N * V / 8;
  const int blocks = (int)std::min<int64_t>((nvec + 255) / 256, 256 * 64);
  if (dtype == 1)
    hipLaunchKernelGGL(ce_bwd_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (bf16*)logits, lse, targets, N, V,
                       softcap, scale);
  else
    hipLaunchKernelGGL(ce_bwd_kernel<float>, dim3(blocks), dim3(256), 0, s, (float*)logits, lse, targets, N, V,
                       softcap, scale);
  return hipGetLastError();
}

}  // namespace gk
