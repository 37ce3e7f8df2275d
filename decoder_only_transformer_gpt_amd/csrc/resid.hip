// Per-layer residual scalars and value embeddings (aethryn.com "Nanochat:
// full-stack LLM training in 8,000 lines for $72", section "A Llama-class
// transformer with ten modern departures": resid_lambdas and x0_lambdas mix
// each layer's residual stream with the normalised embedding; a gated
// embedding lookup adds to V at alternating layers; atlas.blal.pro "nanochat
// — full-stack ChatGPT in ~8k lines", section "How it works", item 0).
//
// The library's reading: before layer l, x <- resid_lambdas[l] * x +
// x0_lambdas[l] * x0 (x0 = rmsnorm(wte[idx])); on layers 0, 2, 4, ...
// v <- v + gate_j * ve_j[idx] right after the QKV projection.
//
// All of it is elementwise and HBM-bound (16-byte vector access). The scalar
// gradients are dot products over the whole batch: fixed grids write one
// partial per block and a single block adds the partials in order, so every
// sum is bitwise reproducible.

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int kPartBlocks = 1024;  // grid of the partial-sum kernels

DEV float block_sum256(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float s = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return s;
}

// x_prev stash = x; x = lr * x + l0 * x0 (8 elements per lane-step)
template <typename T>
__global__ __launch_bounds__(256) void x0_mix_kernel(T* __restrict__ x, const T* __restrict__ x0,
                                                     T* __restrict__ xprev, const T* __restrict__ lam_r,
                                                     const T* __restrict__ lam_0, int64_t n8) {
  const float lr = to_f32(*lam_r), l0 = to_f32(*lam_0);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    float a[8], b[8];
    load8(x + i * 8, a);
    load8(x0 + i * 8, b);
    store8(xprev + i * 8, a);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = lr * a[e] + l0 * b[e];
    store8(x + i * 8, a);
  }
}

// Backward of the mix at layer l, d = dL/dx_in (fp32 in dres, or in the
// activation dtype in dres_lp alone when dres is null):
//   partials: sum d * x_prev, sum d * x0 (for the two scalars' gradients);
//   l > 0: dx0acc += l0 * d, d <- lr * d;  l == 0 (x_prev is x0 itself):
//   d <- lr * d + l0 * d + dx0acc, the whole gradient reaching x0.
template <typename T>
__global__ __launch_bounds__(256) void x0_mix_bwd_kernel(float* __restrict__ dres, T* __restrict__ dres_lp,
                                                         const T* __restrict__ xprev, const T* __restrict__ x0,
                                                         float* __restrict__ dx0acc, const T* __restrict__ lam_r,
                                                         const T* __restrict__ lam_0, int first, int64_t n8,
                                                         float* __restrict__ partials) {
  __shared__ float red[4];
  const float lr = to_f32(*lam_r), l0 = to_f32(*lam_0);
  float pr = 0.f, p0 = 0.f;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    float d[8], xp[8], z[8], acc[8];
    if (dres)
      load8(dres + i * 8, d);
    else
      load8(dres_lp + i * 8, d);
    load8(xprev + i * 8, xp);
    load8(x0 + i * 8, z);
    load8(dx0acc + i * 8, acc);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr += d[e] * xp[e];
      p0 += d[e] * z[e];
    }
    if (first) {
#pragma unroll
      for (int e = 0; e < 8; ++e) d[e] = lr * d[e] + l0 * d[e] + acc[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[e] += l0 * d[e];
        d[e] *= lr;
      }
      store8(dx0acc + i * 8, acc);
    }
    if (dres) store8(dres + i * 8, d);
    store8(dres_lp + i * 8, d);
  }
  pr = block_sum256(pr, red);
  p0 = block_sum256(p0, red);
  if (threadIdx.x == 0) {
    partials[blockIdx.x * 2] = pr;
    partials[blockIdx.x * 2 + 1] = p0;
  }
}

// out[j] (+)= sum over p of partials[p * nout + j], one block per output,
// fixed order
__global__ __launch_bounds__(256) void scalar_grad_kernel(const float* __restrict__ partials, int nparts, int nout,
                                                          float* out0, float* out1, int accumulate) {
  __shared__ float red[4];
  const int j = blockIdx.x;
  float s = 0.f;
  for (int p = threadIdx.x; p < nparts; p += 256) s += partials[p * nout + j];
  s = block_sum256(s, red);
  if (threadIdx.x == 0) {
    float* o = j == 0 ? out0 : out1;
    *o = accumulate ? *o + s : s;
  }
}

// v[n] += gate * ve[idx[n]]: 16 lanes per token, 8 values per lane
template <typename T>
__global__ __launch_bounds__(256) void ve_add_kernel(T* __restrict__ qkv, int64_t ld, int col0,
                                                     const int32_t* __restrict__ idx, const T* __restrict__ ve,
                                                     const T* __restrict__ gate, int N, int V) {
  const int n = blockIdx.x * 16 + (threadIdx.x >> 4), j = threadIdx.x & 15;
  if (n >= N) return;
  const int id = idx[n];
  if ((unsigned)id >= (unsigned)V) return;  // the embedding kernel has raised the device flag
  const float g = to_f32(*gate);
  T* v = qkv + (int64_t)n * ld + col0 + j * 8;
  float a[8], b[8];
  load8(v, a);
  load8(ve + (int64_t)id * 128 + j * 8, b);
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] += g * b[e];
  store8(v, a);
}

// partials[block] = sum over the block's tokens of <dv[n], ve[idx[n]]>
template <typename T>
__global__ __launch_bounds__(256) void ve_gate_partials_kernel(const T* __restrict__ dqkv, int64_t ld, int col0,
                                                               const int32_t* __restrict__ idx,
                                                               const T* __restrict__ ve, int N, int V,
                                                               float* __restrict__ partials) {
  __shared__ float red[4];
  const int j = threadIdx.x & 15;
  float s = 0.f;
  for (int n = blockIdx.x * 16 + (threadIdx.x >> 4); n < N; n += gridDim.x * 16) {
    const int id = idx[n];
    if ((unsigned)id >= (unsigned)V) continue;
    float a[8], b[8];
    load8(dqkv + (int64_t)n * ld + col0 + j * 8, a);
    load8(ve + (int64_t)id * 128 + j * 8, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += a[e] * b[e];
  }
  s = block_sum256(s, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

}  // namespace

size_t resid_partials_elems() { return 2 * kPartBlocks; }

hipError_t launch_x0_mix(int dtype, void* x, const void* x0, void* xprev, const void* lam_r, const void* lam_0,
                         int64_t n, hipStream_t s) {
  if (n % 8 != 0) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  const int blocks = (int)std::min<int64_t>((n8 + 255) / 256, 4096);
  if (blocks == 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(x0_mix_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (bf16*)x, (const bf16*)x0, (bf16*)xprev,
                       (const bf16*)lam_r, (const bf16*)lam_0, n8);
  else
    hipLaunchKernelGGL(x0_mix_kernel<float>, dim3(blocks), dim3(256), 0, s, (float*)x, (const float*)x0,
                       (float*)xprev, (const float*)lam_r, (const float*)lam_0, n8);
  return hipGetLastError();
}

hipError_t launch_x0_mix_bwd(int dtype, float* dres, void* dres_lp, const void* xprev, const void* x0, float* dx0acc,
                             const void* lam_r, const void* lam_0, int first, int64_t n, float* partials,
                             float* g_lam_r, float* g_lam_0, int accumulate, hipStream_t s) {
  if (n % 8 != 0) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  if (dtype == 1)
    hipLaunchKernelGGL(x0_mix_bwd_kernel<bf16>, dim3(kPartBlocks), dim3(256), 0, s, dres, (bf16*)dres_lp,
                       (const bf16*)xprev, (const bf16*)x0, dx0acc, (const bf16*)lam_r, (const bf16*)lam_0, first, n8,
                       partials);
  else
    hipLaunchKernelGGL(x0_mix_bwd_kernel<float>, dim3(kPartBlocks), dim3(256), 0, s, dres, (float*)dres_lp,
                       (const float*)xprev, (const float*)x0, dx0acc, (const float*)lam_r, (const float*)lam_0, first,
                       n8, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scalar_grad_kernel, dim3(2), dim3(256), 0, s, (const float*)partials, kPartBlocks, 2, g_lam_r,
                     g_lam_0, accumulate);
  return hipGetLastError();
}

hipError_t launch_ve_add(int dtype, void* qkv, int64_t ld, int col0, const int32_t* idx, const void* ve,
                         const void* gate, int N, int V, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(ve_add_kernel<bf16>, dim3((N + 15) / 16), dim3(256), 0, s, (bf16*)qkv, ld, col0, idx,
                       (const bf16*)ve, (const bf16*)gate, N, V);
  else
    hipLaunchKernelGGL(ve_add_kernel<float>, dim3((N + 15) / 16), dim3(256), 0, s, (float*)qkv, ld, col0, idx,
                       (const float*)ve, (const float*)gate, N, V);
  return hipGetLastError();
}

hipError_t launch_ve_gate_grad(int dtype, const void* dqkv, int64_t ld, int col0, const int32_t* idx, const void* ve,
                               int N, int V, float* partials, float* g_gate, int accumulate, hipStream_t s) {
  if (dtype == 1)
    hipLaunchKernelGGL(ve_gate_partials_kernel<bf16>, dim3(kPartBlocks), dim3(256), 0, s, (const bf16*)dqkv, ld, col0,
                       idx, (const bf16*)ve, N, V, partials);
  else
    hipLaunchKernelGGL(ve_gate_partials_kernel<float>, dim3(kPartBlocks), dim3(256), 0, s, (const float*)dqkv, ld,
                       col0, idx, (const float*)ve, N, V, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scalar_grad_kernel, dim3(1), dim3(256), 0, s, (const float*)partials, kPartBlocks, 1, g_gate,
                     g_gate, accumulate);
  return hipGetLastError();
}

}  // namespace gk
