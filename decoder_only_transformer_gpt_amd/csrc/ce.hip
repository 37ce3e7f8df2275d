// Softcapped cross-entropy over the vocabulary.
//
// The LM head GEMM epilogue has already squashed the logits to
// z' = c * tanh(z / c) (c = 15, in fp32; aethryn.com "Nanochat: full-stack LLM
// training in 8,000 lines for $72", section "A Llama-class transformer with
// ten modern departures") and emitted, per row and 64 columns, the partial
// sums of exp(z' - c). Because |z'| < c every term lies in (e^-2c, 1], so the
// log-sum-exp is c + log(sum of partials) with no running maximum.
//
//   row loss  l_n = lse_n - z'_{n, target}
//   loss      = mean over all B*T rows (fixed-order reduction: deterministic)
//   backward  dz_nv = (exp(z'_nv - lse_n) - [v == target]) * dloss / N * (1 - (z'_nv / c)^2)
//
// The epilogue stores q_nv = exp(z'_nv - c) (1 - (z'_nv / c)^2) instead of z'.
// With s_n = exp(lse_n - c) (the row's sum of exp(z' - c)) and
// r_n = dloss / (N s_n), dz_nv = r_n q_nv except at the target, where
// dz = r_n (q - (1 - (z'/c)^2) s_n). The backward therefore never makes a
// pass over the N x V matrix: one wave per row rewrites the target entry
// (from the fp32 z' at the target, with the same exp2 the epilogue used),
// stores r_n, and writes the row of the final-norm output scaled by r_n; the
// LM-head dW GEMM reads that scaled copy, and the dX GEMM's rows are scaled
// by r_n in the final norm's backward.

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
  // 16-byte loads, four per lane in flight per round (nparts = V / 64 is a
  // multiple of 4), then a fixed butterfly over the lanes
  float s = 0.f;
  if ((nparts & 3) == 0) {
    const int n4 = nparts >> 2;
    int i = lane;
    for (; i + 192 < n4; i += 256) {
      f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * i), b = *reinterpret_cast<const f32x4*>(p + 4 * (i + 64));
      f32x4 c2 = *reinterpret_cast<const f32x4*>(p + 4 * (i + 128)), d = *reinterpret_cast<const f32x4*>(p + 4 * (i + 192));
      s += ((a[0] + a[1]) + (a[2] + a[3])) + ((b[0] + b[1]) + (b[2] + b[3])) + ((c2[0] + c2[1]) + (c2[2] + c2[3])) +
           ((d[0] + d[1]) + (d[2] + d[3]));
    }
    for (; i < n4; i += 64) {
      f32x4 a = *reinterpret_cast<const f32x4*>(p + 4 * i);
      s += (a[0] + a[1]) + (a[2] + a[3]);
    }
  } else {
    for (int i = lane; i < nparts; i += 64) s += p[i];
  }
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

// Single block: mean of N row losses in a fixed order (16-byte loads, four
// in flight per thread).
__global__ __launch_bounds__(1024) void mean_kernel(const float* __restrict__ x, int N, float* __restrict__ out) {
  __shared__ float red[16];
  float s = 0.f;
  const int n4 = N >> 2;
  int i = threadIdx.x;
  for (; i + 3072 < n4; i += 4096) {
    const f32x4 a = reinterpret_cast<const f32x4*>(x)[i], b = reinterpret_cast<const f32x4*>(x)[i + 1024];
    const f32x4 c = reinterpret_cast<const f32x4*>(x)[i + 2048], d = reinterpret_cast<const f32x4*>(x)[i + 3072];
    s += ((a[0] + a[1]) + (a[2] + a[3])) + ((b[0] + b[1]) + (b[2] + b[3])) + ((c[0] + c[1]) + (c[2] + c[3])) +
         ((d[0] + d[1]) + (d[2] + d[3]));
  }
  for (; i < n4; i += 1024) {
    const f32x4 a = reinterpret_cast<const f32x4*>(x)[i];
    s += (a[0] + a[1]) + (a[2] + a[3]);
  }
  for (int j = 4 * n4 + (int)threadIdx.x; j < N; j += 1024) s += x[j];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x < 64) {
    float v = threadIdx.x < 16 ? red[threadIdx.x] : 0.f;
    v = wave_sum(v);
    if (threadIdx.x == 0) *out = v / (float)N;
  }
}

// One wave per row: the target-column fix of q, the row scale r, and the
// final-norm output row h scaled by r (bf16 or fp32 like h).
template <typename T, int J>
__global__ __launch_bounds__(256) void ce_grad_prep_kernel(T* __restrict__ q, const float* __restrict__ lse,
                                                           const float* __restrict__ ztgt,
                                                           const int32_t* __restrict__ targets, int N, int V,
                                                           float c, float scale, const T* __restrict__ h, int C,
                                                           T* __restrict__ hs, float* __restrict__ rscale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  if (row >= N) return;
  // the row of h is requested before r is known (J groups of 512 columns;
  // lanes past the row re-read its last 8 columns, so no load is conditional)
  const int64_t off = (int64_t)row * C;
  float v[J][8];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int k = j * 512 + lane * 8;
    load8(h + off + (k < C ? k : C - 8), v[j]);
  }
  const float s = expf(lse[row] - c);
  const float r = scale / s;
  if (lane == 0) {
    rscale[row] = r;
    const int t = targets[row];
    if ((unsigned)t < (unsigned)V) {
      const float z = ztgt[row], u = z / c;
      const float e = __builtin_amdgcn_exp2f((z - c) * 1.4426950408889634f);
      q[(int64_t)row * V + t] = from_f32<T>((1.f - u * u) * (e - s));
    }
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int k = j * 512 + lane * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[j][e] *= r;
    if (k < C) store8(hs + off + k, v[j]);
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

template <typename T, int J>
hipError_t ce_grad_prep_j(void* q, const float* lse, const float* ztgt, const int32_t* targets, int N, int V,
                          float softcap, float scale, const void* h, int C, void* hs, float* rscale, hipStream_t s) {
  hipLaunchKernelGGL((ce_grad_prep_kernel<T, J>), dim3((N + 3) / 4), dim3(256), 0, s, (T*)q, lse, ztgt, targets, N, V,
                     softcap, scale, (const T*)h, C, (T*)hs, rscale);
  return hipGetLastError();
}

template <typename T>
hipError_t ce_grad_prep_t(void* q, const float* lse, const float* ztgt, const int32_t* targets, int N, int V,
                          float softcap, float scale, const void* h, int C, void* hs, float* rscale, hipStream_t s) {
  switch ((C + 511) / 512) {  // 512-column groups per row
    case 1: return ce_grad_prep_j<T, 1>(q, lse, ztgt, targets, N, V, softcap, scale, h, C, hs, rscale, s);
    case 2: return ce_grad_prep_j<T, 2>(q, lse, ztgt, targets, N, V, softcap, scale, h, C, hs, rscale, s);
    case 3: return ce_grad_prep_j<T, 3>(q, lse, ztgt, targets, N, V, softcap, scale, h, C, hs, rscale, s);
    case 4: return ce_grad_prep_j<T, 4>(q, lse, ztgt, targets, N, V, softcap, scale, h, C, hs, rscale, s);
    case 5: return ce_grad_prep_j<T, 5>(q, lse, ztgt, targets, N, V, softcap, scale, h, C, hs, rscale, s);
    case 6: return ce_grad_prep_j<T, 6>(q, lse, ztgt, targets, N, V, softcap, scale, h, C, hs, rscale, s);
    case 7: return ce_grad_prep_j<T, 7>(q, lse, ztgt, targets, N, V, softcap, scale, h, C, hs, rscale, s);
    case 8: return ce_grad_prep_j<T, 8>(q, lse, ztgt, targets, N, V, softcap, scale, h, C, hs, rscale, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_ce_grad_prep(int dtype, void* q, const float* lse, const float* ztgt, const int32_t* targets, int N,
                               int V, float softcap, float scale, const void* h, int C, void* hs, float* rscale,
                               hipStream_t s) {
  if (C % 8 != 0 || C < 8 || C > 4096) return hipErrorInvalidValue;
  return dtype == 1 ? ce_grad_prep_t<bf16>(q, lse, ztgt, targets, N, V, softcap, scale, h, C, hs, rscale, s)
                    : ce_grad_prep_t<float>(q, lse, ztgt, targets, N, V, softcap, scale, h, C, hs, rscale, s);
}

}  // namespace gk
