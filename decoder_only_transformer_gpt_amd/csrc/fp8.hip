// Per-tensor FP8 (OCP e4m3) quantisation of matmul operands: the absolute
// maximum of a tensor, then codes = e4m3(x * s) with s = 448 / amax, written
// row-major and/or transposed.
//
// FP8 training is named on repo-explainer.com "karpathy/nanochat: The $100
// Full-Stack LLM", section "The Engine Room: Muon and FP8", and FP8 matmuls as
// an option on atlas.blal.pro "nanochat — full-stack ChatGPT in ~8k lines",
// section "How it works", item "2. Pretrain". The pages give no recipe; the
// library's reading: current per-tensor scaling, s = 448 / amax in fp32
// (s = 1 for an all-zero tensor), round to nearest even, saturation at +-448.
//
// Both kernels are HBM-bound streams. The amax kernel reads 16 bytes per lane
// per load and folds a block's maximum into the tensor's slot with one atomic
// (non-negative floats order like their bit patterns). The quantiser takes a
// 64 x 64 tile per block: 16 consecutive elements per lane in, 16 codes per
// lane out row-major, and the transpose through a byte tile in LDS so that
// the transposed copy is also written 16 bytes per lane.

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int kAmaxElemsPerBlock = 256 * 8 * 8;  // 256 lanes x 8 loads x 8 bf16

// Tensor of this block in a batched table: the last whose first block (amax
// pass or quantise pass) is at most blockIdx.x.
template <bool AMAX>
DEV int find_desc(const QuantDesc* table, int n) {
  int t = 0;
  while (t + 1 < n && (int64_t)blockIdx.x >= (AMAX ? table[t + 1].amax_block0 : table[t + 1].quant_block0)) ++t;
  return t;
}

// A single tensor runs on a capped grid, each block striding over chunks of
// kAmaxElemsPerBlock elements, so that few blocks contend for the one atomic
// slot; a batched table gives every tensor one block per chunk.
__global__ __launch_bounds__(256) void amax_kernel(const QuantDesc* __restrict__ table, int n, QuantDesc one) {
  const QuantDesc d = table ? table[find_desc<true>(table, n)] : one;
  const int64_t ne = (int64_t)d.rows * d.cols;
  const int64_t stride = table ? (int64_t)1 << 62 : (int64_t)gridDim.x * kAmaxElemsPerBlock;
  float m = 0.f;
  for (int64_t base = ((int64_t)blockIdx.x - d.amax_block0) * kAmaxElemsPerBlock; base < ne; base += stride) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t e = base + ((int64_t)i * 256 + threadIdx.x) * 8;
      if (e < ne) {
        float v[8];
        load8(reinterpret_cast<const bf16*>(d.src) + e, v);
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
      }
    }
  }
  m = wave_max(m);
  __shared__ float wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
    atomicMax(reinterpret_cast<unsigned*>(d.amax), __float_as_uint(m));
  }
}

DEV float clamp448(float y) { return y > 448.f ? 448.f : (y < -448.f ? -448.f : y); }  // NaN passes

__global__ __launch_bounds__(256) void quantize_kernel(const QuantDesc* __restrict__ table, int n, QuantDesc one) {
  constexpr int P = 80;  // LDS pitch (bytes) of the [64 cols][64 rows] code tile, 16-byte aligned rows
  __shared__ __attribute__((aligned(16))) uint8_t tt[64 * P];
  const QuantDesc d = table ? table[find_desc<false>(table, n)] : one;
  const int64_t local = (int64_t)blockIdx.x - d.quant_block0;
  const int tiles_c = d.cols / 64 + (d.cols % 64 != 0);
  const int r0 = (int)(local / tiles_c) * 64, c0 = (int)(local % tiles_c) * 64;
  const float am = *d.amax;
  const float s = am > 0.f ? 448.f / am : 1.f;
  const int tid = threadIdx.x, r = tid >> 2, cs = (tid & 3) * 16;
  const int gr = r0 + r, gc = c0 + cs;
  const bool in = gr < d.rows && gc < d.cols;
  float v[16];
  if (in) {
    const bf16* p = reinterpret_cast<const bf16*>(d.src) + (int64_t)gr * d.ld + gc;
    load8(p, *reinterpret_cast<float(*)[8]>(&v[0]));
    load8(p + 8, *reinterpret_cast<float(*)[8]>(&v[8]));
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = 0.f;
  }
  u32x4 q;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    q[w] = pack_fp8x4(clamp448(v[4 * w] * s), clamp448(v[4 * w + 1] * s), clamp448(v[4 * w + 2] * s),
                      clamp448(v[4 * w + 3] * s));
  if (d.q && in) st16(d.q + (int64_t)gr * d.cols + gc, q);
  if (!d.qT) return;  // uniform per block
#pragma unroll
  for (int k = 0; k < 16; ++k) tt[(cs + k) * P + r] = (uint8_t)(q[k >> 2] >> (8 * (k & 3)));
  __syncthreads();
  const int oc = tid >> 2, orow = (tid & 3) * 16;  // output row c0 + oc, columns r0 + orow ..
  if (c0 + oc < d.cols && r0 + orow < d.ldT)
    st16(d.qT + (int64_t)(c0 + oc) * d.ldT + r0 + orow, ld16(tt + oc * P + orow));
}

}  // namespace

int64_t quant_blocks(const QuantDesc& d) {
  const int64_t rows = d.qT ? (d.ldT > d.rows ? d.ldT : d.rows) : d.rows;
  return ((rows + 63) / 64) * ((d.cols + 63) / 64);
}
int64_t amax_blocks(const QuantDesc& d) {
  return ((int64_t)d.rows * d.cols + kAmaxElemsPerBlock - 1) / kAmaxElemsPerBlock;
}

hipError_t check_quant_desc(const QuantDesc& d) {
  if (!d.src || !d.amax || d.rows < 0 || d.cols < 0 || d.cols % 16 != 0 || d.ld % 8 != 0 || d.ld < d.cols)
    return hipErrorInvalidValue;
  if (d.qT && (d.ldT < d.rows || d.ldT % 16 != 0)) return hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_fp8_amax(const QuantDesc& d, hipStream_t s) {
  if (hipError_t e = check_quant_desc(d); e != hipSuccess) return e;
  if (d.ld != d.cols) return hipErrorInvalidValue;  // the amax pass streams a contiguous tensor
  QuantDesc one = d;
  one.amax_block0 = 0;
  const int64_t nb = std::min<int64_t>(amax_blocks(d), 1024);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)nb), dim3(256), 0, s, (const QuantDesc*)nullptr, 0, one);
  return hipGetLastError();
}

hipError_t launch_fp8_quantize(const QuantDesc& d, hipStream_t s) {
  if (hipError_t e = check_quant_desc(d); e != hipSuccess) return e;
  QuantDesc one = d;
  one.quant_block0 = 0;
  const int64_t nb = quant_blocks(d);
  if (nb == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)nb), dim3(256), 0, s, (const QuantDesc*)nullptr, 0, one);
  return hipGetLastError();
}

hipError_t launch_fp8_amax_batched(const QuantDesc* table, int n, int64_t total_blocks, hipStream_t s) {
  if (total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)total_blocks), dim3(256), 0, s, table, n, QuantDesc{});
  return hipGetLastError();
}

hipError_t launch_fp8_quantize_batched(const QuantDesc* table, int n, int64_t total_blocks, hipStream_t s) {
  if (total_blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)total_blocks), dim3(256), 0, s, table, n, QuantDesc{});
  return hipGetLastError();
}

}  // namespace gk
