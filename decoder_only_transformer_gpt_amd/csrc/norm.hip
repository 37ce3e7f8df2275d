// Row-wise kernels: embedding gather + RMSNorm, RMSNorm forward/backward, and
// the fused RoPE + QK-RMSNorm forward/backward.
//
// RMSNorm has no learnable gain and is applied after the embedding, before
// every attention and MLP block and before the LM head; RoPE (base 10,000) is
// applied to q and k, then q and k are RMS-normalised (aethryn.com "Nanochat:
// full-stack LLM training in 8,000 lines for $72", section "A Llama-class
// transformer with ten modern departures"; energyai.berlin "nanochat vs
// GPT-OSS", section "Architectural decisions", subsections RoPE, RMSNorm and
// QK normalization). eps and the RoPE pairing are the library's stated
// conventions (i with i + D/2, rotation by +t * theta^(-2i/D)).
//
// All of these are HBM-bound: one wave owns a row (RMSNorm) or a 16-lane
// group owns one 128-wide head (RoPE + QK-norm), rows are read once with
// 16-byte vector loads kept in registers, reduced with cross-lane shuffles,
// and written once.

#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int kMaxChunks = 8;  // 8-element chunks per lane: C <= 64 * 8 * 8 = 4096

// A wave owns a row; lane L holds the 8-element chunks L + 64 j, j < J, with
// J = ceil(C / 512) a template argument (register arrays sized to the row).
// Where the last round has no chunk for a lane, the lane loads the row's last
// chunk again and drops it: every load is issued unconditionally, back to
// back, before the first use. (A load under a per-lane test is waited for
// inside the test, so the rounds' loads would go out one round at a time.)
DEV int chunk_of(int lane, int j, int nch) { return min(lane + j * 64, nch - 1); }

// --------------------------------------------------------------- RMSNorm --

template <typename T, bool GATHER, int J>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* __restrict__ src, const int32_t* __restrict__ idx,
                                                      int N, int C, int V, float eps, T* __restrict__ y,
                                                      float* __restrict__ rstd, int* flag) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= N) return;
  int64_t srow = row;
  bool bad = false;
  if constexpr (GATHER) {
    const int id = idx[row];
    bad = (unsigned)id >= (unsigned)V;
    srow = bad ? 0 : id;
  }
  const T* s = src + srow * C;
  const int nch = C >> 3;
  float v[J][8];
#pragma unroll
  for (int j = 0; j < J; ++j) load8(s + chunk_of(lane, j, nch) * 8, v[j]);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) t += v[j][e] * v[j][e];
    ss += lane + j * 64 < nch ? t : 0.f;
  }
  ss = wave_sum(ss);
  float r = rsqrtf(ss / (float)C + eps);
  if (bad) {
    r = __builtin_nanf("");
    if (lane == 0) *flag = FLAG_BAD_TOKEN;
  }
  T* d = y + (int64_t)row * C;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int ch = lane + j * 64;
    if (ch < nch) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = v[j][e] * r;
      store8(d + ch * 8, o);
    }
  }
  if (lane == 0) rstd[row] = r;
}

// dres = (accumulate ? dres : 0) + r * (dy - y * mean(dy * y)); dres_lp = dres (activation dtype).
// With dres null the residual gradient lives in dres_lp alone (activation
// dtype, accumulated in fp32 inside the kernel and rounded once per call).
template <typename T, int J>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const T* __restrict__ dy, const T* __restrict__ y,
                                                          const float* __restrict__ rstd, int N, int C,
                                                          int accumulate, float* __restrict__ dres,
                                                          T* __restrict__ dres_lp,
                                                          const float* __restrict__ dy_row_scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= N) return;
  const int64_t off = (int64_t)row * C;
  const int nch = C >> 3;
  const float gs = dy_row_scale ? dy_row_scale[row] : 1.f;
  const float r = rstd[row];
  float g[J][8], yy[J][8], o[J][8];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int ch = chunk_of(lane, j, nch);
    load8(dy + off + ch * 8, g[j]);
    load8(y + off + ch * 8, yy[j]);
  }
  if (accumulate) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (dres)
        load8(dres + off + chunk_of(lane, j, nch) * 8, o[j]);
      else
        load8(dres_lp + off + chunk_of(lane, j, nch) * 8, o[j]);
    }
  }
  float dot = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      g[j][e] *= gs;
      t += g[j][e] * yy[j][e];
    }
    dot += lane + j * 64 < nch ? t : 0.f;
  }
  dot = wave_sum(dot) / (float)C;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int ch = lane + j * 64;
    if (ch < nch) {
      float out[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dx = r * (g[j][e] - yy[j][e] * dot);
        out[e] = accumulate ? o[j][e] + dx : dx;
      }
      if (dres) store8(dres + off + ch * 8, out);
      store8(dres_lp + off + ch * 8, out);
    }
  }
}

// -------------------------------------------------------- RoPE + QK-norm --
// qkv row layout: [H query heads | 1 K head | 1 V head], 128 each.
// A 16-lane group owns one (token, head); lane j holds x[4j..4j+3] and
// x[64+4j..64+4j+3], so each rotation pair (i, i+64) sits in one lane.

template <typename T>
__global__ __launch_bounds__(256) void rope_qknorm_kernel(T* __restrict__ qkv, int N, int T_, int H, float eps,
                                                          const float* __restrict__ cos_t,
                                                          const float* __restrict__ sin_t,
                                                          float* __restrict__ rstd_qk) {
  const int grp = (blockIdx.x * 256 + threadIdx.x) >> 4;  // (token, head) index
  const int j = threadIdx.x & 15;
  const int nh = H + 1;
  if (grp >= N * nh) return;  // whole 16-lane groups exit together
  const int n = grp / nh, h = grp % nh;
  const int t = n % T_;
  T* p = qkv + (int64_t)n * (H + 2) * 128 + h * 128;
  float a[4], b[4], c[4], s[4];
  load4(p + 4 * j, a);
  load4(p + 64 + 4 * j, b);
  load4(cos_t + t * 64 + 4 * j, c);
  load4(sin_t + t * 64 + 4 * j, s);
  float ra[4], rb[4], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ra[e] = a[e] * c[e] - b[e] * s[e];
    rb[e] = a[e] * s[e] + b[e] * c[e];
    ss += ra[e] * ra[e] + rb[e] * rb[e];
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 16);
  const float r = rsqrtf(ss * (1.f / 128.f) + eps);
#pragma unroll
  for (int e = 0; e < 4; ++e) { ra[e] *= r; rb[e] *= r; }
  store4(p + 4 * j, ra);
  store4(p + 64 + 4 * j, rb);
  if (j == 0) rstd_qk[grp] = r;
}

// dqkv holds d(normalised q, k) and dv; qkv holds the normalised q, k.
// dx_rot = r * (dy - y * mean(dy * y)); dx = R^T dx_rot (rotation by -angle).
template <typename T>
__global__ __launch_bounds__(256) void rope_qknorm_bwd_kernel(T* __restrict__ dqkv, const T* __restrict__ qkv,
                                                              const float* __restrict__ rstd_qk, int N, int T_,
                                                              int H, const float* __restrict__ cos_t,
                                                              const float* __restrict__ sin_t) {
  const int grp = (blockIdx.x * 256 + threadIdx.x) >> 4;
  const int j = threadIdx.x & 15;
  const int nh = H + 1;
  if (grp >= N * nh) return;
  const int n = grp / nh, h = grp % nh;
  const int t = n % T_;
  const int64_t off = (int64_t)n * (H + 2) * 128 + h * 128;
  float ga[4], gb[4], ya[4], yb[4], c[4], s[4];
  load4(dqkv + off + 4 * j, ga);
  load4(dqkv + off + 64 + 4 * j, gb);
  load4(qkv + off + 4 * j, ya);
  load4(qkv + off + 64 + 4 * j, yb);
  load4(cos_t + t * 64 + 4 * j, c);
  load4(sin_t + t * 64 + 4 * j, s);
  float dot = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) dot += ga[e] * ya[e] + gb[e] * yb[e];
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 16);
  dot *= (1.f / 128.f);
  const float r = rstd_qk[grp];
  float oa[4], ob[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float xa = r * (ga[e] - ya[e] * dot), xb = r * (gb[e] - yb[e] * dot);
    oa[e] = xa * c[e] + xb * s[e];
    ob[e] = -xa * s[e] + xb * c[e];
  }
  store4(dqkv + off + 4 * j, oa);
  store4(dqkv + off + 64 + 4 * j, ob);
}

__global__ void fill_kernel(float* p, float v, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Launch a row kernel instance with J = ceil(C / 512) chunks per lane.
template <template <int> class K, typename... Args>
hipError_t launch_rows(int C, dim3 grid, hipStream_t s, Args... args) {
  switch ((C / 8 + 63) / 64) {
    case 1: hipLaunchKernelGGL(K<1>::fn, grid, dim3(256), 0, s, args...); break;
    case 2: hipLaunchKernelGGL(K<2>::fn, grid, dim3(256), 0, s, args...); break;
    case 3: hipLaunchKernelGGL(K<3>::fn, grid, dim3(256), 0, s, args...); break;
    case 4: hipLaunchKernelGGL(K<4>::fn, grid, dim3(256), 0, s, args...); break;
    case 5: hipLaunchKernelGGL(K<5>::fn, grid, dim3(256), 0, s, args...); break;
    case 6: hipLaunchKernelGGL(K<6>::fn, grid, dim3(256), 0, s, args...); break;
    case 7: hipLaunchKernelGGL(K<7>::fn, grid, dim3(256), 0, s, args...); break;
    case 8: hipLaunchKernelGGL(K<8>::fn, grid, dim3(256), 0, s, args...); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <typename T, bool GATHER>
struct RmsK {
  template <int J>
  struct At {
    static constexpr auto fn = rmsnorm_kernel<T, GATHER, J>;
  };
};
template <typename T>
struct RmsBwdK {
  template <int J>
  struct At {
    static constexpr auto fn = rmsnorm_bwd_kernel<T, J>;
  };
};

}  // namespace

hipError_t launch_embed_rmsnorm(int dtype, const void* wte, const int32_t* idx, int N, int C, int V, float eps,
                                void* x, float* rstd, int* flag, hipStream_t s) {
  if (C <= 0 || C % 8 != 0 || C > 64 * 8 * kMaxChunks) return hipErrorInvalidValue;
  dim3 grid((N + 3) / 4);
  if (dtype == 1)
    return launch_rows<RmsK<bf16, true>::At>(C, grid, s, (const bf16*)wte, idx, N, C, V, eps, (bf16*)x, rstd, flag);
  return launch_rows<RmsK<float, true>::At>(C, grid, s, (const float*)wte, idx, N, C, V, eps, (float*)x, rstd, flag);
}

hipError_t launch_rmsnorm(int dtype, const void* x, int N, int C, float eps, void* y, float* rstd, hipStream_t s) {
  if (C <= 0 || C % 8 != 0 || C > 64 * 8 * kMaxChunks) return hipErrorInvalidValue;
  dim3 grid((N + 3) / 4);
  if (dtype == 1)
    return launch_rows<RmsK<bf16, false>::At>(C, grid, s, (const bf16*)x, (const int32_t*)nullptr, N, C, 0, eps,
                                              (bf16*)y, rstd, (int*)nullptr);
  return launch_rows<RmsK<float, false>::At>(C, grid, s, (const float*)x, (const int32_t*)nullptr, N, C, 0, eps,
                                             (float*)y, rstd, (int*)nullptr);
}

hipError_t launch_rmsnorm_bwd(int dtype, const void* dy, const void* y, const float* rstd, int N, int C,
                              int accumulate, float* dres, void* dres_lp, hipStream_t s, const float* dy_row_scale) {
  if (C <= 0 || C % 8 != 0 || C > 64 * 8 * kMaxChunks) return hipErrorInvalidValue;
  dim3 grid((N + 3) / 4);
  if (dtype == 1)
    return launch_rows<RmsBwdK<bf16>::At>(C, grid, s, (const bf16*)dy, (const bf16*)y, rstd, N, C, accumulate, dres,
                                          (bf16*)dres_lp, dy_row_scale);
  return launch_rows<RmsBwdK<float>::At>(C, grid, s, (const float*)dy, (const float*)y, rstd, N, C, accumulate,
                                         dres, (float*)dres_lp, dy_row_scale);
}

hipError_t launch_rope_qknorm(int dtype, void* qkv, int B, int T, int H, float eps, const float* cos_t,
                              const float* sin_t, float* rstd_qk, hipStream_t s) {
  const int N = B * T;
  const int64_t groups = (int64_t)N * (H + 1);
  dim3 grid((unsigned)((groups * 16 + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(rope_qknorm_kernel<bf16>, grid, dim3(256), 0, s, (bf16*)qkv, N, T, H, eps, cos_t, sin_t,
                       rstd_qk);
  else
    hipLaunchKernelGGL(rope_qknorm_kernel<float>, grid, dim3(256), 0, s, (float*)qkv, N, T, H, eps, cos_t, sin_t,
                       rstd_qk);
  return hipGetLastError();
}

hipError_t launch_rope_qknorm_bwd(int dtype, void* dqkv, const void* qkv, const float* rstd_qk, int B, int T,
                                  int H, const float* cos_t, const float* sin_t, hipStream_t s) {
  const int N = B * T;
  const int64_t groups = (int64_t)N * (H + 1);
  dim3 grid((unsigned)((groups * 16 + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(rope_qknorm_bwd_kernel<bf16>, grid, dim3(256), 0, s, (bf16*)dqkv, (const bf16*)qkv,
                       rstd_qk, N, T, H, cos_t, sin_t);
  else
    hipLaunchKernelGGL(rope_qknorm_bwd_kernel<float>, grid, dim3(256), 0, s, (float*)dqkv, (const float*)qkv,
                       rstd_qk, N, T, H, cos_t, sin_t);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(fill_kernel, dim3(blocks), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace gk

namespace gk {
namespace {

// Batched 2-D transpose of activation-dtype matrices: for every tensor t,
// dst[t][c][r] = src[t][r][c]. One 64x64 tile per block, staged through LDS
// (+1 column of padding against bank conflicts; 16-element vector accesses
// for whole tiles, element by element at ragged edges); tiles of all tensors are
// numbered consecutively and a block finds its tensor by a binary search of
// the (few dozen) tile-start offsets (a linear scan, one dependent scalar load
// per tensor, had cost more than the block's own 16 KiB of traffic).
template <typename T>
__global__ __launch_bounds__(256) void transpose_batched_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                                const TransposeDesc* __restrict__ desc, int ndesc) {
  __shared__ float tile[64][65];
  int lo = 0, hi = ndesc;  // desc[lo].tile0 <= blockIdx.x < desc[hi].tile0 (desc[ndesc] past the end)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)blockIdx.x >= desc[mid].tile0) lo = mid;
    else hi = mid;
  }
  const int t = lo;
  const TransposeDesc d = desc[t];
  const int64_t local = blockIdx.x - d.tile0;
  const int tiles_c = (d.cols + 63) / 64;
  const int r0 = (int)(local / tiles_c) * 64, c0 = (int)(local % tiles_c) * 64;
  const T* s = src + d.offset;
  T* o = dst + d.offset;
  // whole tiles of 16-byte-aligned rows: each lane reads 16 consecutive
  // elements of one row and writes 16 consecutive elements of one output row
  // (element-wise accesses under per-element bounds tests had run at a
  // fraction of the HBM rate)
  const bool whole = r0 + 64 <= d.rows && c0 + 64 <= d.cols && d.rows % 16 == 0 && d.cols % 16 == 0 &&
                     (d.offset * (int64_t)sizeof(T)) % 16 == 0;
  if (whole) {  // uniform per block
    const int q = threadIdx.x & 3, rc = threadIdx.x >> 2;
    float v[2][8];
    const T* sp = s + (int64_t)(r0 + rc) * d.cols + c0 + q * 16;
    load8(sp, v[0]);
    load8(sp + 8, v[1]);
#pragma unroll
    for (int k = 0; k < 16; ++k) tile[rc][q * 16 + k] = v[k >> 3][k & 7];
    __syncthreads();
    // lane (rc, q) writes output row c0 + rc, columns r0 + 16q ..: for a fixed
    // k the 64 lanes read banks (16q + rc) mod 64 of the padded tile
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k >> 3][k & 7] = tile[q * 16 + k][rc];
    T* op = o + (int64_t)(c0 + rc) * d.rows + r0 + q * 16;
    store8(op, v[0]);
    store8(op + 8, v[1]);
    return;
  }
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i / 64, c = i % 64;
    if (r0 + r < d.rows && c0 + c < d.cols) tile[r][c] = to_f32(s[(int64_t)(r0 + r) * d.cols + c0 + c]);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int c = i / 64, r = i % 64;
    if (r0 + r < d.rows && c0 + c < d.cols) o[(int64_t)(c0 + c) * d.rows + r0 + r] = from_f32<T>(tile[r][c]);
  }
}

}  // namespace

hipError_t launch_transpose_batched(int dtype, const void* src, void* dst, const TransposeDesc* desc, int ndesc,
                                    int64_t total_tiles, hipStream_t s) {
  if (total_tiles <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(transpose_batched_kernel<bf16>, dim3((unsigned)total_tiles), dim3(256), 0, s,
                       (const bf16*)src, (bf16*)dst, desc, ndesc);
  else
    hipLaunchKernelGGL(transpose_batched_kernel<float>, dim3((unsigned)total_tiles), dim3(256), 0, s,
                       (const float*)src, (float*)dst, desc, ndesc);
  return hipGetLastError();
}

}  // namespace gk
