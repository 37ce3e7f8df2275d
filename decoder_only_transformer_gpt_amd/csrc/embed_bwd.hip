// Embedding backward: dwte[v] += sum over positions n with idx[n] == v of the
// gradient of x0[n] = rmsnorm(wte[idx[n]]) (the post-embedding RMSNorm of
// aethryn.com "Nanochat: full-stack LLM training in 8,000 lines for $72",
// section "A Llama-class transformer with ten modern departures").
//
// With y = wte[v] * r_n the norm backward is r_n * dres_n - wte[v] * k_n where
// k_n = r_n^3 / C * <dres_n, wte[v]>, so
//   dwte[v] += sum_n r_n * dres_n  -  wte[v] * sum_n k_n.
//
// Token ids follow a skewed (Zipf-like) law, so a scatter with float atomics
// would serialise on the frequent rows and make the result depend on timing.
// Instead: (1) per-token k_n, (2) a stable LSD radix sort of the ids
// (2 passes of 8 bits, V <= 65536) carrying the token index, (3) segment sums
// over fixed chunks of the sorted list, where runs that cross a chunk boundary
// leave partial rows that (4) one block per crossing segment adds up in chunk
// order. Every sum has a fixed order, so the result is bitwise reproducible.

#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int kSortChunk = 256;  // items per block in the radix passes
constexpr int kSegChunk = 32;    // sorted entries per block in the segment sums

// Sort input: key = token id, value = position (negative for an invalid id,
// which the segment sums skip).
__global__ __launch_bounds__(256) void sort_init_kernel(const int32_t* __restrict__ idx, int N, int V,
                                                        int32_t* __restrict__ keys, int32_t* __restrict__ vals) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int id = idx[n];
  const bool ok = (unsigned)id < (unsigned)V;
  keys[n] = ok ? id : 0;
  vals[n] = ok ? n : -1 - n;
}

template <typename T>
__global__ __launch_bounds__(256) void embed_coef_kernel(const T* __restrict__ wte, const int32_t* __restrict__ idx,
                                                         const float* __restrict__ dres,
                                                         const float* __restrict__ rstd0, int N, int C, int V,
                                                         float* __restrict__ coef) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int id = idx[n];
  const bool ok = (unsigned)id < (unsigned)V;
  const T* w = wte + (int64_t)(ok ? id : 0) * C;
  const float* g = dres + (int64_t)n * C;
  float dot = 0.f;
  for (int ch = lane; ch < (C >> 3); ch += 64) {
    float a[8], b[8];
    load8(w + ch * 8, a);
    load8(g + ch * 8, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) dot += a[e] * b[e];
  }
  dot = wave_sum(dot);
  if (lane == 0) {
    const float r = rstd0[n];
    // An invalid id (the forward already raised the device flag) contributes nothing.
    coef[n] = ok ? r * r * r * dot / (float)C : 0.f;
  }
}

// Per-chunk digit histogram, stored digit-major: hist[d * nchunks + chunk].
__global__ __launch_bounds__(kSortChunk) void radix_hist_kernel(const int32_t* __restrict__ keys, int N, int shift,
                                                                int nchunks, int32_t* __restrict__ hist) {
  __shared__ int cnt[256];
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int i = blockIdx.x * kSortChunk + threadIdx.x;
  if (i < N) atomicAdd(&cnt[(keys[i] >> shift) & 255], 1);
  __syncthreads();
  hist[threadIdx.x * nchunks + blockIdx.x] = cnt[threadIdx.x];
}

// Exclusive scan of n ints in place, one block of 1024 threads.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ a, int n) {
  __shared__ int part[1024];
  const int per = (n + 1023) / 1024;
  const int beg = min(n, threadIdx.x * per), end = min(n, beg + per);
  int s = 0;
  for (int i = beg; i < end; ++i) s += a[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // Hillis-Steele inclusive scan
    int v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = threadIdx.x ? part[threadIdx.x - 1] : 0;
  for (int i = beg; i < end; ++i) {
    const int v = a[i];
    a[i] = run;
    run += v;
  }
}

// Stable scatter: rank within the chunk among equal digits = earlier equal items.
__global__ __launch_bounds__(kSortChunk) void radix_scatter_kernel(const int32_t* __restrict__ kin,
                                                                   const int32_t* __restrict__ vin, int N, int shift,
                                                                   int nchunks, const int32_t* __restrict__ hist,
                                                                   int32_t* __restrict__ kout,
                                                                   int32_t* __restrict__ vout) {
  __shared__ int dig[kSortChunk];
  const int i = blockIdx.x * kSortChunk + threadIdx.x;
  const bool valid = i < N;
  const int key = valid ? kin[i] : 0;
  const int d = valid ? (key >> shift) & 255 : -1;
  dig[threadIdx.x] = d;
  __syncthreads();
  if (!valid) return;
  int rank = 0;
  for (int j = 0; j < (int)threadIdx.x; ++j) rank += (dig[j] == d);
  const int pos = hist[d * nchunks + blockIdx.x] + rank;
  kout[pos] = key;
  vout[pos] = vin[i];
}

// Segment sums over chunks of kSegChunk sorted entries. Complete runs are
// added to dwte directly; a run cut by a chunk boundary leaves a partial row
// (C values + the k sum) in carry slot 0 (run began before this chunk) or 1
// (run begins in this chunk and continues after it).
__global__ __launch_bounds__(256) void seg_partial_kernel(const int32_t* __restrict__ keys,
                                                          const int32_t* __restrict__ vals,
                                                          const float* __restrict__ dres,
                                                          const float* __restrict__ rstd0,
                                                          const float* __restrict__ coef, const void* wte_raw,
                                                          int wte_bf16, int N, int C, float* __restrict__ dwte,
                                                          float* __restrict__ carry) {
  const int c = blockIdx.x;
  const int e0 = c * kSegChunk, e1 = min(N, e0 + kSegChunk);
  for (int col0 = 0; col0 < C; col0 += 256) {
    const int col = col0 + threadIdx.x;
    const bool cv = col < C;
    float acc = 0.f, ks = 0.f;
    int rs = e0;  // run start
    for (int e = e0; e < e1; ++e) {
      const int v = keys[e];
      const int n = vals[e];
      if (n >= 0) {
        if (cv) acc += rstd0[n] * dres[(int64_t)n * C + col];
        ks += coef[n];
      }
      const bool run_end = (e + 1 == e1) || keys[e + 1] != v;
      if (!run_end) continue;
      const bool seg_start = (rs == 0) || keys[rs - 1] != v;
      const bool seg_end = (e + 1 == N) || keys[e + 1] != v;
      if (seg_start && seg_end) {
        if (cv) {
          const float w = wte_bf16 ? (float)((const bf16*)wte_raw)[(int64_t)v * C + col]
                                   : ((const float*)wte_raw)[(int64_t)v * C + col];
          dwte[(int64_t)v * C + col] += acc - w * ks;
        }
      } else {
        float* slot = carry + ((int64_t)c * 2 + (seg_start ? 1 : 0)) * (C + 1);
        if (cv) slot[col] = acc;
        if (threadIdx.x == 0) slot[C] = ks;
      }
      acc = 0.f;
      ks = 0.f;
      rs = e + 1;
    }
  }
}

// Last sorted position holding id v, searching from position `from` (whose
// key is v): a binary search over the ascending keys.
DEV int segment_last(const int32_t* __restrict__ keys, int N, int from, int v) {
  int lo = from, hi = N;  // keys[lo] == v; keys[hi] != v (or hi == N)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (keys[mid] == v) lo = mid;
    else hi = mid;
  }
  return lo;
}

// One block per chunk in which a boundary-crossing segment starts: adds the
// partials of that segment in chunk order and finalises its row. The chunk
// holding the segment's last entry is found first (binary search), so the
// partial rows are summed over a known range with many loads in flight.
__global__ __launch_bounds__(256) void seg_fixup_kernel(const int32_t* __restrict__ keys, int N, int C, int nchunks,
                                                        const void* wte_raw, int wte_bf16,
                                                        const float* __restrict__ carry, float* __restrict__ dwte) {
  const int c = blockIdx.x;
  const int e0 = c * kSegChunk, e1 = min(N, e0 + kSegChunk);
  const int last = e1 - 1;
  if (e1 >= N) return;                      // nothing continues past the end
  const int v = keys[last];
  if (keys[e1] != v) return;                // last run does not continue
  // did the segment start inside this chunk?
  int s = last;
  while (s > e0 && keys[s - 1] == v) --s;
  if (s == e0 && e0 > 0 && keys[e0 - 1] == v) return;  // began earlier: owned by an earlier chunk
  const int cend = min(nchunks - 1, segment_last(keys, N, e1, v) / kSegChunk);
  // column C of a partial row carries the k sum
  __shared__ float ks_sh;
  if (threadIdx.x == 0) {
    float ks = carry[((int64_t)c * 2 + 1) * (C + 1) + C];
#pragma unroll 8
    for (int cc = c + 1; cc <= cend; ++cc) ks += carry[((int64_t)cc * 2 + 0) * (C + 1) + C];
    ks_sh = ks;
  }
  __syncthreads();
  const float ks = ks_sh;
  for (int col = threadIdx.x; col < C; col += 256) {
    float acc = carry[((int64_t)c * 2 + 1) * (C + 1) + col];
#pragma unroll 8
    for (int cc = c + 1; cc <= cend; ++cc) acc += carry[((int64_t)cc * 2 + 0) * (C + 1) + col];
    const float w = wte_bf16 ? (float)((const bf16*)wte_raw)[(int64_t)v * C + col]
                             : ((const float*)wte_raw)[(int64_t)v * C + col];
    dwte[(int64_t)v * C + col] += acc - w * ks;
  }
}

// Value-embedding gradient: dve[v] += gate * sum over positions n with
// idx[n] == v of dv[n] (128 values, at column col0 of a row of pitch ld), by
// the same chunked segment sums over the sorted ids; one thread per column.
template <typename T>
__global__ __launch_bounds__(128) void ve_seg_partial_kernel(const int32_t* __restrict__ keys,
                                                             const int32_t* __restrict__ vals,
                                                             const T* __restrict__ src, int64_t ld, int col0,
                                                             const T* __restrict__ gate, int N,
                                                             float* __restrict__ dve, float* __restrict__ carry) {
  const int c = blockIdx.x, col = threadIdx.x;
  const int e0 = c * kSegChunk, e1 = min(N, e0 + kSegChunk);
  const float g = to_f32(*gate);
  float acc = 0.f;
  int rs = e0;
  for (int e = e0; e < e1; ++e) {
    const int v = keys[e];
    const int n = vals[e];
    if (n >= 0) acc += to_f32(src[(int64_t)n * ld + col0 + col]);
    const bool run_end = (e + 1 == e1) || keys[e + 1] != v;
    if (!run_end) continue;
    const bool seg_start = (rs == 0) || keys[rs - 1] != v;
    const bool seg_end = (e + 1 == N) || keys[e + 1] != v;
    if (seg_start && seg_end) dve[(int64_t)v * 128 + col] += g * acc;
    else carry[((int64_t)c * 2 + (seg_start ? 1 : 0)) * 129 + col] = acc;
    acc = 0.f;
    rs = e + 1;
  }
}

template <typename T>
__global__ __launch_bounds__(128) void ve_seg_fixup_kernel(const int32_t* __restrict__ keys, int N, int nchunks,
                                                           const T* __restrict__ gate,
                                                           const float* __restrict__ carry, float* __restrict__ dve) {
  const int c = blockIdx.x, col = threadIdx.x;
  const int e0 = c * kSegChunk, e1 = min(N, e0 + kSegChunk);
  const int last = e1 - 1;
  if (e1 >= N) return;
  const int v = keys[last];
  if (keys[e1] != v) return;
  int s = last;
  while (s > e0 && keys[s - 1] == v) --s;
  if (s == e0 && e0 > 0 && keys[e0 - 1] == v) return;
  const int cend = min(nchunks - 1, segment_last(keys, N, e1, v) / kSegChunk);
  float acc = carry[((int64_t)c * 2 + 1) * 129 + col];
#pragma unroll 8
  for (int cc = c + 1; cc <= cend; ++cc) acc += carry[((int64_t)cc * 2 + 0) * 129 + col];
  dve[(int64_t)v * 128 + col] += to_f32(*gate) * acc;
}

}  // namespace

hipError_t launch_embed_sort(const int32_t* idx, int N, int V, int32_t* keys_a, int32_t* vals_a, int32_t* keys_b,
                             int32_t* vals_b, int32_t* hist, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(sort_init_kernel, dim3((N + 255) / 256), dim3(256), 0, s, idx, N, V, keys_a, vals_a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nchunks = (N + kSortChunk - 1) / kSortChunk;
  int32_t *kin = keys_a, *vin = vals_a, *kout = keys_b, *vout = vals_b;
  for (int shift = 0; shift < 16; shift += 8) {
    hipLaunchKernelGGL(radix_hist_kernel, dim3(nchunks), dim3(kSortChunk), 0, s, kin, N, shift, nchunks, hist);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, hist, 256 * nchunks);
    hipLaunchKernelGGL(radix_scatter_kernel, dim3(nchunks), dim3(kSortChunk), 0, s, kin, vin, N, shift, nchunks, hist,
                       kout, vout);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    std::swap(kin, kout);
    std::swap(vin, vout);
  }
  return hipSuccess;  // two passes: the sorted ids are back in keys_a / vals_a
}

hipError_t launch_ve_scatter(int dtype, const int32_t* keys, const int32_t* vals, const void* dqkv, int64_t ld,
                             int col0, const void* gate, int N, int V, int accumulate, float* dve, float* carry,
                             hipStream_t s) {
  hipError_t e;
  if (!accumulate && (e = launch_fill_f32(dve, 0.f, (int64_t)V * 128, s)) != hipSuccess) return e;
  if (N <= 0) return hipSuccess;
  const int nseg = (N + kSegChunk - 1) / kSegChunk;
  if (dtype == 1) {
    hipLaunchKernelGGL(ve_seg_partial_kernel<bf16>, dim3(nseg), dim3(128), 0, s, keys, vals, (const bf16*)dqkv, ld,
                       col0, (const bf16*)gate, N, dve, carry);
    hipLaunchKernelGGL(ve_seg_fixup_kernel<bf16>, dim3(nseg), dim3(128), 0, s, keys, N, nseg, (const bf16*)gate,
                       (const float*)carry, dve);
  } else {
    hipLaunchKernelGGL(ve_seg_partial_kernel<float>, dim3(nseg), dim3(128), 0, s, keys, vals, (const float*)dqkv, ld,
                       col0, (const float*)gate, N, dve, carry);
    hipLaunchKernelGGL(ve_seg_fixup_kernel<float>, dim3(nseg), dim3(128), 0, s, keys, N, nseg, (const float*)gate,
                       (const float*)carry, dve);
  }
  return hipGetLastError();
}

size_t embed_bwd_hist_elems(int N) { return (size_t)256 * ((N + kSortChunk - 1) / kSortChunk); }
size_t embed_bwd_carry_elems(int N, int C) { return (size_t)2 * ((N + kSegChunk - 1) / kSegChunk) * (C + 1); }

hipError_t launch_embed_bwd(const EmbedBwdArgs& a, hipStream_t s) {
  const int N = a.N, C = a.C;
  hipError_t e;
  if (!a.accumulate) {
    if ((e = launch_fill_f32(a.dwte, 0.f, (int64_t)a.V * C, s)) != hipSuccess) return e;
  }
  if (N <= 0) return hipSuccess;
  if (a.dtype == 1)
    hipLaunchKernelGGL(embed_coef_kernel<bf16>, dim3((N + 3) / 4), dim3(256), 0, s, (const bf16*)a.wte, a.idx,
                       a.dres, a.rstd0, N, C, a.V, a.coef);
  else
    hipLaunchKernelGGL(embed_coef_kernel<float>, dim3((N + 3) / 4), dim3(256), 0, s, (const float*)a.wte, a.idx,
                       a.dres, a.rstd0, N, C, a.V, a.coef);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // the ids were sorted by launch_embed_sort into keys_a / vals_a
  const int32_t* kin = a.keys_a;
  const int32_t* vin = a.vals_a;
  const int nseg = (N + kSegChunk - 1) / kSegChunk;
  hipLaunchKernelGGL(seg_partial_kernel, dim3(nseg), dim3(256), 0, s, kin, vin, a.dres, a.rstd0, a.coef, a.wte,
                     a.dtype == 1, N, C, a.dwte, a.carry);
  hipLaunchKernelGGL(seg_fixup_kernel, dim3(nseg), dim3(256), 0, s, kin, N, C, nseg, a.wte, a.dtype == 1, a.carry,
                     a.dwte);
  return hipGetLastError();
}

}  // namespace gk
