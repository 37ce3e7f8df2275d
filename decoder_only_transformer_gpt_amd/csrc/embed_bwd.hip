// Embedding backward: dwte[v] += sum over positions n with idx[n] == v of the
// gradient of x0[n] = rmsnorm(wte[idx[n]]) (the post-embedding RMSNorm of
// aethryn.com "Nanochat: full-stack LLM training in 8,000 lines for $72",
// section "A Llama-class transformer with ten modern departures").
//
// With y = wte[v] * r_n the norm backward is r_n * dres_n - wte[v] * k_n where
// k_n = r_n^3 / C * <dres_n, wte[v]>, so
//   dwte[v] += sum_n r_n * dres_n  -  wte[v] * sum_n k_n:
// one pass over the gradient rows accumulates one C-vector and, per lane, the
// k terms of each id (the embedding row travels with every gradient row), and
// one wave reduction per id (or per part of an id's run) gives the k sum.
//
// Token ids follow a skewed (Zipf-like) law, so a scatter with float atomics
// would serialise on the frequent rows and make the result depend on timing.
// Instead: (1) a stable LSD radix sort of the ids (2 passes of 8 bits,
// V <= 65536) carrying the token index; (2) one wave per chunk of 32 sorted
// entries sums each run of equal ids over whole rows, finishing runs that
// lie inside the chunk and leaving a partial row plus its k sum for the two
// runs that cross the chunk's edges; (3) one block per (chunk where a crossing
// run starts, 512 columns) adds those partials (four waves over contiguous
// quarters of the run's chunks, then the quarters in order). Every sum has a
// fixed order, so the result is bitwise reproducible.

#include <type_traits>

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

// Block-wide inclusive scan of one int per thread (256 threads).
DEV int block_scan256(int v, int* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {  // Hillis-Steele
    const int u = threadIdx.x >= o ? sh[threadIdx.x - o] : 0;
    __syncthreads();
    sh[threadIdx.x] += u;
    __syncthreads();
  }
  return sh[threadIdx.x];
}

// One block per digit d: exclusive scan of the digit's per-chunk counts
// hist[d * nchunks + c] in place, and the digit's total count.
__global__ __launch_bounds__(256) void digit_scan_kernel(int32_t* __restrict__ hist, int nchunks,
                                                         int32_t* __restrict__ total) {
  __shared__ int sh[256];
  int32_t* h = hist + (int64_t)blockIdx.x * nchunks;
  const int per = (nchunks + 255) / 256;
  const int beg = min(nchunks, (int)threadIdx.x * per), end = min(nchunks, beg + per);
  int s = 0;
  for (int i = beg; i < end; ++i) s += h[i];
  const int incl = block_scan256(s, sh);
  int run = incl - s;
  for (int i = beg; i < end; ++i) {
    const int v = h[i];
    h[i] = run;
    run += v;
  }
  if (threadIdx.x == 255) total[blockIdx.x] = incl;
}

// Stable scatter: position = start of the digit (exclusive scan of the digit
// totals) + the chunk's offset within the digit + the rank within the chunk
// among equal digits (earlier equal items).
__global__ __launch_bounds__(kSortChunk) void radix_scatter_kernel(const int32_t* __restrict__ kin,
                                                                   const int32_t* __restrict__ vin, int N, int shift,
                                                                   int nchunks, const int32_t* __restrict__ hist,
                                                                   const int32_t* __restrict__ total,
                                                                   int32_t* __restrict__ kout,
                                                                   int32_t* __restrict__ vout) {
  static_assert(kSortChunk == 256, "one thread per digit");
  __shared__ int dig[kSortChunk];
  __shared__ int base[256];
  {
    const int t = total[threadIdx.x];
    const int incl = block_scan256(t, base);
    __syncthreads();
    base[threadIdx.x] = incl - t;
  }
  const int i = blockIdx.x * kSortChunk + threadIdx.x;
  const bool valid = i < N;
  const int key = valid ? kin[i] : 0;
  const int d = valid ? (key >> shift) & 255 : -1;
  dig[threadIdx.x] = d;
  __syncthreads();
  if (!valid) return;
  int rank = 0;
  for (int j = 0; j < (int)threadIdx.x; ++j) rank += (dig[j] == d);
  const int pos = base[d] + hist[d * nchunks + blockIdx.x] + rank;
  kout[pos] = key;
  vout[pos] = vin[i];
}

// 8 consecutive values of an embedding row, kept raw while the load is in
// flight and widened to fp32 when used.
template <typename T>
struct Raw8;
template <>
struct Raw8<bf16> {
  u32x4 r;
  DEV void load(const bf16* p) { r = ld16(p); }
  DEV void get(float (&v)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r[i] << 16);
      v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
  }
};
template <>
struct Raw8<float> {
  u32x4 a, b;
  DEV void load(const float* p) {
    a = ld16(p);
    b = ld16(p + 4);
  }
  DEV void get(float (&v)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a[i]);
      v[4 + i] = __uint_as_float(b[i]);
    }
  }
};

// One wave per chunk of kSegChunk sorted entries; lane l holds columns
// j * 512 + 8l .. +8 of every row (J = ceil(C / 512) groups). For each run of
// equal ids in the chunk the wave accumulates a1 = sum r_n dres_n and, per
// lane, the run's part of ks = sum_n (r_n^3 / C) <dres_n, wte[v]>. The
// gradient rows and embedding rows of the next R - 1 entries are in flight
// while the current one is added (rings of R row buffers, the loop unrolled
// by R so every slot is a fixed register set; the embedding row is requested
// for every entry so that no load is conditional, repeats of an id hitting
// the cache). At a run's end ks is a wave reduction; a run that starts and
// ends inside the chunk adds a1 - wte[v] * ks to dwte[v] (stores it when the
// backward overwrites: dwte was zeroed first); a run cut by the chunk's first
// (last) edge stores a1 and ks in carry slot 0 (1) of the chunk instead
// (slots of C + 8 floats: the row, then ks).
template <typename T, typename DR, int J, int R, bool ACC>
__global__ __launch_bounds__(256) void embed_seg_kernel(const int32_t* __restrict__ keys,
                                                        const int32_t* __restrict__ vals,
                                                        const DR* __restrict__ dres,
                                                        const float* __restrict__ rstd0, const T* __restrict__ wte,
                                                        int N, int C, float* __restrict__ dwte,
                                                        float* __restrict__ carry) {
  static_assert(kSegChunk <= 64, "one entry per lane");
  static_assert(R >= 2 && R <= 4, "one to three rows in flight");
  const int lane = threadIdx.x & 63;
  // wave-uniform (scalar) chunk index, so the entry loop and its tests are scalar
  const int c = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int nseg = (N + kSegChunk - 1) / kSegChunk;
  if (c >= nseg) return;
  const int e0 = c * kSegChunk, e1 = min(N, e0 + kSegChunk), ne = e1 - e0;
  // the chunk's entries, one per lane, and the ids just outside it
  const int me = e0 + (lane < ne ? lane : 0);
  const int key_l = keys[me];
  const int val_l = vals[me];
  const float r_l = rstd0[val_l >= 0 ? val_l : 0];  // unused for an invalid id
  const int prev_key = e0 > 0 ? keys[e0 - 1] : -1;
  const int next_key = e1 < N ? keys[e1] : -1;
  // retire these loads on every path, so the entry loop's reads of them need
  // no wait (otherwise its header, reachable before any row request, waits
  // for every load in flight)
  wait_vmcnt<0>();
  const float invC = 1.f / (float)C;
  int col[J], colc[J];
  bool cv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    col[j] = j * 512 + lane * 8;
    cv[j] = col[j] < C;
    colc[j] = cv[j] ? col[j] : C - 8;
  }
  float a1[J][8], rows[R][J][8], dk = 0.f;
  Raw8<T> wring[R][J];
  auto key_at = [&](int e) { return __builtin_amdgcn_readlane(key_l, e); };
  // entry f's gradient row and embedding row into slot u (lanes past the row
  // re-read its last 8 columns, so every load is unconditional and the
  // compiler's waits count exactly the loads issued since)
  auto request = [&](int f, int u) __attribute__((always_inline)) {
    const int n = __builtin_amdgcn_readlane(val_l, f);
    const DR* row = dres + (int64_t)(n < 0 ? 0 : n) * C;
    const T* w = wte + (int64_t)key_at(f) * C;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      load8(row + colc[j], rows[u][j]);
      wring[u][j].load(w + colc[j]);
    }
  };
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int q = 0; q < 8; ++q) a1[j][q] = 0.f;
  // requests past the chunk's last entry repeat that entry: every path then
  // issues the same loads, and the compiler's waits stay exact
#pragma unroll
  for (int u = 0; u + 1 < R; ++u) request(min(u, ne - 1), u);
  int rs = 0;  // run start (entry index within the chunk)
  // entry e sits in slot u = e % R; entry e + R - 1 goes to slot (u + R - 1) % R
  auto step = [&](int e, auto slot) __attribute__((always_inline)) {
    constexpr int u = decltype(slot)::value;
    const int v = key_at(e);
    const int n = __builtin_amdgcn_readlane(val_l, e);
    const float r = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r_l), e));
    request(min(e + R - 1, ne - 1), (u + R - 1) % R);
    float w[J][8];
#pragma unroll
    for (int j = 0; j < J; ++j) wring[u][j].get(w[j]);
    if (n >= 0) {  // an invalid id (the forward raised the device flag) adds nothing
      const float r3 = r * r * r * invC;
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float dj = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          a1[j][q] = fmaf(r, rows[u][j][q], a1[j][q]);
          dj = fmaf(rows[u][j][q], w[j][q], dj);
        }
        d += cv[j] ? dj : 0.f;
      }
      dk = fmaf(r3, d, dk);
    }
    const int vn = e + 1 < ne ? key_at(e + 1) : next_key;
    if (vn != v || e + 1 == ne) {
      // end of a run inside this chunk (it may continue in the next chunk)
      const bool starts_here = rs > 0 || prev_key != v;
      const bool ends_here = vn != v;
      const float ks = wave_sum(dk);
      if (starts_here && ends_here) {
        float* drow = dwte + (int64_t)v * C;
#pragma unroll
        for (int j = 0; j < J; ++j)
          if (cv[j]) {
            float o[8];
            if constexpr (ACC) load8(drow + col[j], o);
#pragma unroll
            for (int q = 0; q < 8; ++q) o[q] = (ACC ? o[q] : 0.f) + a1[j][q] - w[j][q] * ks;
            store8(drow + col[j], o);
          }
      } else {
        float* slot = carry + ((int64_t)c * 2 + (starts_here ? 1 : 0)) * (C + 8);
#pragma unroll
        for (int j = 0; j < J; ++j)
          if (cv[j]) store8(slot + col[j], a1[j]);
        if (lane == 0) slot[C] = ks;
      }
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int q = 0; q < 8; ++q) a1[j][q] = 0.f;
      dk = 0.f;
      rs = e + 1;
    }
  };
  for (int e = 0; e < ne; e += R) {
    step(e, std::integral_constant<int, 0>{});
    if (e + 1 < ne) step(e + 1, std::integral_constant<int, 1 % R>{});
    if constexpr (R > 2) if (e + 2 < ne) step(e + 2, std::integral_constant<int, 2 % R>{});
    if constexpr (R > 3) if (e + 3 < ne) step(e + 3, std::integral_constant<int, 3 % R>{});
  }
}

// Last chunk that a run of id v reaches, for a run that begins in chunk c and
// goes on past it (keys ascending, so the run's chunks are those whose first
// entry holds v). The wave's lanes probe the first entries of chunks S apart
// (lane 0 at a chunk known to start inside the run); the first probe outside
// bounds the run, and one more round probes the S chunks before it: two
// rounds of loads per 63 S chunks of run, where a binary search over the
// entries takes one dependent load per halving.
DEV int run_last_chunk(const int32_t* __restrict__ keys, int nchunks, int c, int v, int lane) {
  constexpr int S = 16;
  int in = c + 1;  // starts inside the run: the run goes on past chunk c
  for (;;) {
    const int p = in + lane * S;
    const uint64_t out = __ballot(p >= nchunks || keys[p * kSegChunk] != v);
    if (out == 0) {  // every probe inside: lane 63's chunk starts inside
      in += 63 * S;
      continue;
    }
    const int lo = in + (__builtin_ctzll(out) - 1) * S;  // inside; lo + S is outside or past the end
    const int q = lo + lane;
    const uint64_t out2 = __ballot(lane >= S || q >= nchunks || keys[q * kSegChunk] != v);
    return lo + __builtin_ctzll(out2) - 1;  // out2 has a bit at or below S, and none at 0
  }
}

// One block of four waves per (chunk in which a boundary-crossing run starts,
// 512 columns): adds that run's partial rows (slot 1 of its first chunk and
// slot 0 of every later chunk it reaches) and their k sums, and adds
// a1 - wte[v] * ks to dwte[v]. The chunk holding the run's last entry is found
// by probing chunk starts across the wave's lanes; each wave sums a contiguous
// quarter of the slot-0 range (eight rows in flight per lane), and wave 0 adds
// slot 1 and the quarters in order, so the frequent ids' long runs are summed
// by four waves in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void seg_fixup_kernel(const int32_t* __restrict__ keys, int N, int C, int nchunks,
                                                        const T* __restrict__ wte, const float* __restrict__ carry,
                                                        float* __restrict__ dwte) {
  __shared__ float part[4][512];
  __shared__ float kpart[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int ngrp = (C + 511) / 512;
  const int c = blockIdx.x / ngrp, grp = blockIdx.x % ngrp;
  if (c >= nchunks) return;
  const int e0 = c * kSegChunk, e1 = min(N, e0 + kSegChunk);
  const int last = e1 - 1;
  if (e1 >= N) return;                      // nothing continues past the end
  const int v = keys[last];
  if (keys[e1] != v) return;                // last run does not continue
  // did the run start inside this chunk?
  if (keys[e0] == v && e0 > 0 && keys[e0 - 1] == v) return;  // began earlier: owned by an earlier chunk
  const int cend = run_last_chunk(keys, nchunks, c, v, lane);
  const int n = cend - c;  // slot-0 partials: chunks c+1 .. cend
  const int q0 = c + 1 + (int)((int64_t)n * wave / 4), q1 = c + 1 + (int)((int64_t)n * (wave + 1) / 4);
  // this wave's k sums: lane-strided partial sums combined by a fixed butterfly
  float ks = 0.f;
  for (int cc = q0 + lane; cc < q1; cc += 64) ks += carry[((int64_t)cc * 2 + 0) * (C + 8) + C];
  ks = wave_sum(ks);
  const int col = grp * 512 + lane * 8;
  const bool valid = col < C;
  const int colc = valid ? col : C - 8;  // lanes past the row re-read its last 8 columns
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  int cc = q0;
  for (; cc + 7 < q1; cc += 8) {
    float x[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) load8(carry + ((int64_t)(cc + u) * 2 + 0) * (C + 8) + colc, x[u]);
    // all eight rows requested before the first add (left to itself the
    // scheduler interleaves each load with its add, two or three in flight)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += x[u][q];
  }
  for (; cc < q1; ++cc) {
    float x[8];
    load8(carry + ((int64_t)cc * 2 + 0) * (C + 8) + colc, x);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += x[q];
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) part[wave][lane * 8 + q] = acc[q];
  if (lane == 0) kpart[wave] = ks;
  __syncthreads();
  if (wave != 0 || !valid) return;
  float tot[8];
  load8(carry + ((int64_t)c * 2 + 1) * (C + 8) + col, tot);
  float kt = carry[((int64_t)c * 2 + 1) * (C + 8) + C];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
#pragma unroll
    for (int q = 0; q < 8; ++q) tot[q] += part[w][lane * 8 + q];
    kt += kpart[w];
  }
  float wv[8], o[8];
  load8(wte + (int64_t)v * C + col, wv);
  float* drow = dwte + (int64_t)v * C + col;
  load8(drow, o);
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] += tot[q] - wv[q] * kt;
  store8(drow, o);
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
  const int cend = run_last_chunk(keys, nchunks, c, v, col & 63);
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
    int32_t* total = hist + (size_t)256 * nchunks;
    hipLaunchKernelGGL(radix_hist_kernel, dim3(nchunks), dim3(kSortChunk), 0, s, kin, N, shift, nchunks, hist);
    hipLaunchKernelGGL(digit_scan_kernel, dim3(256), dim3(256), 0, s, hist, nchunks, total);
    hipLaunchKernelGGL(radix_scatter_kernel, dim3(nchunks), dim3(kSortChunk), 0, s, kin, vin, N, shift, nchunks, hist,
                       total, kout, vout);
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

// per-chunk digit counts, then the 256 digit totals
size_t embed_bwd_hist_elems(int N) { return (size_t)256 * ((N + kSortChunk - 1) / kSortChunk) + 256; }
// two partial-row slots of C + 8 floats per chunk of sorted entries (the
// value-embedding sums use slots of 129 floats in the same buffer)
size_t embed_bwd_carry_elems(int N, int C) {
  return (size_t)2 * ((N + kSegChunk - 1) / kSegChunk) * (size_t)(C + 8 > 129 ? C + 8 : 129);
}

template <typename T, int J>
hipError_t embed_seg(const EmbedBwdArgs& a, int nseg, hipStream_t s) {
  // rows in flight per wave: about J * ((8 + 4 or 8) R + 16) registers must
  // stay within ~220 (two waves per SIMD)
  constexpr int per = sizeof(T) == 2 ? 12 : 16;
  constexpr int R = (220 / J - 16) / per >= 4 ? 4 : (220 / J - 16) / per >= 3 ? 3 : 2;
  const dim3 grid((nseg + 3) / 4);
  if (a.dres) {  // fp32 gradient rows
    if (a.accumulate)
      hipLaunchKernelGGL((embed_seg_kernel<T, float, J, R, true>), grid, dim3(256), 0, s, a.keys_a, a.vals_a, a.dres,
                         a.rstd0, (const T*)a.wte, a.N, a.C, a.dwte, a.carry);
    else
      hipLaunchKernelGGL((embed_seg_kernel<T, float, J, R, false>), grid, dim3(256), 0, s, a.keys_a, a.vals_a, a.dres,
                         a.rstd0, (const T*)a.wte, a.N, a.C, a.dwte, a.carry);
  } else {  // gradient rows in the activation dtype
    if (a.accumulate)
      hipLaunchKernelGGL((embed_seg_kernel<T, T, J, R, true>), grid, dim3(256), 0, s, a.keys_a, a.vals_a,
                         (const T*)a.dres_lp, a.rstd0, (const T*)a.wte, a.N, a.C, a.dwte, a.carry);
    else
      hipLaunchKernelGGL((embed_seg_kernel<T, T, J, R, false>), grid, dim3(256), 0, s, a.keys_a, a.vals_a,
                         (const T*)a.dres_lp, a.rstd0, (const T*)a.wte, a.N, a.C, a.dwte, a.carry);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t embed_seg_j(const EmbedBwdArgs& a, int nseg, hipStream_t s) {
  switch ((a.C + 511) / 512) {
    case 1: return embed_seg<T, 1>(a, nseg, s);
    case 2: return embed_seg<T, 2>(a, nseg, s);
    case 3: return embed_seg<T, 3>(a, nseg, s);
    case 4: return embed_seg<T, 4>(a, nseg, s);
    case 5: return embed_seg<T, 5>(a, nseg, s);
    case 6: return embed_seg<T, 6>(a, nseg, s);
    case 7: return embed_seg<T, 7>(a, nseg, s);
    case 8: return embed_seg<T, 8>(a, nseg, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_embed_bwd(const EmbedBwdArgs& a, hipStream_t s) {
  const int N = a.N, C = a.C;
  if (C % 8 != 0 || C > 4096 || (!a.dres && !a.dres_lp)) return hipErrorInvalidValue;
  hipError_t e;
  if (!a.accumulate && !a.dwte_zeroed) {
    if ((e = launch_fill_f32(a.dwte, 0.f, (int64_t)a.V * C, s)) != hipSuccess) return e;
  }
  if (N <= 0) return hipSuccess;
  // the ids were sorted by launch_embed_sort into keys_a / vals_a
  const int nseg = (N + kSegChunk - 1) / kSegChunk;
  e = a.dtype == 1 ? embed_seg_j<bf16>(a, nseg, s) : embed_seg_j<float>(a, nseg, s);
  if (e != hipSuccess) return e;
  const int items = nseg * ((C + 511) / 512);  // one block per (chunk, 512 columns)
  if (a.dtype == 1)
    hipLaunchKernelGGL(seg_fixup_kernel<bf16>, dim3(items), dim3(256), 0, s, a.keys_a, N, C, nseg,
                       (const bf16*)a.wte, a.carry, a.dwte);
  else
    hipLaunchKernelGGL(seg_fixup_kernel<float>, dim3(items), dim3(256), 0, s, a.keys_a, N, C, nseg,
                       (const float*)a.wte, a.carry, a.dwte);
  return hipGetLastError();
}

}  // namespace gk
