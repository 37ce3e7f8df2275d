// Causal multi-query flash attention, head_dim 128, forward and backward.
//
// Every query head shares the single K/V head (energyai.berlin "nanochat vs
// GPT-OSS", section "Architectural decisions", subsection MQA); q and k arrive
// RoPE-rotated and RMS-normalised per head (aethryn.com "Nanochat: full-stack
// LLM training in 8,000 lines for $72", section "A Llama-class transformer
// with ten modern departures": QK normalization after RoPE). Scores are
// s = q.k / sqrt(D) with key u <= query t.
//
// Fixed-shift softmax: with RMS-normalised q and k, |q.k| <= |q||k| = D, so
// |s| <= sqrt(D) ~ 11.31 and exp(s - sqrt(D)) lies in [e^-22.7, ~1]. The row
// sum therefore accumulates without a running maximum or rescaling, and
// lse = sqrt(D) + log(sum) is exact up to rounding. (This relies on QK-norm.)
//
// All contractions run on MFMA 32x32 tiles. The kernels put the output
// dimension that must be reduced over on the accumulator's lane axis, e.g.
// the forward computes S^T = K Q^T so each lane owns one query and its
// softmax row sum stays inside the lane. When an operand held in registers
// (P, dS) feeds the next MFMA, the k index of that MFMA is permuted to match
// the accumulator layout; the LDS operand is read with the same permutation
// (any fixed k order gives the same sum).
//
// qkv row (one token): [H query heads | K | V] x 128. LSE and delta are fp32
// [B, H, T]. Grid blocks are ordered heavy-first for causal load balance.

#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int D = 128;
constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
struct AT {
  static constexpr int V = Vec<T>::N;     // elements per 16 B
  static constexpr int KS = 2 * V;        // k per fragment step
  static constexpr int NDS = D / KS;      // fragment steps over D
  static constexpr int P = D + V;         // pitch of [rows][D] tiles
  static constexpr int PT = 64 + V;       // pitch of [D][64] tiles
};

// rows x 128 tile, rows contiguous in global (pitch ld), to LDS [rows][P].
template <typename T, int ROWS>
DEV void tile_rows(T* lds, const T* src, int64_t ld, int rows_valid, int tid) {
  constexpr int V = AT<T>::V, CPR = D / V;  // 16-byte chunks per row
  constexpr int ITEMS = ROWS * CPR / 256;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int q = tid + i * 256;
    const int r = q / CPR, c = q % CPR;
    u32x4 v = {0, 0, 0, 0};
    if (r < rows_valid) v = ld16(src + (int64_t)r * ld + c * V);
    st16(lds + r * AT<T>::P + c * V, v);
  }
}

// rows x 128 tile to LDS transposed: [128][PT] with the row index contiguous.
// Loaded as V x V blocks and transposed in registers.
template <typename T, int ROWS>
DEV void tile_T(T* lds, const T* src, int64_t ld, int rows_valid, int tid) {
  constexpr int V = AT<T>::V;
  constexpr int RB = ROWS / V, CB = D / V, NB = RB * CB;
  constexpr int ITEMS = (NB + 255) / 256;
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int b = tid + i * 256;
    if (b >= NB) break;
    const int rb = b % RB, cb = b / RB;
    u32x4 in[V], out[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int r = rb * V + e;
      in[e] = (r < rows_valid) ? ld16(src + (int64_t)r * ld + cb * V) : u32x4{0, 0, 0, 0};
    }
    if constexpr (V == 8) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int d = 0; d < 4; ++d)
          out[j][d] = __builtin_amdgcn_perm(in[2 * d + 1][j >> 1], in[2 * d][j >> 1],
                                            (j & 1) ? 0x07060302u : 0x05040100u);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) out[j][e] = in[e][j];
    }
#pragma unroll
    for (int j = 0; j < V; ++j) st16(lds + (cb * V + j) * AT<T>::PT + rb * V, out[j]);
  }
}

// Packs accumulator values of 32x32 block `acc` into the register operand of
// the next MFMA for k-step kk: element e is the value at accumulator row
// blk*8 + g*4 + r with blk = kk*(V/4) + e/4, r = e%4.
template <typename T>
DEV u32x4 pack_frag(const f32x16& acc, int kk) {
  constexpr int V = AT<T>::V;
  u32x4 f;
  if constexpr (V == 8) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int e = 2 * d;
      const int i0 = (kk * 2 + e / 4) * 4 + e % 4;
      f[d] = pack_bf16x2(acc[i0], acc[i0 + 1]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __float_as_uint(acc[kk * 4 + e]);
  }
  return f;
}

// Reads the matching LDS operand: row `row` of a [.][PT] tile, k positions
// base + (kk*(V/4) + e/4)*8 + g*4 + e%4.
template <typename T>
DEV u32x4 read_perm(const T* lds, int row, int base, int kk, int g) {
  constexpr int V = AT<T>::V;
  const T* p = lds + row * AT<T>::PT + base + g * 4;
  if constexpr (V == 8) {
    u32x2 a = ld8(p + (kk * 2) * 8), b = ld8(p + (kk * 2 + 1) * 8);
    return u32x4{a[0], a[1], b[0], b[1]};
  } else {
    return ld16(p + kk * 8);
  }
}

DEV f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ------------------------------------------------------------- forward --
// Block: 128 queries of one (batch, head) = 4 waves x 32. KV tiles of 64 keys.
template <typename T>
__global__ __launch_bounds__(256) void attn_fwd_kernel(const T* __restrict__ qkv, int T_, int H, T* __restrict__ o,
                                                       float* __restrict__ lse) {
  using A = AT<T>;
  constexpr int V = A::V;
  __shared__ __attribute__((aligned(16))) T Ks[64 * A::P];
  __shared__ __attribute__((aligned(16))) T VTs[D * A::PT];
  const int nqb = (T_ + 127) / 128;
  const int qb = nqb - 1 - blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int64_t ld = (int64_t)(H + 2) * D;
  const T* base = qkv + (int64_t)b * T_ * ld;
  const int q = qb * 128 + w * 32 + l32;

  u32x4 qf[A::NDS];
#pragma unroll
  for (int ks = 0; ks < A::NDS; ++ks)
    qf[ks] = (q < T_) ? ld16(base + (int64_t)q * ld + h * D + ks * A::KS + g * V) : u32x4{0, 0, 0, 0};

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = zero16();
  float rsum = 0.f;
  const float shift = sqrtf((float)D);
  const float sl2 = kLog2e / shift, sh2 = shift * kLog2e;
  const int kend = min(T_, qb * 128 + 128);

  for (int k0 = 0; k0 < kend; k0 += 64) {
    tile_rows<T, 64>(Ks, base + (int64_t)k0 * ld + H * D, ld, T_ - k0, tid);
    tile_T<T, 64>(VTs, base + (int64_t)k0 * ld + (H + 1) * D, ld, T_ - k0, tid);
    __syncthreads();
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero16();
#pragma unroll
      for (int ks = 0; ks < A::NDS; ++ks)
        s[kb] = mfma16(ld16(Ks + (kb * 32 + l32) * A::P + ks * A::KS + g * V), qf[ks], s[kb], (T*)nullptr);
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + kb * 32 + blk * 8 + g * 4 + r;
          const float p = (key <= q && key < T_) ? exp2f(s[kb][blk * 4 + r] * sl2 - sh2) : 0.f;
          s[kb][blk * 4 + r] = p;
          rsum += p;
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kk = 0; kk < 32 / A::KS; ++kk) {
        const u32x4 pf = pack_frag<T>(s[kb], kk);
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = mfma16(read_perm<T>(VTs, db * 32 + l32, kb * 32, kk, g), pf, acc[db], (T*)nullptr);
      }
    __syncthreads();
  }
  rsum += __shfl_xor(rsum, 32, 64);
  if (q < T_) {
    const float inv = 1.f / rsum;
    T* op = o + ((int64_t)b * T_ + q) * H * D + h * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        float v[4] = {acc[db][blk * 4] * inv, acc[db][blk * 4 + 1] * inv, acc[db][blk * 4 + 2] * inv,
                      acc[db][blk * 4 + 3] * inv};
        store4(op + db * 32 + blk * 8 + g * 4, v);
      }
    if (g == 0) lse[((int64_t)b * H + h) * T_ + q] = shift + logf(rsum);
  }
}

// ------------------------------------------------------------- backward --

// delta[b, h, t] = sum_d dO * O (the softmax-Jacobian row term).
template <typename T>
__global__ __launch_bounds__(256) void attn_delta_kernel(const T* __restrict__ o, const T* __restrict__ dout, int N,
                                                         int T_, int H, float* __restrict__ delta) {
  const int grp = (blockIdx.x * 256 + threadIdx.x) >> 4;  // (token, head)
  const int j = threadIdx.x & 15;
  if (grp >= N * H) return;
  const int n = grp / H, h = grp % H;
  const int64_t off = (int64_t)n * H * D + h * D + j * 8;
  float a[8], c[8];
  load8(o + off, a);
  load8(dout + off, c);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += a[e] * c[e];
#pragma unroll
  for (int m = 8; m > 0; m >>= 1) s += __shfl_xor(s, m, 16);
  if (j == 0) {
    const int b = n / T_, t = n % T_;
    delta[((int64_t)b * H + h) * T_ + t] = s;
  }
}

// dQ: block = 128 queries of one (batch, head); loops over KV tiles.
template <typename T>
__global__ __launch_bounds__(256) void attn_dq_kernel(const T* __restrict__ qkv, const T* __restrict__ dout,
                                                      const float* __restrict__ lse, const float* __restrict__ delta,
                                                      int T_, int H, T* __restrict__ dqkv) {
  using A = AT<T>;
  constexpr int V = A::V;
  __shared__ __attribute__((aligned(16))) T Ks[64 * A::P];
  __shared__ __attribute__((aligned(16))) T Vs[64 * A::P];
  __shared__ __attribute__((aligned(16))) T KTs[D * A::PT];
  const int nqb = (T_ + 127) / 128;
  const int qb = nqb - 1 - blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int64_t ld = (int64_t)(H + 2) * D;
  const T* base = qkv + (int64_t)b * T_ * ld;
  const int q = qb * 128 + w * 32 + l32;
  const bool qv = q < T_;

  u32x4 qf[A::NDS], df[A::NDS];
  const T* dop = dout + ((int64_t)b * T_ + q) * H * D + h * D;
#pragma unroll
  for (int ks = 0; ks < A::NDS; ++ks) {
    qf[ks] = qv ? ld16(base + (int64_t)q * ld + h * D + ks * A::KS + g * V) : u32x4{0, 0, 0, 0};
    df[ks] = qv ? ld16(dop + ks * A::KS + g * V) : u32x4{0, 0, 0, 0};
  }
  const float lq = qv ? lse[((int64_t)b * H + h) * T_ + q] : 0.f;
  const float dq_ = qv ? delta[((int64_t)b * H + h) * T_ + q] : 0.f;
  const float scale = rsqrtf((float)D);
  const float sl2 = kLog2e * scale, l2 = lq * kLog2e;

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = zero16();
  const int kend = min(T_, qb * 128 + 128);
  for (int k0 = 0; k0 < kend; k0 += 64) {
    const T* kp = base + (int64_t)k0 * ld + H * D;
    tile_rows<T, 64>(Ks, kp, ld, T_ - k0, tid);
    tile_rows<T, 64>(Vs, kp + D, ld, T_ - k0, tid);
    tile_T<T, 64>(KTs, kp, ld, T_ - k0, tid);
    __syncthreads();
    f32x16 ds[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < A::NDS; ++ks) {
        s = mfma16(ld16(Ks + (kb * 32 + l32) * A::P + ks * A::KS + g * V), qf[ks], s, (T*)nullptr);
        dp = mfma16(ld16(Vs + (kb * 32 + l32) * A::P + ks * A::KS + g * V), df[ks], dp, (T*)nullptr);
      }
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + kb * 32 + blk * 8 + g * 4 + r;
          const int i = blk * 4 + r;
          const float p = (key <= q && key < T_) ? exp2f(s[i] * sl2 - l2) : 0.f;
          ds[kb][i] = p * (dp[i] - dq_);
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kk = 0; kk < 32 / A::KS; ++kk) {
        const u32x4 pf = pack_frag<T>(ds[kb], kk);
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = mfma16(read_perm<T>(KTs, db * 32 + l32, kb * 32, kk, g), pf, acc[db], (T*)nullptr);
      }
    __syncthreads();
  }
  if (qv) {
    T* outp = dqkv + ((int64_t)b * T_ + q) * ld + h * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        float v[4] = {acc[db][blk * 4] * scale, acc[db][blk * 4 + 1] * scale, acc[db][blk * 4 + 2] * scale,
                      acc[db][blk * 4 + 3] * scale};
        store4(outp + db * 32 + blk * 8 + g * 4, v);
      }
  }
}

// dK, dV: block = 128 keys of one batch row (4 waves x 32 keys), summed over
// every query head and every query tile at or after the keys (no atomics).
template <typename T>
__global__ __launch_bounds__(256) void attn_dkv_kernel(const T* __restrict__ qkv, const T* __restrict__ dout,
                                                       const float* __restrict__ lse,
                                                       const float* __restrict__ delta, int T_, int H,
                                                       T* __restrict__ dqkv) {
  using A = AT<T>;
  constexpr int V = A::V;
  __shared__ __attribute__((aligned(16))) T Qs[64 * A::P];
  __shared__ __attribute__((aligned(16))) T QTs[D * A::PT];
  __shared__ __attribute__((aligned(16))) T Ds[64 * A::P];
  __shared__ __attribute__((aligned(16))) T DTs[D * A::PT];
  __shared__ float Ls[64], Es[64];
  const int kb = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int64_t ld = (int64_t)(H + 2) * D;
  const T* base = qkv + (int64_t)b * T_ * ld;
  const int key = kb * 128 + w * 32 + l32;
  const bool kv = key < T_;

  u32x4 kf[A::NDS], vf[A::NDS];
#pragma unroll
  for (int ks = 0; ks < A::NDS; ++ks) {
    kf[ks] = kv ? ld16(base + (int64_t)key * ld + H * D + ks * A::KS + g * V) : u32x4{0, 0, 0, 0};
    vf[ks] = kv ? ld16(base + (int64_t)key * ld + (H + 1) * D + ks * A::KS + g * V) : u32x4{0, 0, 0, 0};
  }
  const float scale = rsqrtf((float)D);
  const float sl2 = kLog2e * scale;
  f32x16 adk[4], adv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { adk[i] = zero16(); adv[i] = zero16(); }

  for (int h = 0; h < H; ++h) {
    const float* lh = lse + ((int64_t)b * H + h) * T_;
    const float* eh = delta + ((int64_t)b * H + h) * T_;
    for (int q0 = kb * 128; q0 < T_; q0 += 64) {
      const T* qp = base + (int64_t)q0 * ld + h * D;
      const T* dp_ = dout + ((int64_t)b * T_ + q0) * H * D + h * D;
      tile_rows<T, 64>(Qs, qp, ld, T_ - q0, tid);
      tile_T<T, 64>(QTs, qp, ld, T_ - q0, tid);
      tile_rows<T, 64>(Ds, dp_, (int64_t)H * D, T_ - q0, tid);
      tile_T<T, 64>(DTs, dp_, (int64_t)H * D, T_ - q0, tid);
      if (tid < 64) {
        const bool v = q0 + tid < T_;
        Ls[tid] = v ? lh[q0 + tid] : 0.f;
        Es[tid] = v ? eh[q0 + tid] : 0.f;
      }
      __syncthreads();
      f32x16 p[2], ds[2];
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2) {
        f32x16 s = zero16(), dpv = zero16();
#pragma unroll
        for (int ks = 0; ks < A::NDS; ++ks) {
          s = mfma16(ld16(Qs + (qb2 * 32 + l32) * A::P + ks * A::KS + g * V), kf[ks], s, (T*)nullptr);
          dpv = mfma16(ld16(Ds + (qb2 * 32 + l32) * A::P + ks * A::KS + g * V), vf[ks], dpv, (T*)nullptr);
        }
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int qi = qb2 * 32 + blk * 8 + g * 4 + r;
            const int qq = q0 + qi;
            const int i = blk * 4 + r;
            const float pv = (qq >= key && qq < T_ && kv) ? exp2f(s[i] * sl2 - Ls[qi] * kLog2e) : 0.f;
            p[qb2][i] = pv;
            ds[qb2][i] = pv * (dpv[i] - Es[qi]);
          }
      }
#pragma unroll
      for (int qb2 = 0; qb2 < 2; ++qb2)
#pragma unroll
        for (int kk = 0; kk < 32 / A::KS; ++kk) {
          const u32x4 pf = pack_frag<T>(p[qb2], kk);
          const u32x4 sf = pack_frag<T>(ds[qb2], kk);
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            adv[db] = mfma16(read_perm<T>(DTs, db * 32 + l32, qb2 * 32, kk, g), pf, adv[db], (T*)nullptr);
            adk[db] = mfma16(read_perm<T>(QTs, db * 32 + l32, qb2 * 32, kk, g), sf, adk[db], (T*)nullptr);
          }
        }
      __syncthreads();
    }
  }
  if (kv) {
    T* outk = dqkv + ((int64_t)b * T_ + key) * ld + H * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int d = db * 32 + blk * 8 + g * 4;
        float vk[4] = {adk[db][blk * 4] * scale, adk[db][blk * 4 + 1] * scale, adk[db][blk * 4 + 2] * scale,
                       adk[db][blk * 4 + 3] * scale};
        float vv[4] = {adv[db][blk * 4], adv[db][blk * 4 + 1], adv[db][blk * 4 + 2], adv[db][blk * 4 + 3]};
        store4(outk + d, vk);
        store4(outk + D + d, vv);
      }
  }
}

template <typename T>
hipError_t fwd_typed(const void* qkv, int B, int T_, int H, void* o, float* lse, hipStream_t s) {
  dim3 grid((T_ + 127) / 128, H, B);
  hipLaunchKernelGGL(attn_fwd_kernel<T>, grid, dim3(256), 0, s, (const T*)qkv, T_, H, (T*)o, lse);
  return hipGetLastError();
}

template <typename T>
hipError_t bwd_typed(const void* qkv, const void* o, const void* dout, const float* lse, int B, int T_, int H,
                     float* delta, void* dqkv, hipStream_t s) {
  const int64_t groups = (int64_t)B * T_ * H;
  hipLaunchKernelGGL(attn_delta_kernel<T>, dim3((unsigned)((groups * 16 + 255) / 256)), dim3(256), 0, s,
                     (const T*)o, (const T*)dout, B * T_, T_, H, delta);
  hipLaunchKernelGGL(attn_dq_kernel<T>, dim3((T_ + 127) / 128, H, B), dim3(256), 0, s, (const T*)qkv,
                     (const T*)dout, lse, delta, T_, H, (T*)dqkv);
  hipLaunchKernelGGL(attn_dkv_kernel<T>, dim3((T_ + 127) / 128, B), dim3(256), 0, s, (const T*)qkv, (const T*)dout,
                     lse, delta, T_, H, (T*)dqkv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(int dtype, const void* qkv, int B, int T, int H, void* o, float* lse, hipStream_t s) {
  return dtype == 1 ? fwd_typed<bf16>(qkv, B, T, H, o, lse, s) : fwd_typed<float>(qkv, B, T, H, o, lse, s);
}

hipError_t launch_attn_bwd(int dtype, const void* qkv, const void* o, const void* dout, const float* lse, int B,
                           int T, int H, float* delta, void* dqkv, hipStream_t s) {
  return dtype == 1 ? bwd_typed<bf16>(qkv, o, dout, lse, B, T, H, delta, dqkv, s)
                    : bwd_typed<float>(qkv, o, dout, lse, B, T, H, delta, dqkv, s);
}

}  // namespace gk
