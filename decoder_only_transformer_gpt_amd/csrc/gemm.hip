// MFMA GEMM for gfx950 with fused epilogues.
//
// C[m, n] = sum_k A(m, k) * B(n, k). Each operand is either k-contiguous
// (row-major [rows, K]) or mn-contiguous (row-major [K, rows]); the three uses
// in the training step are
//   forward  y  = x  W^T   A = x  [M,K] k-contig,  B = W [N,K] k-contig
//   dX       dx = dy W     A = dy [M,N] k-contig,  B = W [N,K] mn-contig
//   dW       dW = dy^T x   A = dy [T,N] mn-contig, B = x [T,K] mn-contig
// (bias-free linears: atlas.blal.pro "nanochat — full-stack ChatGPT in ~8k
// lines", section "How it works", item 0).
//
// Block: 256 threads = 4 waves in a 2x2 grid; each wave owns a
// (BM/2) x (BN/2) sub-tile made of 32x32 MFMA blocks. K is staged through LDS
// in 128-byte rows (64 bf16 or 32 fp32) padded by 16 bytes, which makes the
// 16-byte fragment reads conflict-free. mn-contiguous operands are loaded as
// 8x8 (bf16) or 4x4 (fp32) blocks and transposed in registers before the LDS
// store, so the MFMA always reads k-contiguous fragments. The next K tile is
// prefetched into registers while the current one is consumed.
//
// The MFMA is issued with the B tile as its A operand, so each lane ends up
// holding 4 consecutive output columns of one output row: the epilogue writes
// 8- or 16-byte vectors and row-wise epilogue reductions stay inside a lane.

#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int kThreads = 256;

template <typename T>
struct TileK {
  static constexpr int V = Vec<T>::N;        // elements per 16 bytes
  static constexpr int BK = 128 / sizeof(T); // K elements per LDS row (128 B)
  static constexpr int LDK = BK + V;         // LDS row pitch (elements): +16 B
  static constexpr int KSTEP = 2 * V;        // k per fragment pair (2 lane groups)
};

// Loads a ROWS x BK tile (rows along m or n) into registers.
template <typename T, int ROWS, bool KCONTIG>
struct TileLoader {
  using TK = TileK<T>;
  static constexpr int V = TK::V;
  // k-contiguous: ROWS*8 vectors of 16 B; mn-contiguous: blocks of V x V.
  static constexpr int ITEMS = KCONTIG ? (ROWS * 8 / kThreads)
                                       : ((ROWS / V) * (TK::BK / V) + kThreads - 1) / kThreads;
  static constexpr int REGS = KCONTIG ? ITEMS : ITEMS * V;  // u32x4 registers
  u32x4 r[REGS > 0 ? REGS : 1];

  // base: element (row0, k0) of the operand; rows < rows_valid and
  // k < k_valid are real, the rest reads as zero (k-contiguous operands have
  // K a multiple of BK, so only their rows are checked).
  DEV void load(const T* __restrict__ base, int64_t ld, int rows_valid, int k_valid, int tid) {
    if constexpr (KCONTIG) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        int v = tid + i * kThreads;
        int row = v >> 3, kv = v & 7;
        if (row < rows_valid)
          r[i] = ld16(base + (int64_t)row * ld + kv * V);
        else
          r[i] = u32x4{0, 0, 0, 0};
      }
    } else {
      constexpr int KB = TK::BK / V;  // blocks along k (8)
      constexpr int NB = (ROWS / V) * KB;
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        int b = tid + i * kThreads;
        int kb = b % KB, rb = b / KB;
#pragma unroll
        for (int e = 0; e < V; ++e) {
          int k = kb * V + e;
          if (b < NB && k < k_valid && rb * V < rows_valid)
            r[i * V + e] = ld16(base + (int64_t)k * ld + rb * V);
          else
            r[i * V + e] = u32x4{0, 0, 0, 0};
        }
      }
    }
  }

  // Store to LDS tile [ROWS][LDK] (k contiguous).
  DEV void store(T* lds, int tid) {
    if constexpr (KCONTIG) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        int v = tid + i * kThreads;
        int row = v >> 3, kv = v & 7;
        st16(lds + row * TK::LDK + kv * V, r[i]);
      }
    } else {
      constexpr int KB = TK::BK / V;
      constexpr int NB = (ROWS / V) * KB;
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        int b = tid + i * kThreads;
        if (b >= NB) continue;
        int kb = b % KB, rb = b / KB;
        u32x4 out[V];
        transpose(&r[i * V], out);
#pragma unroll
        for (int j = 0; j < V; ++j) st16(lds + (rb * V + j) * TK::LDK + kb * V, out[j]);
      }
    }
  }

  // in[e] holds row k=e (V consecutive mn values); out[j] holds column mn=j.
  static DEV void transpose(const u32x4* in, u32x4* out) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint32_t lo = in[2 * d][j >> 1], hi = in[2 * d + 1][j >> 1];
          out[j][d] = __builtin_amdgcn_perm(hi, lo, (j & 1) ? 0x07060302u : 0x05040100u);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) out[j][e] = in[e][j];
    }
  }
};

template <typename T, Epi E>
struct Epilogue;

template <typename T, int BM, int BN, bool AK, bool BKc, Epi E>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs args) {
  using TK = TileK<T>;
  constexpr int V = TK::V, BK = TK::BK, LDK = TK::LDK;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(TM >= 1 && TN >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) T smem[(BM + BN) * LDK];
  T* As = smem;
  T* Bs = smem + BM * LDK;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 5, l32 = lane & 31;

  const int M = args.M, N = args.N, K = args.K;
  const int tiles_n = (N + BN - 1) / BN;
  int bid = blockIdx.x;
  const int nb = gridDim.x;
  // Spread consecutive tiles (which share an A row panel) over one XCD:
  // workgroups are dealt round-robin to the 8 XCDs.
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int mt = bid / tiles_n, nt = bid % tiles_n;
  const int m0 = mt * BM, n0 = nt * BN;

  // split-K range: slices of whole BK tiles; the last tile may be ragged
  // (only for mn-contiguous operands, whose k rows are bounds-checked)
  const int kper = ((K + args.splits - 1) / args.splits + BK - 1) / BK * BK;
  const int kbeg = blockIdx.z * kper;
  const int kend = min(K, kbeg + kper);
  const int nk = (kend > kbeg) ? (kend - kbeg + BK - 1) / BK : 0;

  const T* Ap = reinterpret_cast<const T*>(args.A);
  const T* Bp = reinterpret_cast<const T*>(args.B);

  TileLoader<T, BM, AK> la;
  TileLoader<T, BN, BKc> lb;

  auto a_base = [&](int k0) -> const T* {
    return AK ? Ap + (int64_t)m0 * args.lda + k0 : Ap + (int64_t)k0 * args.lda + m0;
  };
  auto b_base = [&](int k0) -> const T* {
    return BKc ? Bp + (int64_t)n0 * args.ldb + k0 : Bp + (int64_t)k0 * args.ldb + n0;
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  if (nk > 0) {
    la.load(a_base(kbeg), args.lda, M - m0, kend - kbeg, tid);
    lb.load(b_base(kbeg), args.ldb, N - n0, kend - kbeg, tid);
  }
  for (int kt = 0; kt < nk; ++kt) {
    la.store(As, tid);
    lb.store(Bs, tid);
    __syncthreads();
    if (kt + 1 < nk) {
      const int k0 = kbeg + (kt + 1) * BK;
      la.load(a_base(k0), args.lda, M - m0, kend - k0, tid);
      lb.load(b_base(k0), args.ldb, N - n0, kend - k0, tid);
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += TK::KSTEP) {
      u32x4 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = ld16(As + (wm * WM + i * 32 + l32) * LDK + kk + g * V);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = ld16(Bs + (wn * WN + j * 32 + l32) * LDK + kk + g * V);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(bfr[j], af[i], acc[i][j], (T*)nullptr);
    }
    __syncthreads();
  }

  Epilogue<T, E>::run(args, acc, m0 + wm * WM, n0 + wn * WN, l32, g);
}

// Walks the accumulators of one wave: row m = mbase + i*32 + l32 and
// columns n = nbase + j*32 + blk*8 + g*4 + {0..3}.
#define EPI_LOOP(BODY)                                                        \
  _Pragma("unroll") for (int i = 0; i < TM; ++i) {                            \
    const int m = mbase + i * 32 + l32;                                        \
    _Pragma("unroll") for (int j = 0; j < TN; ++j)                            \
    _Pragma("unroll") for (int blk = 0; blk < 4; ++blk) {                     \
      const int n = nbase + j * 32 + blk * 8 + g * 4;                          \
      float v[4] = {acc[i][j][blk * 4 + 0], acc[i][j][blk * 4 + 1],           \
                    acc[i][j][blk * 4 + 2], acc[i][j][blk * 4 + 3]};          \
      if (m < a.M && n < a.N) { BODY }                                         \
    }                                                                          \
  }

template <typename T>
struct Epilogue<T, Epi::Store> {
  template <int TM, int TN>
  static DEV void run(const GemmArgs& a, f32x16 (&acc)[TM][TN], int mbase, int nbase, int l32, int g) {
    T* C = reinterpret_cast<T*>(a.C);
    EPI_LOOP(store4(C + (int64_t)m * a.ldc + n, v);)
  }
};

template <typename T>
struct Epilogue<T, Epi::Residual> {
  template <int TM, int TN>
  static DEV void run(const GemmArgs& a, f32x16 (&acc)[TM][TN], int mbase, int nbase, int l32, int g) {
    T* C = reinterpret_cast<T*>(a.C);
    EPI_LOOP({
      float x[4];
      load4(C + (int64_t)m * a.ldc + n, x);
      for (int r = 0; r < 4; ++r) x[r] += v[r];
      store4(C + (int64_t)m * a.ldc + n, x);
    })
  }
};

// relu^2 MLP activation (aethryn.com, section "A Llama-class transformer with
// ten modern departures"): stores u and a = max(u, 0)^2.
template <typename T>
struct Epilogue<T, Epi::Relu2> {
  template <int TM, int TN>
  static DEV void run(const GemmArgs& a, f32x16 (&acc)[TM][TN], int mbase, int nbase, int l32, int g) {
    T* U = reinterpret_cast<T*>(a.C);
    T* A2 = reinterpret_cast<T*>(a.C2);
    EPI_LOOP({
      float s[4];
      for (int r = 0; r < 4; ++r) { float p = fmaxf(v[r], 0.f); s[r] = p * p; }
      store4(U + (int64_t)m * a.ldc + n, v);
      store4(A2 + (int64_t)m * a.ldc2 + n, s);
    })
  }
};

// du = da * 2 max(u, 0)
template <typename T>
struct Epilogue<T, Epi::Relu2Bwd> {
  template <int TM, int TN>
  static DEV void run(const GemmArgs& a, f32x16 (&acc)[TM][TN], int mbase, int nbase, int l32, int g) {
    T* D = reinterpret_cast<T*>(a.C);
    const T* U = reinterpret_cast<const T*>(a.C2);
    EPI_LOOP({
      float u[4];
      load4(U + (int64_t)m * a.ldc2 + n, u);
      for (int r = 0; r < 4; ++r) v[r] *= 2.f * fmaxf(u[r], 0.f);
      store4(D + (int64_t)m * a.ldc + n, v);
    })
  }
};

// LM head with the logit softcap c*tanh(z/c), evaluated on the fp32
// accumulator (aethryn.com, section "A Llama-class transformer with ten modern
// departures": softcap 15, in float32). Emits the capped logits in the
// activation dtype, one fp32 partial sum of exp(z' - c) per row and 128
// columns (terms lie in (e^-2c, 1], so partial sums add without rescaling),
// and the fp32 capped logit at the row's target.
template <typename T>
struct Epilogue<T, Epi::LMHead> {
  template <int TM, int TN>
  static DEV void run(const GemmArgs& a, f32x16 (&acc)[TM][TN], int mbase, int nbase, int l32, int g) {
    static_assert(TN * 32 == kLMHeadPartCols, "one partial per wave column");
    T* Z = reinterpret_cast<T*>(a.C);
    const float c = a.softcap, inv_c = 1.f / a.softcap;
    const int nparts = a.N / kLMHeadPartCols;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = mbase + i * 32 + l32;
      const bool mv = m < a.M;
      const int tgt = mv ? a.targets[m] : -1;
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          const int n = nbase + j * 32 + blk * 8 + g * 4;
          float z[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            z[r] = c * tanhf(acc[i][j][blk * 4 + r] * inv_c);
            s += __expf(z[r] - c);
          }
          if (mv) {
            store4(Z + (int64_t)m * a.ldc + n, z);
            const unsigned d = (unsigned)(tgt - n);
            if (d < 4u) a.ztgt[m] = z[d];
          }
        }
      s += __shfl_xor(s, 32, 64);
      if (mv && g == 0) a.part[(int64_t)m * nparts + nbase / kLMHeadPartCols] = s;
    }
  }
};

template <typename T>
struct Epilogue<T, Epi::GradF32> {
  template <int TM, int TN>
  static DEV void run(const GemmArgs& a, f32x16 (&acc)[TM][TN], int mbase, int nbase, int l32, int g) {
    if (a.splits > 1) {
      float* P = a.split_buf + (int64_t)blockIdx.z * a.M * a.N;
      EPI_LOOP(store4(P + (int64_t)m * a.N + n, v);)
    } else {
      float* G = reinterpret_cast<float*>(a.C);
      const bool accum = a.accumulate != 0;
      EPI_LOOP({
        float* p = G + (int64_t)m * a.ldc + n;
        if (accum) {
          float x[4];
          load4(p, x);
          for (int r = 0; r < 4; ++r) v[r] += x[r];
        }
        store4(p, v);
      })
    }
  }
};

// Sums split-K partials in slice order into the fp32 gradient.
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ P, int splits, int M, int N,
                                                     float* __restrict__ G, int64_t ldg, int accumulate) {
  const int64_t total4 = (int64_t)M * N / 4;
  for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < total4;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = q * 4;
    const int m = (int)(e / N), n = (int)(e % N);
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < splits; ++z) {
      float x[4];
      load4(P + (int64_t)z * M * N + e, x);
      for (int r = 0; r < 4; ++r) s[r] += x[r];
    }
    float* gp = G + (int64_t)m * ldg + n;
    if (accumulate) {
      float x[4];
      load4(gp, x);
      for (int r = 0; r < 4; ++r) s[r] += x[r];
    }
    store4(gp, s);
  }
}

template <typename T, int BM, int BN, bool AK, bool BKc, Epi E>
hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  const int splits = (E == Epi::GradF32) ? a.splits : 1;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, AK, BKc, E>), dim3(tiles, 1, splits), dim3(kThreads), 0, s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || E != Epi::GradF32 || a.splits <= 1) return err;
  const int64_t total4 = (int64_t)a.M * a.N / 4;
  const int blocks = (int)std::min<int64_t>((total4 + 255) / 256, 4096);
  hipLaunchKernelGGL(splitk_reduce, dim3(blocks), dim3(256), 0, s, a.split_buf, a.splits, a.M, a.N,
                     reinterpret_cast<float*>(a.C), a.ldc, a.accumulate);
  return hipGetLastError();
}

// Tile size: the largest that still gives at least ~1 tile per CU.
template <typename T, bool AK, bool BKc, Epi E>
hipError_t launch_layout(const GemmArgs& a, hipStream_t s) {
  if constexpr (E == Epi::LMHead) {
    // one 128-column partial per wave column => BN = 256
    if ((int64_t)((a.M + 255) / 256) * (a.N / 256) >= 256) return launch_tile<T, 256, 256, AK, BKc, E>(a, s);
    return launch_tile<T, 64, 256, AK, BKc, E>(a, s);
  } else {
    const int64_t t256 = (int64_t)((a.M + 255) / 256) * ((a.N + 255) / 256) * a.splits;
    const int64_t t128 = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128) * a.splits;
    if (t256 >= 512 && a.N % 256 == 0) return launch_tile<T, 256, 256, AK, BKc, E>(a, s);
    if (t128 >= 256 || a.N % 64 != 0) return launch_tile<T, 128, 128, AK, BKc, E>(a, s);
    return launch_tile<T, 64, 64, AK, BKc, E>(a, s);
  }
}

template <typename T>
hipError_t launch_typed(Epi epi, const GemmArgs& a, hipStream_t s) {
  const bool nt = a.a_kcontig && a.b_kcontig, nn = a.a_kcontig && !a.b_kcontig,
             tn = !a.a_kcontig && !a.b_kcontig;
  switch (epi) {
    case Epi::Store:
      if (nt) return launch_layout<T, true, true, Epi::Store>(a, s);
      if (nn) return launch_layout<T, true, false, Epi::Store>(a, s);
      break;
    case Epi::Residual:
      if (nt) return launch_layout<T, true, true, Epi::Residual>(a, s);
      break;
    case Epi::Relu2:
      if (nt) return launch_layout<T, true, true, Epi::Relu2>(a, s);
      break;
    case Epi::LMHead:
      if (nt) return launch_layout<T, true, true, Epi::LMHead>(a, s);
      break;
    case Epi::Relu2Bwd:
      if (nn) return launch_layout<T, true, false, Epi::Relu2Bwd>(a, s);
      break;
    case Epi::GradF32:
      if (tn) return launch_layout<T, false, false, Epi::GradF32>(a, s);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int dtype, Epi epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  // Shapes the tile loaders assume: a k-contiguous operand has K a multiple of
  // the 128-byte K tile; an mn-contiguous operand has its rows in whole
  // 16-byte vectors; the epilogue writes groups of 4 columns.
  const int bk = dtype == 1 ? 64 : 32;
  if ((a.a_kcontig || a.b_kcontig) && a.K % bk != 0) return hipErrorInvalidValue;
  if ((!a.a_kcontig && a.M % 8 != 0) || (!a.b_kcontig && a.N % 8 != 0) || a.N % 4 != 0) return hipErrorInvalidValue;
  if (epi == Epi::LMHead && a.N % 256 != 0) return hipErrorInvalidValue;
  if (a.splits < 1 || (a.splits > 1 && a.split_buf == nullptr)) return hipErrorInvalidValue;
  return dtype == 1 ? launch_typed<bf16>(epi, a, s) : launch_typed<float>(epi, a, s);
}

}  // namespace gk
