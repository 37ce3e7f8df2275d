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

#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gk {
namespace {

constexpr int kThreads = 256;
constexpr int kGroupM = 4;  // row panels per tile group (NT kernel)

// Blocks are dealt round-robin to the 8 XCDs (block b runs on XCD b mod 8).
// Map block b to an item index so that each XCD takes one contiguous run of
// items: XCD x's j-th block gets item start(x) + j, the runs sized by how
// many blocks each XCD receives (any grid size; a bijection on [0, nb)).
DEV int xcd_contiguous(int b, int nb) {
  const int x = b & 7, j = b >> 3, q = nb >> 3, r = nb & 7;
  return x * q + (x < r ? x : r) + j;
}

template <typename T>
struct TileK {
  static constexpr int V = Vec<T>::N;        // elements per 16 bytes
  static constexpr int BK = 128 / sizeof(T); // K elements per LDS row (128 B)
  static constexpr int LDK = BK + V;         // LDS row pitch (elements): +16 B
  static constexpr int KSTEP = 2 * V;        // k per fragment pair (2 lane groups)
};

// Loads a ROWS x BK tile (rows along m or n) into registers with buffer
// loads. Per-lane byte offsets inside the tile are computed once; each K tile
// gets a fresh buffer resource (SGPRs) whose base points at the tile and
// whose record count ends at the last valid row, so rows past M and k past
// the end of a ragged split read as zero in hardware: no per-load address
// arithmetic and no selects in the loop.
template <typename T, int ROWS, bool KCONTIG>
struct TileLoader {
  using TK = TileK<T>;
  static constexpr int V = TK::V;
  // k-contiguous: ROWS*8 vectors of 16 B; mn-contiguous: blocks of V x V.
  static constexpr int ITEMS = KCONTIG ? (ROWS * 8 / kThreads)
                                       : ((ROWS / V) * (TK::BK / V) + kThreads - 1) / kThreads;
  static constexpr int REGS = KCONTIG ? ITEMS : ITEMS * V;  // u32x4 registers
  static constexpr uint32_t kOOB = 0x7ffffff0u;             // beyond any record count used
  // 16-byte LDS stores per thread per tile
  static constexpr int NSTORE = KCONTIG ? ITEMS
                                        : ((ROWS / V) * (TK::BK / V) >= kThreads ? ITEMS * V : V);
  using Regs = u32x4[REGS];
  uint32_t voff[REGS];

  DEV void init(int64_t ld, int tid) {
    const uint32_t ldb = (uint32_t)(ld * (int64_t)sizeof(T));
    if constexpr (KCONTIG) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int v = tid + i * kThreads;
        voff[i] = (uint32_t)(v >> 3) * ldb + (uint32_t)(v & 7) * 16u;
      }
    } else {
      constexpr int KB = TK::BK / V, NB = (ROWS / V) * KB;
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int b = tid + i * kThreads;
        const int kb = b % KB, rb = b / KB;
#pragma unroll
        for (int e = 0; e < V; ++e)
          voff[i * V + e] = (b < NB) ? (uint32_t)(kb * V + e) * ldb + (uint32_t)rb * 16u : kOOB;
      }
    }
  }

  // Resource for the tile whose element (row 0, k 0) is at `base`: for a
  // k-contiguous operand rows < rows_valid are real; for an mn-contiguous one
  // k < k_valid are real.
  static DEV __amdgpu_buffer_rsrc_t rsrc(const T* base, int64_t ld, int rows_valid, int k_valid) {
    int64_t n = KCONTIG ? (int64_t)rows_valid * ld * (int64_t)sizeof(T) - 0
                        : (int64_t)min(k_valid, TK::BK) * ld * (int64_t)sizeof(T);
    n = n < 0 ? 0 : (n > (1 << 30) ? (1 << 30) : n);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0, (int)n, 0x00020000);
  }

  DEV void load(Regs& r, __amdgpu_buffer_rsrc_t rs) const {
#pragma unroll
    for (int q = 0; q < REGS; ++q) r[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[q], 0, 0);
  }

  // Store to LDS tile [ROWS][LDK] (k contiguous).
  static DEV void store(const Regs& r, T* lds, int tid) {
    if constexpr (KCONTIG) {
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int v = tid + i * kThreads;
        st16(lds + (v >> 3) * TK::LDK + (v & 7) * V, r[i]);
      }
    } else {
      constexpr int KB = TK::BK / V;
      constexpr int NB = (ROWS / V) * KB;
#pragma unroll
      for (int i = 0; i < ITEMS; ++i) {
        const int b = tid + i * kThreads;
        if (NB % kThreads != 0 && b >= NB) continue;
        const int kb = b % KB, rb = b / KB;
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

  // Two LDS stages: tile kt is consumed from stage kt&1 while tile kt+1 is
  // written to the other stage; one barrier per K tile.
  __shared__ __attribute__((aligned(16))) T smem[2][(BM + BN) * LDK];

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

  using LA = TileLoader<T, BM, AK>;
  using LB = TileLoader<T, BN, BKc>;
  LA la;
  LB lb;
  la.init(args.lda, tid);
  lb.init(args.ldb, tid);
  // element (row 0, k 0) of K tile kt for each operand, and its resource
  auto rs_a = [&](int kt) {
    const int k0 = kbeg + kt * BK;
    const T* p = AK ? Ap + (int64_t)m0 * args.lda + k0 : Ap + (int64_t)k0 * args.lda + m0;
    return LA::rsrc(p, args.lda, M - m0, kend - k0);
  };
  auto rs_b = [&](int kt) {
    const int k0 = kbeg + kt * BK;
    const T* p = BKc ? Bp + (int64_t)n0 * args.ldb + k0 : Bp + (int64_t)k0 * args.ldb + n0;
    return LB::rsrc(p, args.ldb, N - n0, kend - k0);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Global prefetch runs two K tiles ahead in two register sets: tile t is
  // loaded into set t&1 two iterations before it is consumed and stored to
  // LDS stage t&1 one iteration before. Past the end the prefetch re-reads
  // the last tile and the store hits the idle stage (uniform, branch-free
  // body). The loop is unrolled by two so the register set is static.
  typename LA::Regs ra0, ra1;
  typename LB::Regs rb0, rb1;
  if (nk > 0) {
    la.load(ra0, rs_a(0));
    lb.load(rb0, rs_b(0));
    la.load(ra1, rs_a(min(1, nk - 1)));
    lb.load(rb1, rs_b(min(1, nk - 1)));
    LA::store(ra0, smem[0], tid);
    LB::store(rb0, smem[0] + BM * LDK, tid);
    la.load(ra0, rs_a(min(2, nk - 1)));
    lb.load(rb0, rs_b(min(2, nk - 1)));
  }
  __syncthreads();

  constexpr int KSTEPS = BK / TK::KSTEP;
  auto step = [&](int kt, typename LA::Regs& ran, typename LB::Regs& rbn) {
    const T* As = smem[kt & 1];
    const T* Bs = As + BM * LDK;
    LA::store(ran, smem[(kt + 1) & 1], tid);
    LB::store(rbn, smem[(kt + 1) & 1] + BM * LDK, tid);
    la.load(ran, rs_a(min(kt + 3, nk - 1)));
    lb.load(rbn, rs_b(min(kt + 3, nk - 1)));
    __builtin_amdgcn_sched_barrier(0);
    u32x4 af[2][TM], bfr[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[0][i] = ld16(As + (wm * WM + i * 32 + l32) * LDK + g * V);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[0][j] = ld16(Bs + (wn * WN + j * 32 + l32) * LDK + g * V);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int c = ks & 1;
      if (ks + 1 < KSTEPS) {
        const int kk = (ks + 1) * TK::KSTEP;
#pragma unroll
        for (int i = 0; i < TM; ++i) af[c ^ 1][i] = ld16(As + (wm * WM + i * 32 + l32) * LDK + kk + g * V);
#pragma unroll
        for (int j = 0; j < TN; ++j) bfr[c ^ 1][j] = ld16(Bs + (wn * WN + j * 32 + l32) * LDK + kk + g * V);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(bfr[c][j], af[c][i], acc[i][j], (T*)nullptr);
    }
    // MFMA / fragment-read interleave: (TM+TN) reads per step spread over its TM*TN MFMAs
    constexpr int NR = TM + TN, NM = TM * TN, PER = NM / NR > 0 ? NM / NR : 1;
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (ks + 1 < KSTEPS) {
#pragma unroll
        for (int q = 0; q < NR; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (NM > NR * PER) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR * PER, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
      }
    }
    __syncthreads();
  };
  for (int kt = 0; kt < nk; kt += 2) {
    step(kt, ra1, rb1);   // tile kt+1 sits in set 1
    if (kt + 1 < nk) step(kt + 1, ra0, rb0);
  }

  static_assert(4 * 32 * (WN + 4) * sizeof(float) <= sizeof(smem), "epilogue staging must fit the LDS tiles");
  Epilogue<T, E>::template run<TM, TN, WN>(args, acc, reinterpret_cast<float*>(&smem[0][0]) + wave * 32 * (WN + 4),
                                             m0 + wm * WM, n0 + wn * WN, lane);
}

// Writes a wave's (TM*32) x WN accumulator tile through LDS so that global
// stores are row-contiguous: one 32-row slab at a time, the wave stores its
// accumulators (lane = row, 4 consecutive columns per register group) into a
// private [32][WN+4] fp32 region, then reads it back with WN/4 lanes per row
// and hands each lane 4 consecutive columns: op(m, n, v[4]). The +4 pitch
// keeps both the slab writes and the row reads free of bank conflicts.
// The staging slab is private to the wave, so its LDS writes and reads only
// need ordering within the wave (LDS instructions of one wave complete in
// order): a wave-scope fence keeps the compiler from moving them across each
// other, and no block barrier holds the other waves back.
DEV void slab_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int TM, int TN, int WN, class Op>
DEV void staged_store(f32x16 (&acc)[TM][TN], float* st, int mbase, int nbase, int lane, Op op) {
  constexpr int P = WN + 4, LPR = WN / 4, RPP = 64 / LPR;
  const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        float v[4] = {acc[i][j][blk * 4], acc[i][j][blk * 4 + 1], acc[i][j][blk * 4 + 2], acc[i][j][blk * 4 + 3]};
        store4(st + l32 * P + j * 32 + blk * 8 + g * 4, v);
      }
    slab_sync();
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += RPP) {
      const int row = r0 + lane / LPR, col = (lane % LPR) * 4;
      float v[4];
      load4(st + row * P + col, v);
      op(mbase + i * 32 + row, nbase + col, v);
    }
    slab_sync();
  }
}

// 8-column (16-byte) items of a bf16 output (and, for the residual, of its
// operand C): the columns, the row pitch and the base keep every item whole
// and 16-byte aligned
DEV bool row16_aligned(const GemmArgs& a) {
  return a.N % 8 == 0 && a.ldc % 8 == 0 && (reinterpret_cast<uintptr_t>(a.C) & 15) == 0;
}

// staged_store for bf16 outputs that depend on the accumulator alone:
// f(m, n, v) maps the 4 consecutive columns n .. n+3 of row m in place while
// they are still in accumulator order, the results are rounded to bf16
// before they go to the slab (a
// [32][WN+8] bf16 region: half the LDS bytes of the fp32 slab), and each lane
// then hands 8 consecutive bf16 of a row to out(m, n, 16 bytes). The values
// and their single rounding are those of staged_store + a bf16 store.
template <int TM, int TN, int WN>
constexpr bool kBf16Slab = WN % 16 == 0 && 64 % (WN / 8) == 0 && 32 % (64 / (WN / 8)) == 0;

template <int TM, int TN, int WN, class F, class Out>
DEV void staged_store_bf16(f32x16 (&acc)[TM][TN], float* stf, int mbase, int nbase, int lane, F f, Out out) {
  static_assert(kBf16Slab<TM, TN, WN>, "slab rows of whole 16-byte chunks");
  constexpr int PB = WN + 8, LPR = WN / 8, RPP = 64 / LPR;
  bf16* st = reinterpret_cast<bf16*>(stf);
  const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        float v[4] = {acc[i][j][blk * 4], acc[i][j][blk * 4 + 1], acc[i][j][blk * 4 + 2], acc[i][j][blk * 4 + 3]};
        f(mbase + i * 32 + l32, nbase + j * 32 + blk * 8 + g * 4, v);
        u32x2 pk;
        pk[0] = pack_bf16x2(v[0], v[1]);
        pk[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2*>(st + l32 * PB + j * 32 + blk * 8 + g * 4) = pk;
      }
    slab_sync();
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += RPP) {
      const int row = r0 + lane / LPR, col = (lane % LPR) * 8;
      out(mbase + i * 32 + row, nbase + col, ld16(st + row * PB + col));
    }
    slab_sync();
  }
}

// staged_store with a prefetch: pre(m, n) is issued for every (row, 4
// columns) item before the accumulators go to LDS, so those global loads are
// in flight during the staging; op(m, n, v, pre_value). ALL: every slab's
// items are requested up front (the whole tile's loads overlap), else one
// slab's at a time.
template <int TM, int TN, int WN, bool ALL = false, class Pre, class Op>
DEV void staged_store_pre(f32x16 (&acc)[TM][TN], float* st, int mbase, int nbase, int lane, Pre pre, Op op) {
  constexpr int P = WN + 4, LPR = WN / 4, RPP = 64 / LPR, NP = 32 / RPP;
  using PV = decltype(pre(0, 0));
  const int g = lane >> 5, l32 = lane & 31;
  const int prow = lane / LPR, pcol = (lane % LPR) * 4;
  PV pall[ALL ? TM : 1][NP];
  if constexpr (ALL) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int q = 0; q < NP; ++q) pall[i][q] = pre(mbase + i * 32 + q * RPP + prow, nbase + pcol);
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    PV pv[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) pv[q] = ALL ? pall[ALL ? i : 0][q] : pre(mbase + i * 32 + q * RPP + prow, nbase + pcol);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        float v[4] = {acc[i][j][blk * 4], acc[i][j][blk * 4 + 1], acc[i][j][blk * 4 + 2], acc[i][j][blk * 4 + 3]};
        store4(st + l32 * P + j * 32 + blk * 8 + g * 4, v);
      }
    // ALL: every prefetch has landed before the first store goes out. (Left
    // to itself the compiler waits per item, inside the item's bounds test,
    // and once stores are in flight a wait for a load is a wait for all
    // outstanding accesses: each item would wait for the previous store.)
    if (ALL && i == 0) wait_vmcnt<0>();
    slab_sync();
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int row = q * RPP + prow;
      float v[4];
      load4(st + row * P + pcol, v);
      op(mbase + i * 32 + row, nbase + pcol, v, pv[q]);
    }
    slab_sync();
  }
}

// staged_store_pre for bf16 outputs, 8 columns per lane: pre(m, n) returns
// the 16 bytes of operand at (m, n .. n+7) (every item requested up front,
// all landed before the first store), op(m, n, v[8], pre_value). Half the
// load and store instructions of the 4-column form for the same bytes.
template <int TM, int TN, int WN>
constexpr bool kPre8 = WN % 32 == 0 && 64 % (WN / 8) == 0 && 32 % (64 / (WN / 8)) == 0;

template <int TM, int TN, int WN, class Pre, class Op>
DEV void staged_store_pre8(f32x16 (&acc)[TM][TN], float* st, int mbase, int nbase, int lane, Pre pre, Op op) {
  static_assert(kPre8<TM, TN, WN>, "8-column items");
  constexpr int P = WN + 4, LPR = WN / 8, RPP = 64 / LPR, NP = 32 / RPP;
  const int g = lane >> 5, l32 = lane & 31;
  const int prow = lane / LPR, pcol = (lane % LPR) * 8;
  u32x4 pall[TM][NP];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int q = 0; q < NP; ++q) pall[i][q] = pre(mbase + i * 32 + q * RPP + prow, nbase + pcol);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        float v[4] = {acc[i][j][blk * 4], acc[i][j][blk * 4 + 1], acc[i][j][blk * 4 + 2], acc[i][j][blk * 4 + 3]};
        store4(st + l32 * P + j * 32 + blk * 8 + g * 4, v);
      }
    if (i == 0) wait_vmcnt<0>();  // as in staged_store_pre (ALL)
    slab_sync();
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int row = q * RPP + prow;
      float v[8], w[4];
      load4(st + row * P + pcol, w);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = w[e];
      load4(st + row * P + pcol + 4, w);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 + e] = w[e];
      op(mbase + i * 32 + row, nbase + pcol, v, pall[i][q]);
    }
    slab_sync();
  }
}

// Output addressing of a wave's (TM*32) x WN tile at (mbase, nbase) in a
// row-major matrix of leading dimension ld: one 64-bit base per wave and
// 32-bit element offsets from it (the launcher bounds ld by 2^22 so that the
// tile's rows fit), and no per-item bounds test when the whole tile lies
// inside M x N. (64-bit index arithmetic and the bounds test per 4-column
// item were half the instructions of the store path.) Used where it measured
// faster: the residual and fp32-gradient epilogues keep the 64-bit form
// (the residual one, which reads and writes the same positions, ran 17 %
// slower with this).
template <int TM, int WN>
struct TileAddr {
  static_assert(TM * 32 <= 256, "32-bit offsets: at most 256 rows of at most 2^22 elements");
  int64_t base;
  int ld, mbase, nbase, M, N;
  bool full;
  DEV TileAddr(int64_t ld_, int mb, int nb, int M_, int N_)
      : base((int64_t)mb * ld_ + nb), ld((int)ld_), mbase(mb), nbase(nb), M(M_), N(N_),
        full(mb + TM * 32 <= M_ && nb + WN <= N_) {}
  DEV bool in(int m, int n) const { return full || (m < M && n < N); }
  DEV int off(int m, int n) const { return (m - mbase) * ld + (n - nbase); }
};

template <typename T>
struct Epilogue<T, Epi::Store> {
  template <int TM, int TN, int WN, bool FOLD = false>
  static DEV void run(const GemmArgs& a, f32x16 (&acc)[TM][TN], float* lds, int mbase, int nbase, int lane) {
    const TileAddr<TM, WN> t(a.ldc, mbase, nbase, a.M, a.N);
    T* C = reinterpret_cast<T*>(a.C) + t.base;
    if constexpr (sizeof(T) == 2 && kBf16Slab<TM, TN, WN>) {
      if (row16_aligned(a)) {  // 8-column items: whole 16-byte chunks inside the rows
        staged_store_bf16<TM, TN, WN>(acc, lds, mbase, nbase, lane, [](int, int, float (&)[4]) {},
                                      [&](int m, int n, u32x4 v) {
                                        if (t.in(m, n)) st16_nt(C + t.off(m, n), v);
                                      });
        return;
      }
    }
    staged_store<TM, TN, WN>(acc, lds, mbase, nbase, lane, [&](int m, int n, float (&v)[4]) {
      if (t.in(m, n)) store4_nt(C + t.off(m, n), v);
    });
  }
};

template <typename T>
struct Epilogue<T, Epi::Residual> {
  template <int TM, int TN, int WN, bool FOLD = false>
  static DEV void run(const GemmArgs& a, f32x16 (&acc)[TM][TN], float* lds, int mbase, int nbase, int lane) {
    T* C = reinterpret_cast<T*>(a.C);
    if constexpr (sizeof(T) == 2 && kPre8<TM, TN, WN>) {
      if (row16_aligned(a)) {
        auto pre8 = [&](int m, int n) {
          u32x4 r = {0u, 0u, 0u, 0u};
          if (m < a.M && n < a.N) r = ld16_nt(C + (int64_t)m * a.ldc + n);
          return r;
        };
        staged_store_pre8<TM, TN, WN>(acc, lds, mbase, nbase, lane, pre8,
                                      [&](int m, int n, float (&v)[8], u32x4 r) {
          if (m < a.M && n < a.N) {
            u32x4 o;
#pragma unroll
            for (int h = 0; h < 4; ++h)
              o[h] = pack_bf16x2(__uint_as_float(r[h] << 16) + v[2 * h],
                                 __uint_as_float(r[h] & 0xffff0000u) + v[2 * h + 1]);
            st16_nt(C + (int64_t)m * a.ldc + n, o);
          }
        });
        return;
      }
    }
    // bf16: the residual is requested for the whole tile up front (raw, 4
    // values in two dwords); fp32 loads it per item
    auto pre = [&](int m, int n) {
      u32x2 r = {0u, 0u};
      if constexpr (sizeof(T) == 2) {
        if (m < a.M && n < a.N) r = ld8_nt(C + (int64_t)m * a.ldc + n);
      }
      return r;
    };
    staged_store_pre<TM, TN, WN, sizeof(T) == 2>(acc, lds, mbase, nbase, lane, pre,
                                                 [&](int m, int n, float (&v)[4], u32x2 r) {
      if (m < a.M && n < a.N) {
        float x[4];
        if constexpr (sizeof(T) == 2) {
          x[0] = __uint_as_float(r[0] << 16); x[1] = __uint_as_float(r[0] & 0xffff0000u);
          x[2] = __uint_as_float(r[1] << 16); x[3] = __uint_as_float(r[1] & 0xffff0000u);
        } else {
          load4(C + (int64_t)m * a.ldc + n, x);
        }
        for (int q = 0; q < 4; ++q) x[q] += v[q];
        store4_nt(C + (int64_t)m * a.ldc + n, x);
      }
    });
  }
};

// relu^2 MLP activation (aethryn.com, section "A Llama-class transformer with
// ten modern departures"): stores a = max(u, 0)^2 only; the backward recovers
// max(u, 0) as sqrt(a).
template <typename T>
struct Epilogue<T, Epi::Relu2> {
  template <int TM, int TN, int WN, bool FOLD = false>
  static DEV void run(const GemmArgs& a, f32x16 (&acc)[TM][TN], float* lds, int mbase, int nbase, int lane) {
    const TileAddr<TM, WN> t(a.ldc, mbase, nbase, a.M, a.N);
    T* A2 = reinterpret_cast<T*>(a.C) + t.base;
    float mx = 0.f;
    if constexpr (sizeof(T) == 2 && kBf16Slab<TM, TN, WN>) {
      if (row16_aligned(a)) {
        staged_store_bf16<TM, TN, WN>(acc, lds, mbase, nbase, lane,
                                      [&](int m, int n, float (&v)[4]) {
                                        for (int r = 0; r < 4; ++r) {
                                          const float p = fmaxf(v[r], 0.f);
                                          v[r] = p * p;
                                        }
                                        if (FOLD && t.in(m, n))
                                          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, v[r]);
                                      },
                                      [&](int m, int n, u32x4 v) {
                                        if (t.in(m, n)) st16_nt(A2 + t.off(m, n), v);
                                      });
        if constexpr (FOLD)
          if (a.amax_out) amax_fold_block<T>(mx, a.amax_out);
        return;
      }
    }
    staged_store<TM, TN, WN>(acc, lds, mbase, nbase, lane, [&](int m, int n, float (&v)[4]) {
      if (t.in(m, n)) {
        float s[4];
        for (int r = 0; r < 4; ++r) {
          const float p = fmaxf(v[r], 0.f);
          s[r] = p * p;
          mx = fmaxf(mx, s[r]);
        }
        store4_nt(A2 + t.off(m, n), s);
      }
    });
    if constexpr (FOLD)  // the whole block runs the epilogue
      if (a.amax_out) amax_fold_block<T>(mx, a.amax_out);
  }
};

// du = da * 2 max(u, 0) = da * 2 sqrt(a), with a = max(u, 0)^2 read from C2
// (prefetched per slab)
template <typename T>
struct Epilogue<T, Epi::Relu2Bwd> {
  template <int TM, int TN, int WN, bool FOLD = false>
  static DEV void run(const GemmArgs& a, f32x16 (&acc)[TM][TN], float* lds, int mbase, int nbase, int lane) {
    const TileAddr<TM, WN> t(a.ldc, mbase, nbase, a.M, a.N), t2(a.ldc2, mbase, nbase, a.M, a.N);
    T* Dp = reinterpret_cast<T*>(a.C) + t.base;
    const T* A2 = reinterpret_cast<const T*>(a.C2) + t2.base;
    float mx = 0.f;
    // a is prefetched raw (4 bf16 in two dwords) for the whole tile
    auto pre = [&](int m, int n) {
      u32x2 r = {0u, 0u};
      if constexpr (sizeof(T) == 2) {
        if (t.in(m, n)) r = ld8_nt(A2 + t2.off(m, n));
      }
      return r;
    };
    staged_store_pre<TM, TN, WN, sizeof(T) == 2>(acc, lds, mbase, nbase, lane, pre,
                                                 [&](int m, int n, float (&v)[4], u32x2 r) {
      if (t.in(m, n)) {
        float x[4];
        if constexpr (sizeof(T) == 2) {
          x[0] = __uint_as_float(r[0] << 16); x[1] = __uint_as_float(r[0] & 0xffff0000u);
          x[2] = __uint_as_float(r[1] << 16); x[3] = __uint_as_float(r[1] & 0xffff0000u);
        } else {
          load4(A2 + t2.off(m, n), x);
        }
        // v_sqrt_f32 alone, not correctly rounded: sqrtf's correctly rounded
        // expansion costs about fifteen instructions per element here, and the
        // product is rounded to the activation dtype anyway
        for (int q = 0; q < 4; ++q) {
          v[q] *= 2.f * __builtin_amdgcn_sqrtf(x[q]);
          mx = fmaxf(mx, fabsf(v[q]));
        }
        store4_nt(Dp + t.off(m, n), v);
      }
    });
    if constexpr (FOLD)
      if (a.amax_out) amax_fold_block<T>(mx, a.amax_out);
  }
};

// LM head with the logit softcap z' = c*tanh(z/c), evaluated on the fp32
// accumulator (aethryn.com, section "A Llama-class transformer with ten modern
// departures": softcap 15, in float32). Emits one fp32 partial sum of
// exp(z' - c) per row and 64 columns (terms lie in (e^-2c, 1], so partial
// sums add without rescaling), the fp32 z' at the row's target, and, in the
// activation dtype, q = exp(z' - c) (1 - (z'/c)^2) for every entry: the
// softmax numerator times the slope of the softcap, from which the backward
// needs only a per-row scale and a fix at the target column (the cross-entropy
// gradient dz = (exp(z' - lse) - [v == target]) (1 - (z'/c)^2) dloss / N).
// All three come from R = 1 / (exp(2z/c) + 1): tanh(z/c) = 1 - 2R, so
// z' - c = -2cR and 1 - (z'/c)^2 = 4R(1 - R), free of the cancellation of
// the plain forms near tanh = +-1; three transcendentals and six other
// instructions per entry (exp overflow to inf gives R = 0, underflow R = 1).
// Done on the staged rows: 64 columns of a row sit in 16 lanes (4 each),
// reduced by DPP row rotations. The row's target id is prefetched with the slab.
template <typename T>
struct Epilogue<T, Epi::LMHead> {
  template <int TM, int TN, int WN, bool FOLD = false>
  static DEV void run(const GemmArgs& a, f32x16 (&acc)[TM][TN], float* lds, int mbase, int nbase, int lane) {
    static_assert(WN % kLMHeadPartCols == 0 && kLMHeadPartCols == 64, "16 lanes per partial");
    constexpr float kLog2e = 1.4426950408889634f;
    const float c = a.softcap;
    const float k2 = 2.f * kLog2e / c;   // exp(2z/c) as exp2(z * k2)
    const float kq = -2.f * c * kLog2e;  // 4 exp(-2cR) as exp2(R * kq + 2)
    const int nparts = a.N / kLMHeadPartCols;
    const TileAddr<TM, WN> t(a.ldc, mbase, nbase, a.M, a.N);
    T* Z = reinterpret_cast<T*>(a.C) + t.base;
    float* part = a.part + ((int64_t)mbase * nparts + nbase / kLMHeadPartCols);
    auto pre = [&](int m, int) { return m < a.M ? a.targets[m] : -1; };
    staged_store_pre<TM, TN, WN>(acc, lds, mbase, nbase, lane, pre, [&](int m, int n, float (&v)[4], int tgt) {
      const bool mv = t.full || m < a.M;
      float sum4 = 0.f, R[4], q[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        R[r] = __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(v[r] * k2) + 1.f);
        const float e4 = __builtin_amdgcn_exp2f(fmaf(R[r], kq, 2.f));  // 4 exp(z' - c)
        sum4 += e4;
        q[r] = e4 * fmaf(-R[r], R[r], R[r]);
      }
      // the target's column among the lane's 4: chosen from scalars by
      // compares (a select chain over an array is folded into an indexed
      // load that puts the array in scratch memory)
      const unsigned d = (unsigned)(tgt - n);
      const float Rt = d == 0u ? R[0] : (d == 1u ? R[1] : (d == 2u ? R[2] : R[3]));
      if (d < 4u) a.ztgt[m] = fmaf(-2.f * c, Rt, c);
      if (mv) store4_nt(Z + t.off(m, n), q);
      const float sum = row16_sum(0.25f * sum4);  // the row's 64 columns sit in 16 lanes
      if (mv && (lane & 15) == 0) part[(m - mbase) * nparts + (n - nbase) / kLMHeadPartCols] = sum;
    });
  }
};

template <typename T>
struct Epilogue<T, Epi::GradF32> {
  template <int TM, int TN, int WN, bool FOLD = false>
  static DEV void run(const GemmArgs& a, f32x16 (&acc)[TM][TN], float* lds, int mbase, int nbase, int lane) {
    if (a.splits > 1) {
      const int z = a.zslice >= 0 ? a.zslice : (int)blockIdx.z;
      float* P = a.split_buf + (int64_t)z * a.M * a.N;
      staged_store<TM, TN, WN>(acc, lds, mbase, nbase, lane, [&](int m, int n, float (&v)[4]) {
        if (m < a.M && n < a.N) store4_nt(P + (int64_t)m * a.N + n, v);
      });
    } else {
      float* G = reinterpret_cast<float*>(a.C);
      const bool accum = a.accumulate != 0;
      staged_store<TM, TN, WN>(acc, lds, mbase, nbase, lane, [&](int m, int n, float (&v)[4]) {
        if (m < a.M && n < a.N) {
          float* p = G + (int64_t)m * a.ldc + n;
          if (accum) {
            float x[4];
            load4_nt(p, x);
            for (int r = 0; r < 4; ++r) v[r] += x[r];
          }
          store4_nt(p, v);
        }
      });
    }
  }
};

// GEMM with both operands k-contiguous (y = x W^T and, with a transposed
// weight copy, dx = dy W; with token-major transposed copies also dW), fed by
// direct-to-LDS buffer loads. ES is the operand element size: 2 = bf16
// (32x32x16 MFMA), 1 = fp8 e4m3 (32x32x64 MFMA on the same byte tiles, two
// 16-byte fragments per operand, and the accumulator scaled by
// 1 / (s_a s_b) from the operands' amax slots before the epilogue). Split-K
// (GradF32 only) runs slices of whole K tiles over a slice-major 1-D grid.
//
// K tiles are 64- or 128-byte rows (BK elements) and live in NSTAGE
// LDS stages; tile kt + NSTAGE - 1 is requested while tile kt is consumed. A
// wave's buffer_load ... lds writes 1 KiB contiguous (lane L at +16L), i.e.
// 1024/ROWB rows; each lane picks the global 16-byte chunk it fetches so that
// chunk c of row r lands at position c ^ ((r / RP) mod CH), RP = 256/ROWB
// rows per 256 bytes, CH = ROWB/16 chunks per row. A 16-lane slice of an
// MFMA fragment read (16 consecutive rows, one chunk) then covers all 64 banks
// once: rows in one 256-byte bank line differ in their row offset, rows RP
// apart in the chunk position. Rows past M read as zero (buffer record count).
// One explicit vmcnt wait and one barrier per K tile.
template <int BM, int BN, int NSTAGE, int OCC, Epi E, int NW = 4, int BK = 32, int ES = 2, bool PP = false>
__global__ __launch_bounds__(NW * 64, OCC) void gemm_nt_lds_kernel(GemmArgs args) {
  using T = bf16;  // output (epilogue) type
  constexpr int ROWB = BK * ES, CH = ROWB / 16, RP = 256 / ROWB, RPK = 1024 / ROWB;
  constexpr int KSTEPS = ROWB / 32;  // 16-byte fragment pairs (lane groups 0/1) per row
  constexpr int WGN = NW / 2;                              // waves along n (2 along m)
  constexpr int WM = BM / 2, WN = BN / WGN, TM = WM / 32, TN = WN / 32;
  constexpr int STAGE = (BM + BN) * ROWB;                  // bytes per stage
  constexpr int LA = BM * ROWB / 1024 / NW, LB = BN * ROWB / 1024 / NW;  // 1 KiB loads per wave per tile
  constexpr int NLOAD = LA + LB;
  static_assert(ROWB == 64 || ROWB == 128, "K tile");
  static_assert(ES == 2 || ES == 1, "bf16 or fp8 operands");
  static_assert(LA >= 1 && LB >= 1, "tile too small for the wave count");
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "two to four stage arrays");
  // one array per stage, so the compiler can tell the stages' LDS-direct
  // loads apart and wait only for the oldest tile
  __shared__ __attribute__((aligned(1024))) char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[NSTAGE >= 3 ? STAGE : 1024];
  __shared__ __attribute__((aligned(1024))) char st3[NSTAGE == 4 ? STAGE : 1024];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wm = wave / WGN, wn = wave % WGN, g = lane >> 5, l32 = lane & 31;
  const int M = args.M, N = args.N, K = args.K;
  const int tiles_n = (N + BN - 1) / BN, tiles = ((M + BM - 1) / BM) * tiles_n;
  // blocks are dealt round-robin to the 8 XCDs: remap so that each XCD takes
  // a contiguous run of items (neighbouring tiles, whole split-K slices).
  // Within a slice, tiles go in groups of kGroupM row panels, down the group
  // first: the blocks an XCD runs side by side cover a few row panels and a
  // few column panels, so both operands' K windows are shared in its L2
  // (row-major order would stream every column panel of B once per row panel).
  int item = blockIdx.x;
  const int nb = gridDim.x;
  item = xcd_contiguous(item, nb);
  // batched products: product-major, then split-K slices, then tiles
  const int bz = item / (tiles * args.splits);
  item -= bz * tiles * args.splits;
  const int split = item / tiles, bid = item % tiles;
  const int tiles_m = tiles / tiles_n;
  const int grp = bid / (kGroupM * tiles_n), first_m = grp * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM), r = bid - grp * kGroupM * tiles_n;
  const int m0 = (first_m + r % gm) * BM, n0 = (r / gm) * BN;
  const int kper = ((K + args.splits - 1) / args.splits + BK - 1) / BK * BK;
  const int kbeg = split * kper;
  const int kend = min(K, kbeg + kper);
  const int nk = kend > kbeg ? (kend - kbeg) / BK : 0;
  const char* Ap = reinterpret_cast<const char*>(args.A) + bz * args.stride_a + ((int64_t)m0 * args.lda + kbeg) * ES;
  const char* Bp = reinterpret_cast<const char*>(args.B) + bz * args.stride_b + ((int64_t)n0 * args.ldb + kbeg) * ES;
  const uint32_t lda_b = (uint32_t)(args.lda * ES), ldb_b = (uint32_t)(args.ldb * ES);
  // record counts (bytes from the tile's first row), clamped to 1 GiB; plain
  // integer ternaries (a templated 64-bit min() would go through f64 VALU
  // math and make the resource look divergent)
  const int64_t ra64 = (int64_t)(M - m0 < BM ? M - m0 : BM) * lda_b;
  const int64_t rb64 = (int64_t)(N - n0 < BN ? N - n0 : BN) * ldb_b;
  const int rec_a = ra64 > (1 << 30) ? (1 << 30) : (int)ra64;
  const int rec_b = rb64 > (1 << 30) ? (1 << 30) : (int)rb64;

  // per-lane global byte offsets of this wave's 1 KiB slots (RPK rows each);
  // the swizzle depends on the tile row, not on the row within the slot
  const int lrow = lane / CH, lpos = lane % CH;
  uint32_t voa[LA], vob[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = (wave * LA + i) * RPK + lrow;
    voa[i] = (uint32_t)r * lda_b + (uint32_t)(lpos ^ ((r / RP) & (CH - 1))) * 16u;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = (wave * LB + i) * RPK + lrow;
    vob[i] = (uint32_t)r * ldb_b + (uint32_t)(lpos ^ ((r / RP) & (CH - 1))) * 16u;
  }

  auto stage = [&](int q) -> char* { return q == 0 ? st0 : q == 1 ? st1 : q == 2 ? st2 : st3; };
  auto issue = [&](int kt, char* st) {
    const int k0 = kt * ROWB;  // bytes
    const __amdgpu_buffer_rsrc_t ra = uniform_rsrc(Ap + k0, rec_a);
    const __amdgpu_buffer_rsrc_t rb = uniform_rsrc(Bp + k0, rec_b);
#pragma unroll
    for (int i = 0; i < LA; ++i)
      lds_direct16(ra, st + (wave * LA + i) * 1024, voa[i]);
#pragma unroll
    for (int i = 0; i < LB; ++i)
      lds_direct16(rb, st + BM * ROWB + (wave * LB + i) * 1024, vob[i]);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragment byte offsets inside a stage for each k-step (row l32 of a 32-row block)
  const int swz = (l32 / RP) & (CH - 1);
  int fo[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) fo[ks] = l32 * ROWB + ((ks * 2 + g) ^ swz) * 16;

  issue(0, st0);
  if constexpr (PP) {
    // Ping-pong: the waves of rows 0..WM-1 (group 0, one per SIMD) and of
    // rows WM.. (group 1) take turns. A K tile is NP parts of two MFMA
    // k-steps, and every wave runs the same sequence per tile: read the
    // fragments of a part, multiply them, one phase each, a barrier starting
    // every phase. Group 1 runs one phase behind group 0, so in every phase
    // one wave per SIMD feeds the matrix core while the other waits on LDS.
    // A wave requests its part of tile m + NSTAGE - 1 when it starts reading
    // tile m (that stage was last read by group 1 in the phase before group 0
    // starts tile m) and waits for its part of tile m + 1 before its last
    // phase of tile m, which ends before group 0 reads tile m + 1.
    static_assert(NW == 8 && KSTEPS % 2 == 0, "two groups of four waves, k-step pairs");
    constexpr int NP = KSTEPS / 2;
    u32x4 af[2][TM], bfr[2][TN];
    auto readf = [&](const char* cur, int part) __attribute__((always_inline)) {
      const char* As = cur + wm * WM * ROWB;
      const char* Bs = cur + BM * ROWB + wn * WN * ROWB;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int ks = part * 2 + k;
#pragma unroll
        for (int i = 0; i < TM; ++i) af[k][i] = ld16(As + i * 32 * ROWB + fo[ks]);
#pragma unroll
        for (int j = 0; j < TN; ++j) bfr[k][j] = ld16(Bs + j * 32 * ROWB + fo[ks]);
      }
    };
    auto mma = [&]() __attribute__((always_inline)) {
      if constexpr (ES == 2) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(bfr[k][j], af[k][i], acc[i][j], (T*)nullptr);
      } else {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma_fp8(bfr[0][j], bfr[1][j], af[0][i], af[1][i], acc[i][j]);
      }
    };
    auto phase = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    constexpr int YOUNG = NLOAD * (NSTAGE - 2);  // loads of the tiles after the one awaited
    auto tile_pp = [&](int m, const char* cur, char* nxt) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        phase();
        if (p == 0) issue(min(m + NSTAGE - 1, nk - 1), nxt);  // past the end: a harmless re-read into a free stage
        readf(cur, p);
        if (p == NP - 1) wait_vmcnt<YOUNG>();  // this wave's part of tile m + 1 has landed
        phase();
        mma();
      }
    };
    if (NSTAGE >= 3) issue(min(1, nk - 1), st1);
    if (NSTAGE == 4) issue(min(2, nk - 1), st2);
    wait_vmcnt<YOUNG>();   // tile 0
    if (wm == 1) phase();  // group 1 starts one phase later
    if constexpr (NSTAGE == 4) {
      for (int m = 0; m < nk; m += 4) {
        tile_pp(m, st0, st3);
        if (m + 1 < nk) tile_pp(m + 1, st1, st0);
        if (m + 2 < nk) tile_pp(m + 2, st2, st1);
        if (m + 3 < nk) tile_pp(m + 3, st3, st2);
      }
    } else if constexpr (NSTAGE == 3) {
      for (int m = 0; m < nk; m += 3) {
        tile_pp(m, st0, st2);
        if (m + 1 < nk) tile_pp(m + 1, st1, st0);
        if (m + 2 < nk) tile_pp(m + 2, st2, st1);
      }
    } else {
      for (int m = 0; m < nk; m += 2) {
        tile_pp(m, st0, st1);
        if (m + 1 < nk) tile_pp(m + 1, st1, st0);
      }
    }
    if (wm == 0) phase();  // and group 0 ends one phase later
  } else {
  if (NSTAGE >= 3) issue(max(0, min(1, nk - 1)), st1);
  if (NSTAGE == 4) issue(max(0, min(2, nk - 1)), st2);
  // tile kt sits in stage kt % NSTAGE; the loop is unrolled by NSTAGE so
  // every stage is a distinct, statically known LDS object
  auto tile = [&](int kt, const char* cur, char* nxt) {
    // tile kt's loads are the oldest outstanding: wait until only the
    // NSTAGE-2 younger tiles' loads remain, then make everyone's visible
    // (a bare s_barrier: __syncthreads' release fence would wait for every
    // outstanding LDS-direct load, including the younger tiles')
    constexpr int YOUNG = NLOAD * (NSTAGE - 2);
    __builtin_amdgcn_s_waitcnt(((YOUNG >> 4) << 14) | (0x7 << 4) | (0xF << 8) | (YOUNG & 15));
    __builtin_amdgcn_s_barrier();
    issue(min(kt + NSTAGE - 1, nk - 1), nxt);  // into the stage freed by tile kt-1 (past the end: harmless re-read)
    const char* As = cur + wm * WM * ROWB;
    const char* Bs = cur + BM * ROWB + wn * WN * ROWB;
    u32x4 af[KSTEPS][TM], bfr[KSTEPS][TN];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int i = 0; i < TM; ++i) af[ks][i] = ld16(As + i * 32 * ROWB + fo[ks]);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[ks][j] = ld16(Bs + j * 32 * ROWB + fo[ks]);
    }
    if constexpr (ES == 2) {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(bfr[ks][j], af[ks][i], acc[i][j], (T*)nullptr);
    } else {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ks += 2)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = mfma_fp8(bfr[ks][j], bfr[ks + 1][j], af[ks][i], af[ks + 1][i], acc[i][j]);
    }
    // interleave: the reads of step s+1 between the MFMAs of step s (an fp8
    // step consumes two fragment pairs)
    constexpr int RPS = ES == 2 ? 1 : 2, MSTEPS = KSTEPS / RPS;
    constexpr int NR = (TM + TN) * RPS, NM = TM * TN, PER = NM / NR > 0 ? NM / NR : 1;
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int ms = 0; ms < MSTEPS; ++ms) {
      if (ms + 1 < MSTEPS) {
#pragma unroll
        for (int q = 0; q < NR; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (NM > NR * PER) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR * PER, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
      }
    }
  };
  if constexpr (NSTAGE == 4) {
    for (int kt = 0; kt < nk; kt += 4) {
      tile(kt, st0, st3);
      if (kt + 1 < nk) tile(kt + 1, st1, st0);
      if (kt + 2 < nk) tile(kt + 2, st2, st1);
      if (kt + 3 < nk) tile(kt + 3, st3, st2);
    }
  } else if constexpr (NSTAGE == 3) {
    for (int kt = 0; kt < nk; kt += 3) {
      tile(kt, st0, st2);
      if (kt + 1 < nk) tile(kt + 1, st1, st0);
      if (kt + 2 < nk) tile(kt + 2, st2, st1);
    }
  } else {
    for (int kt = 0; kt < nk; kt += 2) {
      tile(kt, st0, st1);
      if (kt + 1 < nk) tile(kt + 1, st1, st0);
    }
  }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no LDS-direct load may land during the epilogue
  __syncthreads();
  // each wave stages its 32-row slabs in a private region: two waves per
  // stage when two slabs fit, else one stage per wave
  constexpr int SLAB = 32 * (WN + 4) * (int)sizeof(float);
  constexpr int PERST = STAGE / SLAB;  // slabs per stage
  static_assert(PERST >= 1 && (NW + PERST - 1) / PERST <= NSTAGE, "epilogue slabs must fit the stages");
  float* slab = reinterpret_cast<float*>(stage(wave / PERST) + (wave % PERST) * SLAB);
  if constexpr (ES == 1) {
    const float aa = *args.amax_a, ab = *args.amax_b;
    const float sa = aa > 0.f ? 448.f / aa : 1.f, sb = ab > 0.f ? 448.f / ab : 1.f;
    const float f = 1.f / (sa * sb);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] *= f;
  }
  GemmArgs ea = args;
  ea.zslice = split;
  ea.C = reinterpret_cast<char*>(args.C) + bz * args.stride_c;
  // FP8 products (ES = 1) fold the |max| of a relu^2 / relu^2-backward output
  Epilogue<T, E>::template run<TM, TN, WN, ES == 1>(ea, acc, slab, m0 + wm * WM, n0 + wn * WN, lane);
}

// bf16 GEMM with both operands mn-contiguous (dW = dy^T x: A = dy [K, M] and
// B = x [K, N], k = token), fed by direct-to-LDS buffer loads and read with
// the transposing LDS read (ds_read_b64_tr_b16), so no register transposes.
//
// A K tile of 32 rows lands as [32][BM] and [32][BN] bf16. A wave's 1 KiB
// load covers 1024/(2*BM) k rows; chunk c of k row r sits at position
// c ^ s(r) with s(r) = ((r & 7) << 2) mod (chunks per row), which shifts each
// row's 64-byte windows so that the four k rows one half-wave's transposing
// read touches fall on distinct banks. The MFMA k order is the one the
// transposing read delivers (rows 4g+e, then 8+4g+e, of each 16-row step),
// the same for both operands. Pipeline and epilogue as in the NT kernel;
// split-K slices are whole K tiles.
template <int BM, int BN, int NSTAGE, int OCC, Epi E, int NW = 4, int BK = 32, bool PP = false>
__global__ __launch_bounds__(NW * 64, OCC) void gemm_tn_lds_kernel(GemmArgs args) {
  using T = bf16;
  constexpr int KK = BK / 16;                   // MFMA k-steps per K tile
  constexpr int ROWA = BM * 2, ROWB = BN * 2;   // bytes per k row
  constexpr int CHA = ROWA / 16, CHB = ROWB / 16;
  constexpr int WGN = NW / 2;                   // waves along n (2 along m)
  constexpr int WM = BM / 2, WN = BN / WGN, TM = WM / 32, TN = WN / 32;
  constexpr int STAGE = BK * (ROWA + ROWB);
  constexpr int LA = BK * ROWA / 1024 / NW, LB = BK * ROWB / 1024 / NW;  // 1 KiB loads per wave per tile
  constexpr int NLOAD = LA + LB;
  static_assert(LA >= 1 && LB >= 1 && CHA >= 16 && CHB >= 16, "tile shape");
  static_assert(BK == 32 || BK == 64, "K tile");
  __shared__ __attribute__((aligned(1024))) char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[NSTAGE >= 3 ? STAGE : 1024];
  __shared__ __attribute__((aligned(1024))) char st3[NSTAGE == 4 ? STAGE : 1024];
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "two to four stage arrays");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN, g = lane >> 5;
  const int M = args.M, N = args.N, K = args.K;
  const int tiles_n = (N + BN - 1) / BN, tiles = ((M + BM - 1) / BM) * tiles_n;
  // 1-D grid over (split-K slice, tile), slice-major. Blocks are dealt
  // round-robin to the 8 XCDs; remap so that each XCD takes a contiguous run
  // of items, i.e. whole slices: the tiles of one slice stream through the
  // same K window together and share it in that XCD's L2.
  int item = blockIdx.x;
  const int nb = gridDim.x;
  item = xcd_contiguous(item, nb);
  const int split = item / tiles, bid = item % tiles;
  const int m0 = (bid / tiles_n) * BM, n0 = (bid % tiles_n) * BN;
  const int kper = ((K + args.splits - 1) / args.splits + BK - 1) / BK * BK;
  const int kbeg = split * kper;
  const int kend = min(K, kbeg + kper);
  const int nk = kend > kbeg ? (kend - kbeg) / BK : 0;
  const T* Ap = reinterpret_cast<const T*>(args.A) + m0;
  const T* Bp = reinterpret_cast<const T*>(args.B) + n0;
  const uint32_t lda_b = (uint32_t)(args.lda * 2), ldb_b = (uint32_t)(args.ldb * 2);
  // record counts from a tile's first element: 31 full rows, then the last
  // row up to column M (resp. N); integer ternaries keep them scalar
  const int64_t ra64 = (int64_t)(BK - 1) * lda_b + (int64_t)(M - m0 < BM ? M - m0 : BM) * 2;
  const int64_t rb64 = (int64_t)(BK - 1) * ldb_b + (int64_t)(N - n0 < BN ? N - n0 : BN) * 2;
  const int rec_a = ra64 > (1 << 30) ? (1 << 30) : (int)ra64;
  const int rec_b = rb64 > (1 << 30) ? (1 << 30) : (int)rb64;

  // per-lane global offsets of this wave's 1 KiB slots
  uint32_t voa[LA], vob[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = (wave * LA + i) * (1024 / ROWA) + lane / CHA, p = lane % CHA;
    const int c = p ^ (((r & 7) << 2) & (CHA - 1));
    voa[i] = (uint32_t)r * lda_b + (uint32_t)c * 16u;
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = (wave * LB + i) * (1024 / ROWB) + lane / CHB, p = lane % CHB;
    const int c = p ^ (((r & 7) << 2) & (CHB - 1));
    vob[i] = (uint32_t)r * ldb_b + (uint32_t)c * 16u;
  }
  auto stage = [&](int q) -> char* { return q == 0 ? st0 : q == 1 ? st1 : q == 2 ? st2 : st3; };
  auto issue = [&](int kt, char* st) {
    const int64_t k0 = kbeg + (int64_t)kt * BK;
    const __amdgpu_buffer_rsrc_t ra = uniform_rsrc(Ap + k0 * args.lda, rec_a);
    const __amdgpu_buffer_rsrc_t rb = uniform_rsrc(Bp + k0 * args.ldb, rec_b);
#pragma unroll
    for (int i = 0; i < LA; ++i) lds_direct16(ra, st + (wave * LA + i) * 1024, voa[i]);
#pragma unroll
    for (int i = 0; i < LB; ++i) lds_direct16(rb, st + BK * ROWA + (wave * LB + i) * 1024, vob[i]);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // transposing-read offsets: source lane 4e + c of each 16-lane group names k
  // row 4g + e (+8 for the second half) and columns [4c, 4c + 4) of its
  // group's 16 (group parity picks columns 0-15 or 16-31 of a 32-column block)
  const int e4 = (lane >> 2) & 3, c4 = lane & 3, grp = lane >> 4;
  const int x = 4 * g + e4;                    // k row within a 16-row step (first half)
  const int c0 = 2 * (grp & 1) + (c4 >> 1);    // chunk within a 32-column block
  const int sa = (x << 2) & (CHA - 1), sb = (x << 2) & (CHB - 1);
  int ofa[TM], ofb[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) ofa[i] = x * ROWA + ((((wm * WM + i * 32) >> 3) ^ sa) + c0) * 16 + (c4 & 1) * 8;
#pragma unroll
  for (int j = 0; j < TN; ++j) ofb[j] = x * ROWB + ((((wn * WN + j * 32) >> 3) ^ sb) + c0) * 16 + (c4 & 1) * 8;
  auto frag = [](const char* base, int off, int row_b) -> u32x4 {
    const u32x2 lo = ld_tr16(base + off), hi = ld_tr16(base + off + 8 * row_b);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };

  issue(0, st0);
  if (NSTAGE >= 3) issue(max(0, min(1, nk - 1)), st1);
  if (NSTAGE == 4) issue(max(0, min(2, nk - 1)), st2);
  if constexpr (PP) {
    // Ping-pong as in the k-contiguous kernel: the two row-half wave groups
    // (one wave per SIMD each) alternate between reading a K tile's
    // fragments (transposing reads) and multiplying them, group 1 one phase
    // behind, a barrier starting every phase. A wave requests its part of
    // tile m + NSTAGE - 1 when it starts reading tile m and waits for its
    // part of tile m + 1 before it multiplies tile m.
    static_assert(NW == 8, "two groups of four waves");
    constexpr int YOUNG = NLOAD * (NSTAGE - 2);
    u32x4 af[KK][TM], bfr[KK][TN];
    auto readf = [&](const char* cur) __attribute__((always_inline)) {
      const char* As = cur;
      const char* Bs = cur + BK * ROWA;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int i = 0; i < TM; ++i) af[kk][i] = frag(As + kk * 16 * ROWA, ofa[i], ROWA);
#pragma unroll
        for (int j = 0; j < TN; ++j) bfr[kk][j] = frag(Bs + kk * 16 * ROWB, ofb[j], ROWB);
      }
    };
    auto mma = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(bfr[kk][j], af[kk][i], acc[i][j], (T*)nullptr);
    };
    auto phase = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    auto tile_pp = [&](int m, const char* cur, char* nxt) __attribute__((always_inline)) {
      phase();
      issue(min(m + NSTAGE - 1, nk - 1), nxt);  // past the end: a harmless re-read into a free stage
      readf(cur);
      wait_vmcnt<YOUNG>();  // this wave's part of tile m + 1 has landed
      phase();
      mma();
    };
    wait_vmcnt<YOUNG>();   // tile 0
    if (wm == 1) phase();  // group 1 starts one phase later
    if constexpr (NSTAGE == 4) {
      for (int m = 0; m < nk; m += 4) {
        tile_pp(m, st0, st3);
        if (m + 1 < nk) tile_pp(m + 1, st1, st0);
        if (m + 2 < nk) tile_pp(m + 2, st2, st1);
        if (m + 3 < nk) tile_pp(m + 3, st3, st2);
      }
    } else if constexpr (NSTAGE == 3) {
      for (int m = 0; m < nk; m += 3) {
        tile_pp(m, st0, st2);
        if (m + 1 < nk) tile_pp(m + 1, st1, st0);
        if (m + 2 < nk) tile_pp(m + 2, st2, st1);
      }
    } else {
      for (int m = 0; m < nk; m += 2) {
        tile_pp(m, st0, st1);
        if (m + 1 < nk) tile_pp(m + 1, st1, st0);
      }
    }
    if (wm == 0) phase();  // and group 0 ends one phase later
  } else {
  auto tile = [&](int kt, const char* cur, char* nxt) {
    constexpr int YOUNG = NLOAD * (NSTAGE - 2);
    __builtin_amdgcn_s_waitcnt(((YOUNG >> 4) << 14) | (0x7 << 4) | (0xF << 8) | (YOUNG & 15));
    __builtin_amdgcn_s_barrier();
    issue(min(kt + NSTAGE - 1, nk - 1), nxt);
    const char* As = cur;
    const char* Bs = cur + BK * ROWA;
    u32x4 af[KK][TM], bfr[KK][TN];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i) af[kk][i] = frag(As + kk * 16 * ROWA, ofa[i], ROWA);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[kk][j] = frag(Bs + kk * 16 * ROWB, ofb[j], ROWB);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(bfr[kk][j], af[kk][i], acc[i][j], (T*)nullptr);
    // per k-step: 2 (TM+TN) transposing reads spread over its TM*TN MFMAs
    constexpr int NR = 2 * (TM + TN), NM = TM * TN, PER = NM / NR > 0 ? NM / NR : 1;
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + 1 < KK) {
#pragma unroll
        for (int q = 0; q < NR; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (NM > NR * PER) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR * PER, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
      }
    }
  };
  if constexpr (NSTAGE == 4) {
    for (int kt = 0; kt < nk; kt += 4) {
      tile(kt, st0, st3);
      if (kt + 1 < nk) tile(kt + 1, st1, st0);
      if (kt + 2 < nk) tile(kt + 2, st2, st1);
      if (kt + 3 < nk) tile(kt + 3, st3, st2);
    }
  } else if constexpr (NSTAGE == 3) {
    for (int kt = 0; kt < nk; kt += 3) {
      tile(kt, st0, st2);
      if (kt + 1 < nk) tile(kt + 1, st1, st0);
      if (kt + 2 < nk) tile(kt + 2, st2, st1);
    }
  } else {
    for (int kt = 0; kt < nk; kt += 2) {
      tile(kt, st0, st1);
      if (kt + 1 < nk) tile(kt + 1, st1, st0);
    }
  }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  constexpr int SLAB = 32 * (WN + 4) * (int)sizeof(float);
  constexpr int PERST = STAGE / SLAB;  // slabs per stage
  static_assert(PERST >= 1 && (NW + PERST - 1) / PERST <= NSTAGE, "epilogue slabs must fit the stages");
  float* slab = reinterpret_cast<float*>(stage(wave / PERST) + (wave % PERST) * SLAB);
  GemmArgs ea = args;
  ea.zslice = split;
  Epilogue<T, E>::template run<TM, TN, WN>(ea, acc, slab, m0 + wm * WM, n0 + wn * WN, lane);
}

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
      load4_nt(P + (int64_t)z * M * N + e, x);
      for (int r = 0; r < 4; ++r) s[r] += x[r];
    }
    float* gp = G + (int64_t)m * ldg + n;
    if (accumulate) {
      float x[4];
      load4_nt(gp, x);
      for (int r = 0; r < 4; ++r) s[r] += x[r];
    }
    store4_nt(gp, s);
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
  // tile: 1 = 256x256, 2 = 128x128, 3 = 64x64 (0 = by shape)
  if constexpr (E == Epi::LMHead) {
    // one 128-column partial per wave column => BN = 256
    int tile = a.tile;
    if (tile == 0) tile = (int64_t)((a.M + 255) / 256) * (a.N / 256) >= 256 ? 1 : 3;
    if (tile == 1) return launch_tile<T, 256, 256, AK, BKc, E>(a, s);
    return launch_tile<T, 64, 256, AK, BKc, E>(a, s);
  } else {
    const int64_t t256 = (int64_t)((a.M + 255) / 256) * ((a.N + 255) / 256) * a.splits;
    const int64_t t128 = (int64_t)((a.M + 127) / 128) * ((a.N + 127) / 128) * a.splits;
    int tile = a.tile;
    if (tile == 0) tile = (t256 >= 512 && a.N % 256 == 0) ? 1 : (t128 >= 256 ? 2 : 3);
    if (tile == 1) return launch_tile<T, 256, 256, AK, BKc, E>(a, s);
    if (tile == 2) return launch_tile<T, 128, 128, AK, BKc, E>(a, s);
    return launch_tile<T, 64, 64, AK, BKc, E>(a, s);
  }
}

template <int BM, int BN, int NSTAGE, int OCC, Epi E, int NW = 4, int BK = 32, int ES = 2, bool PP = false>
hipError_t launch_nt_lds(const GemmArgs& a, hipStream_t s) {
  if (a.K % BK != 0) return hipErrorInvalidValue;
  const int splits = E == Epi::GradF32 ? a.splits : 1;
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  GemmArgs g = a;
  g.splits = splits;
  hipLaunchKernelGGL((gemm_nt_lds_kernel<BM, BN, NSTAGE, OCC, E, NW, BK, ES, PP>), dim3(tiles * splits * a.batch),
                     dim3(NW * 64), 0, s, g);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || splits <= 1) return err;
  const int64_t total4 = (int64_t)a.M * a.N / 4;
  const int blocks = (int)std::min<int64_t>((total4 + 255) / 256, 4096);
  hipLaunchKernelGGL(splitk_reduce, dim3(blocks), dim3(256), 0, s, a.split_buf, splits, a.M, a.N,
                     reinterpret_cast<float*>(a.C), a.ldc, a.accumulate);
  return hipGetLastError();
}


template <int BM, int BN, int NSTAGE, int OCC, Epi E, int NW = 4, int BK = 32, bool PP = false>
hipError_t launch_tn_lds(const GemmArgs& a, hipStream_t s) {
  // split-K slices are whole K tiles and K itself a whole number of them
  if (a.K % BK != 0) return hipErrorInvalidValue;
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_tn_lds_kernel<BM, BN, NSTAGE, OCC, E, NW, BK, PP>), dim3(tiles * a.splits), dim3(NW * 64), 0,
                     s, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.splits <= 1) return err;
  const int64_t total4 = (int64_t)a.M * a.N / 4;
  const int blocks = (int)std::min<int64_t>((total4 + 255) / 256, 4096);
  hipLaunchKernelGGL(splitk_reduce, dim3(blocks), dim3(256), 0, s, a.split_buf, a.splits, a.M, a.N,
                     reinterpret_cast<float*>(a.C), a.ldc, a.accumulate);
  return hipGetLastError();
}

template <Epi E>
hipError_t launch_nt_lds_tile(const GemmArgs& a, hipStream_t s) {
  const int64_t t256 = (int64_t)((a.M + 255) / 256) * ((a.N + 255) / 256) * a.batch;
  // tile: 1 = 256x256 (8 waves, two per SIMD; 64-wide K tiles, with the
  // ping-pong main loop, when K allows),
  // 2 = 256x128 (4 waves, two CTAs per CU), 3 = 128x128. By shape: 256x256
  // when there are at least two tiles per CU, else 128x128.
  int tile = a.tile;
  if (tile == 0) tile = (t256 >= 512 && a.N % 256 == 0) ? 1 : 3;
  if constexpr (E == Epi::LMHead) {  // exp-sum partials per 64 columns: BN a multiple of 128
    if (tile == 1 && a.K % 64 == 0) return launch_nt_lds<256, 256, 2, 1, E, 8, 64, 2, true>(a, s);
    if (tile == 1) return launch_nt_lds<256, 256, 4, 1, E>(a, s);
    if (tile == 2) return launch_nt_lds<256, 128, 3, 2, E>(a, s);
    return launch_nt_lds<128, 256, 4, 1, E>(a, s);
  } else {
    if (tile == 1 && a.K % 64 == 0) return launch_nt_lds<256, 256, 2, 1, E, 8, 64, 2, true>(a, s);
    if (tile == 1) return launch_nt_lds<256, 256, 4, 1, E, 8>(a, s);
    if (tile == 2) return launch_nt_lds<256, 128, 3, 2, E>(a, s);
    return launch_nt_lds<128, 128, 4, 1, E>(a, s);
  }
}

// fp8 operands: the bf16 kernels' byte tiles (BK doubles in elements).
// tile: 1 = 256x256 (8 waves, 128-byte rows), 2 = 256x128 (two CTAs per CU),
// 3 = 128x128; by shape 256x256 when that gives two tiles per CU (split-K
// slices counted), else 128x128.
template <Epi E>
hipError_t launch_nt_fp8_tile(const GemmArgs& a, hipStream_t s) {
  const int splits = E == Epi::GradF32 ? a.splits : 1;
  const int64_t t256 = (int64_t)((a.M + 255) / 256) * ((a.N + 255) / 256) * splits;
  int tile = a.tile;
  if (tile == 0) tile = (t256 >= 512 && a.N % 256 == 0) ? 1 : 3;
  if (tile == 1) return launch_nt_lds<256, 256, 2, 1, E, 8, 128, 1, true>(a, s);
  if (tile == 2) return launch_nt_lds<256, 128, 3, 2, E, 4, 64, 1>(a, s);
  return launch_nt_lds<128, 128, 4, 1, E, 4, 64, 1>(a, s);
}

hipError_t launch_fp8(Epi epi, const GemmArgs& a, hipStream_t s) {
  if (!a.a_kcontig || !a.b_kcontig || a.K % 128 != 0 || !a.amax_a || !a.amax_b) return hipErrorInvalidValue;
  switch (epi) {
    case Epi::Store: return launch_nt_fp8_tile<Epi::Store>(a, s);
    case Epi::Residual: return launch_nt_fp8_tile<Epi::Residual>(a, s);
    case Epi::Relu2: return launch_nt_fp8_tile<Epi::Relu2>(a, s);
    case Epi::Relu2Bwd: return launch_nt_fp8_tile<Epi::Relu2Bwd>(a, s);
    case Epi::GradF32: return launch_nt_fp8_tile<Epi::GradF32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_typed(Epi epi, const GemmArgs& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (a.a_kcontig && a.b_kcontig && a.K % 32 == 0) {
      switch (epi) {
        case Epi::Store: return launch_nt_lds_tile<Epi::Store>(a, s);
        case Epi::Residual: return launch_nt_lds_tile<Epi::Residual>(a, s);
        case Epi::Relu2: return launch_nt_lds_tile<Epi::Relu2>(a, s);
        case Epi::LMHead: return launch_nt_lds_tile<Epi::LMHead>(a, s);
        case Epi::Relu2Bwd: return launch_nt_lds_tile<Epi::Relu2Bwd>(a, s);
        default: break;
      }
    }
  }
  if constexpr (sizeof(T) == 2) {
    if (!a.a_kcontig && !a.b_kcontig && epi == Epi::GradF32 && a.K % 32 == 0 && a.M % 128 == 0 &&
        a.N % 128 == 0) {
      // tile: 1 = 256x256, 2 = 128x128 (0 = 256x256 when that fills the chip)
      const int64_t t256 = (int64_t)((a.M + 255) / 256) * ((a.N + 255) / 256) * a.splits;
      int tile = a.tile;
      if (tile == 0) tile = (t256 >= 256 && a.M % 256 == 0 && a.N % 256 == 0) ? 1 : 2;
      if (tile == 1 && a.M % 256 == 0 && a.N % 256 == 0)
        return launch_tn_lds<256, 256, 4, 1, Epi::GradF32, 8, 32, true>(a, s);
      return launch_tn_lds<128, 128, 4, 1, Epi::GradF32>(a, s);
    }
  }
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
      if (nt) return launch_layout<T, true, true, Epi::Relu2Bwd>(a, s);
      break;
    case Epi::GradF32:
      if (tn) return launch_layout<T, false, false, Epi::GradF32>(a, s);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Split-K partials for callers that cannot allocate (gpt_fp8_matmul_noalloc):
// a fixed device array, one copy per GPU for the life of the process. Host
// code never passes the array's name to a kernel: each device's address is
// looked up once, with that device current, and cached.
namespace {
__device__ __align__(256) float scratch[kNoAllocScratchFloats];
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(float** out) {
  *out = nullptr;
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_gemm(int dtype, Epi epi, const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
  // epilogues address a wave's output tile (at most 256 rows) with 32-bit
  // element offsets
  if (a.ldc > (1 << 22) || a.ldc2 > (1 << 22) || a.N > (1 << 22)) return hipErrorInvalidValue;
  if (a.batch > 1) {
    if ((epi != Epi::Store && epi != Epi::Residual) || a.splits != 1) return hipErrorInvalidValue;
    // one launch on the bf16 direct-to-LDS kernel; any other path, product by product
    if (!(dtype == 1 && a.a_kcontig && a.b_kcontig && a.K % 64 == 0 && a.N % 4 == 0)) {
      for (int j = 0; j < a.batch; ++j) {
        GemmArgs g = a;
        g.batch = 1;
        g.A = reinterpret_cast<const char*>(a.A) + j * a.stride_a;
        g.B = reinterpret_cast<const char*>(a.B) + j * a.stride_b;
        g.C = reinterpret_cast<char*>(a.C) + j * a.stride_c;
        if (hipError_t e = launch_gemm(dtype, epi, g, s); e != hipSuccess) return e;
      }
      return hipSuccess;
    }
  }
  // Shapes the tile loaders assume: a k-contiguous operand has K a multiple of
  // the 128-byte K tile; an mn-contiguous operand has its rows in whole
  // 16-byte vectors; the epilogue writes groups of 4 columns.
  if (a.splits < 1 || (a.splits > 1 && a.split_buf == nullptr)) return hipErrorInvalidValue;
  if (dtype == 2) return a.N % 4 != 0 ? hipErrorInvalidValue : launch_fp8(epi, a, s);
  const int bk = dtype == 1 ? 64 : 32;
  if ((a.a_kcontig || a.b_kcontig) && a.K % bk != 0) return hipErrorInvalidValue;
  if ((!a.a_kcontig && a.M % 8 != 0) || (!a.b_kcontig && a.N % 8 != 0) || a.N % 4 != 0) return hipErrorInvalidValue;
  if (epi == Epi::LMHead && a.N % 256 != 0) return hipErrorInvalidValue;
  return dtype == 1 ? launch_typed<bf16>(epi, a, s) : launch_typed<float>(epi, a, s);
}

}  // namespace gk
