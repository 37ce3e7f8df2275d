// Device-side helpers shared by the gfx950 kernels: storage types, 16-byte
// vector loads/stores, MFMA wrappers. Written for CDNA4 (wave64) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define DEV __device__ __forceinline__

constexpr int WAVE = 64;

// ----------------------------------------------------------------- scalars --

DEV float to_f32(float x) { return x; }
DEV float to_f32(bf16 x) { return (float)x; }
template <typename T> DEV T from_f32(float x);
template <> DEV float from_f32<float>(float x) { return x; }
template <> DEV bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE (v_cvt_pk_bf16_f32)

// ------------------------------------------------------ 16-byte vector I/O --

DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
DEV void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
DEV u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
DEV void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// Elements of T per 16 bytes.
template <typename T> struct Vec;
template <> struct Vec<bf16> { static constexpr int N = 8; };
template <> struct Vec<float> { static constexpr int N = 4; };

// Load / store 8 consecutive elements as fp32.
DEV void load8(const bf16* p, float (&v)[8]) {
  u32x4 r = ld16(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(r[i] << 16);
    v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}
DEV void load8(const float* p, float (&v)[8]) {
  u32x4 a = ld16(p), b = ld16(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = __uint_as_float(a[i]); v[4 + i] = __uint_as_float(b[i]); }
}
// Two floats to a bf16 pair (RNE), lo in the low half: one v_cvt_pk_bf16_f32.
DEV uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
DEV void store8(bf16* p, const float (&v)[8]) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  st16(p, r);
}
DEV void store8(float* p, const float (&v)[8]) {
  u32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = __float_as_uint(v[i]); b[i] = __float_as_uint(v[4 + i]); }
  st16(p, a);
  st16(p + 4, b);
}
// 4 consecutive elements.
DEV void load4(const bf16* p, float (&v)[4]) {
  u32x2 r = ld8(p);
  v[0] = __uint_as_float(r[0] << 16); v[1] = __uint_as_float(r[0] & 0xffff0000u);
  v[2] = __uint_as_float(r[1] << 16); v[3] = __uint_as_float(r[1] & 0xffff0000u);
}
DEV void load4(const float* p, float (&v)[4]) {
  u32x4 r = ld16(p);
  for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(r[i]);
}
DEV void store4(bf16* p, const float (&v)[4]) {
  u32x2 r; r[0] = pack_bf16x2(v[0], v[1]); r[1] = pack_bf16x2(v[2], v[3]);
  st8(p, r);
}
DEV void store4(float* p, const float (&v)[4]) {
  u32x4 r; for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(v[i]);
  st16(p, r);
}

// Non-temporal (streaming) variants: for outputs and operands touched once,
// so that they do not evict data other workgroups still reuse from the L2
// (the GEMM operand panels).
DEV void st8_nt(void* p, u32x2 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p)); }
DEV void st16_nt(void* p, u32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p)); }
DEV u32x2 ld8_nt(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)); }
DEV u32x4 ld16_nt(const void* p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
DEV void store4_nt(bf16* p, const float (&v)[4]) {
  u32x2 r; r[0] = pack_bf16x2(v[0], v[1]); r[1] = pack_bf16x2(v[2], v[3]);
  st8_nt(p, r);
}
DEV void store4_nt(float* p, const float (&v)[4]) {
  u32x4 r; for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(v[i]);
  st16_nt(p, r);
}
DEV void load4_nt(const float* p, float (&v)[4]) {
  u32x4 r = ld16_nt(p);
  for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(r[i]);
}

// ---------------------------------------------------------- reductions -----

DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum over each row of 16 lanes (lanes 16k..16k+15), every lane of the row
// receiving the total: four DPP row rotations (by 8, 4, 2, 1), no LDS traffic.
// A fixed association order, so the result is reproducible.
DEV float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false));
  return v;
}
DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Folds the threads' running |max| of values a kernel stores as T into a
// float slot: the block's maximum, rounded to T (rounding is monotonic, so
// this is the maximum of the stored values), by one atomic max of the bit
// pattern per block (non-negative floats order like their bits; the slot
// starts at 0). Every thread of the block must call it (it has a barrier);
// at most 16 waves per block. Meant for kernels with few, long-running
// blocks: the atomics of many short blocks on one address serialise.
template <typename T>
DEV void amax_fold_block(float m, float* slot) {
  __shared__ float red[16];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) v = fmaxf(v, red[w]);
    if constexpr (sizeof(T) == 2) v = (float)(bf16)v;
    atomicMax(reinterpret_cast<unsigned*>(slot), __float_as_uint(v));
  }
}

// ------------------------------------------------------------- MFMA -------
// Lane layout (checked on gfx950): for the 32x32 shapes, lane l feeds row
// (l % 32) of the A operand and column (l % 32) of the B operand with the
// k-slice owned by lane group g = l / 32; the 16 accumulator values of lane l
// are C[blk*8 + g*4 + r][l % 32] at index blk*4 + r. Any fixed assignment of
// k values to (g, element) works as long as A and B use the same one.

// One 16-byte fragment per operand per lane: bf16 -> one 32x32x16 MFMA;
// fp32 -> four 32x32x2 MFMAs (one element each), i.e. 8 k per fragment pair.
DEV f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c, bf16*) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
DEV f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c, float*) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[j]), __uint_as_float(b[j]), c, 0, 0, 0);
  return c;
}

// fp8 (OCP e4m3) x fp8 -> fp32, 32x32x64: each operand is 32 bytes per lane,
// given as two 16-byte fragments (the k assignment is whatever the caller's
// fragment reads make it, the same for both operands). Format code 0 selects
// e4m3 for A and B; the E8M0 block scales are fixed at 2^0 (127).
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
DEV f32x16 mfma_fp8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x16 c) {
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Four floats to four e4m3 bytes (a in the lowest byte), round to nearest
// even. Finite magnitudes above 448 are not saturated by the conversion (it
// gives NaN past 464): callers clamp first.
DEV uint32_t pack_fp8x4(float a, float b, float c, float d) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)lo, true);
#else
  (void)a; (void)b; (void)c; (void)d;
  return 0u;
#endif
}

// ------------------------------------------------- buffer loads to LDS -----
// Buffer resource over [p, p + bytes) (raw, stride 0): loads at offsets past
// `bytes` return zero. Made wave-uniform (SGPRs) with readfirstlane; callers
// pass block-uniform values. `bytes` must be below 2^31.
DEV __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int bytes) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const int n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, 0x00020000);
}

// Direct-to-LDS buffer loads: lane L of the wave writes LDS bytes
// [lds + 16L, lds + 16L + 16) (resp. 4 bytes at lds + 4L); `lds` must be
// wave-uniform. The address-space cast only exists in the device pass.
DEV void lds_direct16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
#endif
}
DEV void lds_direct4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, 0, 0, 0);
#endif
}

// s_waitcnt on the vector-memory counter only: wait until at most n (< 64)
// vector loads of this wave are outstanding (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).
template <int N>
DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (0x7 << 4) | (0xF << 8) | (N & 15));
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane j names 8 bytes (4 consecutive 16-bit values) at its address; lane i
// receives value (i % 4) of lane 4e + i/4 as its element e, e = 0..3. Pointing
// lane 4e + c at row r_e, columns [col0 + 4c, col0 + 4c + 4) of a row-major
// tile therefore hands lane i column col0 + i of rows r_0..r_3.
DEV u32x2 ld_tr16(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
#else
  (void)p;
  return u32x2{0, 0};
#endif
}

// -------------------------------------------------------- device flag ------
// Bit 0: a token id outside [0, V). Set with a plain vector store (no atomics
// needed: every writer stores the same bit pattern).
enum { FLAG_BAD_TOKEN = 1 };
