// Device-side building blocks shared by the MSA kernels (gfx950 / CDNA4).
//
// Matrix work uses the 32x32 MFMA family.  A "k-slice" is 16 contraction
// slots; in every operand fragment lane l holds 8 of them (element j), with
// the same (l >> 5, j) -> slot map for the A and the B operand, so any
// consistent slot permutation computes the same contraction.
//
//   A fragment (M x 16): lane l -> row  m = l & 31, 8 slots
//   B fragment (16 x N): lane l -> col  n = l & 31, 8 slots
//   accumulator (32x32 fp32, 16 per lane): lane l -> col n = l & 31,
//       element i -> row ((i >> 2) << 3) + ((l >> 5) << 2) + (i & 3)
//
// "Natural" slots: element j of lane l is slot ((l >> 5) << 3) + j, i.e. 8
// contiguous elements of a row of the operand in memory.
// "Accumulator" slots: element j of lane l in k-slice s of a 32-row
// accumulator tile is row  s*16 + ((j >> 2) << 3) + ((l >> 5) << 2) + (j & 3),
// so the accumulator's elements [8s, 8s+8) are directly a fragment whose
// slots are the accumulator's rows.  The operand paired with it is read from a
// row-major LDS tile with lds_col_frag() (LDS transpose reads for bf16).
//
// bf16 tiles use v_mfma_f32_32x32x16_bf16.  fp32 tiles use eight
// v_mfma_f32_32x32x2f32 steps per k-slice (step j contracts slot pair j).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace msa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float NEG_BIG = -1.0e30f;   // finite "minus infinity" for running maxima

template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; typedef bf16x4 half; };
template <> struct Frag<float> { typedef f32x8 type; typedef f32x4 half; };
template <typename T> using frag_t = typename Frag<T>::type;
template <typename T> using half_t = typename Frag<T>::half;

__device__ __forceinline__ void mma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// 8 contiguous elements (16-byte aligned for bf16, 16-byte aligned for fp32).
__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 ld8(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f32x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) { r[j] = a[j]; r[j + 4] = b[j]; }
  return r;
}
// Two runs of 4 contiguous elements -> one fragment (accumulator-slot reads).
__device__ __forceinline__ bf16x8 ld4x2(const bf16* p0, const bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) { r[j] = a[j]; r[j + 4] = b[j]; }
  return r;
}
__device__ __forceinline__ f32x8 ld4x2(const float* p0, const float* p1) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p0);
  f32x4 b = *reinterpret_cast<const f32x4*>(p1);
  f32x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) { r[j] = a[j]; r[j + 4] = b[j]; }
  return r;
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

// Elements [8s, 8s+8) of an accumulator as an operand fragment (accumulator slots).
template <typename T>
__device__ __forceinline__ frag_t<T> acc_frag(const f32x16& acc, int s) {
  frag_t<T> r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = from_f32<T>(acc[s * 8 + j]);
  return r;
}

// One gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of
// 16 lanes, every lane supplies the address of 4 consecutive 16-bit values;
// lane i of the group receives element (i % 4) of the values supplied by
// lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12, in that order.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 lds_tr4(const bf16* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(const_cast<bf16*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// LDS reads at a 32-bit LDS byte address plus a compile-time offset.  The
// base is meant to come from lds_base_add(): an add the compiler cannot take
// apart, so that every read of a stage reuses the same base register and the
// constant lands in the instruction's offset field.
__device__ __forceinline__ uint32_t lds_base_add(uint32_t uniform_base, uint32_t lane_off) {
  uint32_t r;
  asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(uniform_base), "v"(lane_off));
  return r;
}
// a ^ C in a vector register, opaque to the compiler so that it is formed
// where it is used instead of being hoisted out of the stage loop (where it
// would hold a register for the whole kernel).
template <uint32_t C>
__device__ __forceinline__ uint32_t xr(uint32_t a) {
  if constexpr (C == 0) {
    return a;
  } else {
    uint32_t r;
    asm volatile("v_xor_b32 %0, %2, %1" : "=v"(r) : "v"(a), "i"(C));
    return r;
  }
}
// v if (x + C) < w as unsigned integers, else 0.  The causal / document mask
// of an accumulator element with constant row offset C: x = (row of element
// 0) - lo and w = hi - lo, so the test is lo <= row < hi.  One asm block per
// element keeps the compiler from hoisting sixteen compare masks into scalar
// registers ahead of the interleaved softmax.
template <uint32_t C>
__device__ __forceinline__ float keep_if(float v, uint32_t x, uint32_t w) {
  float r;
  uint32_t t;
  asm volatile("v_add_u32 %1, %3, %4\n\tv_cmp_lt_u32 vcc, %1, %5\n\tv_cndmask_b32 %0, 0, %2, vcc"
               : "=v"(r), "=&v"(t)
               : "v"(v), "i"(C), "v"(x), "v"(w)
               : "vcc");
  return r;
}
typedef __attribute__((address_space(3))) const unsigned char lds_u8;
template <int OFF>
__device__ __forceinline__ bf16x8 lds_ld8(uint32_t base) {
  typedef __attribute__((address_space(3))) const bf16x8 lds_v8;
  return *reinterpret_cast<lds_v8*>(reinterpret_cast<lds_u8*>((uintptr_t)base) + OFF);
}
template <int OFF>
__device__ __forceinline__ bf16x4 lds_tr4_at(uint32_t base) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(reinterpret_cast<lds_u8*>((uintptr_t)base) + OFF));
  return __builtin_bit_cast(bf16x4, v);
}
// Two transpose reads (the rows of an accumulator-slot fragment and the rows
// 8 further down) joined into one fragment.
template <int OFF>
__device__ __forceinline__ bf16x8 tr_pair_at(uint32_t a, uint32_t b) {
  const bf16x4 x = lds_tr4_at<OFF>(a), y = lds_tr4_at<OFF>(b);
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) { r[j] = x[j]; r[j + 4] = y[j]; }
  return r;
}

// Operand fragment in accumulator slots read from a row-major LDS tile X
// (ld elements per row) whose rows are the contraction index: lane l gets
// column n0 + (l & 31) and rows k0 + ((j >> 2) << 3) + ((l >> 5) << 2) + (j & 3)
// for element j.  It pairs with acc_frag() of an accumulator tile whose rows
// are the same contraction index.  bf16: two transpose reads, where source
// lane s of group g reads row k0 + 4 (l >> 5) + (s >> 2) (and that + 8),
// columns n0 + 16 (g & 1) + 4 (s & 3) .. + 3.  fp32: eight scalar reads.
template <typename T>
__device__ __forceinline__ frag_t<T> lds_col_frag(const T* X, int ld, int k0, int n0, int lane);
template <>
__device__ __forceinline__ bf16x8 lds_col_frag<bf16>(const bf16* X, int ld, int k0, int n0, int lane) {
  const int s = lane & 15, g = lane >> 4, hi = lane >> 5;
  const bf16* p = X + (k0 + hi * 4 + (s >> 2)) * ld + n0 + 16 * (g & 1) + 4 * (s & 3);
  const bf16x4 a = lds_tr4(p), b = lds_tr4(p + 8 * ld);
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) { r[j] = a[j]; r[j + 4] = b[j]; }
  return r;
}
template <>
__device__ __forceinline__ f32x8 lds_col_frag<float>(const float* X, int ld, int k0, int n0, int lane) {
  const int c = n0 + (lane & 31), hi = lane >> 5;
  f32x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = X[(k0 + ((j >> 2) << 3) + hi * 4 + (j & 3)) * ld + c];
  return r;
}

// ---------------------------------------------------------------------------
// Row-major LDS tiles without padding whose 16-byte chunks are XOR-swizzled by
// row.  gfx950's LDS has 64 four-byte banks and serves 16 lanes per cycle for
// 16-byte reads and 32 lanes per cycle for 8-byte reads; these swizzles make
// both access patterns used here conflict-free: a 16-byte read of the same
// chunk from 16 consecutive rows, and the transpose reads of lds_col_frag
// (4 consecutive rows x 32 bytes per 16-lane group).
//   16 chunks per row (256 B): chunk ^ ((r & 3) << 2 | (r >> 2) & 3)
//    8 chunks per row (128 B): chunk ^ (((r >> 1) & 1) << 2 | (r >> 2) & 3)
//   fewer chunks: no swizzle (only the small fp32 / d = 64 tiles)
template <int CPR>
__device__ __forceinline__ int swz(int r, int chunk) {
  if constexpr (CPR >= 16) return chunk ^ (((r & 3) << 2) | ((r >> 2) & 3));
  else if constexpr (CPR == 8) return chunk ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  else return chunk;
}
template <typename T, int COLS>
struct Tile {
  static constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  static constexpr int CPR = COLS / EPC;            // chunks per row
  static constexpr int ELEMS_PER_ROW = COLS;
  __device__ static __forceinline__ int off(int r, int c) {
    return r * COLS + swz<CPR>(r, c / EPC) * EPC + (c % EPC);
  }
  // 8 consecutive elements of row r starting at column c (c % 8 == 0)
  __device__ static __forceinline__ frag_t<T> row8(const T* X, int r, int c);
  // transposed fragment: see lds_col_frag
  __device__ static __forceinline__ frag_t<T> col(const T* X, int k0, int n0, int lane);
};
template <typename T, int COLS>
__device__ __forceinline__ frag_t<T> Tile<T, COLS>::row8(const T* X, int r, int c) {
  if constexpr (sizeof(T) == 2) {
    return ld8(X + off(r, c));
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(X + off(r, c));
    const f32x4 b = *reinterpret_cast<const f32x4*>(X + off(r, c + 4));
    f32x8 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) { v[j] = a[j]; v[j + 4] = b[j]; }
    return v;
  }
}
template <typename T, int COLS>
__device__ __forceinline__ frag_t<T> Tile<T, COLS>::col(const T* X, int k0, int n0, int lane) {
  if constexpr (sizeof(T) == 2) {
    const int s = lane & 15, g = lane >> 4, hi = lane >> 5;
    const int r = k0 + hi * 4 + (s >> 2);
    const int c = n0 + 16 * (g & 1) + 4 * (s & 3);
    const bf16x4 a = lds_tr4(X + off(r, c)), b = lds_tr4(X + off(r + 8, c));
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) { v[j] = a[j]; v[j + 4] = b[j]; }
    return v;
  } else {
    const int c = n0 + (lane & 31), hi = lane >> 5;
    f32x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = X[off(k0 + ((j >> 2) << 3) + hi * 4 + (j & 3), c)];
    return v;
  }
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Asynchronous global -> LDS copies (gfx950 global_load_lds).  Lane l's bytes
// land at LDS byte address lds + l * size; lds must be wave-uniform.  The
// copies are counted by vmcnt like other vector loads, so a stage is known to
// have landed once vmcnt has dropped to the number of loads issued after it;
// the callers wait for that explicitly (wait_vmcnt) and then barrier.
//
// The copies are issued from inline assembly on purpose.  Through the
// compiler builtin, a workgroup barrier waits for every copy in flight (the
// copies count as LDS stores), which serialises the ring of stages.  Hidden
// from the compiler, the copies can only make its own vmcnt waits more
// conservative: vector loads retire in order, so loads it does not know of
// only delay the point where its counts are reached.  M0 carries the LDS
// address; it is saved and restored around the copy, with the one wait state
// the hardware needs between writing M0 and the copy reading it.  The
// "memory" clobber keeps LDS reads of earlier stages from moving past a copy.
__device__ __forceinline__ uint32_t lds_offset(const void* shared_array) {
  // only for pointers taken directly from a __shared__ array
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)shared_array;
}
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\ts_nop 0\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds))
      : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "global_load_lds_dword %1, off\n\ts_nop 0\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds))
      : "memory");
}
typedef int i32x4 __attribute__((ext_vector_type(4)));
// Buffer descriptor of a raw byte range (gfx9 layout: base, stride 0,
// num_records in bytes, 32-bit data format).  Every field is wave-uniform.
__device__ __forceinline__ i32x4 make_srd(const void* base, uint32_t nbytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)nbytes);
  r[3] = 0x00020000;
  return r;
}

// Buffer -> LDS copies (lane l's bytes land at LDS byte address lds + l * size;
// lds must be wave-uniform).  Issued from inline assembly for the same reason
// as the global -> LDS copies elsewhere: hidden from the compiler, a barrier
// does not wait for them; the kernel waits with explicit vmcnt counts.  M0 is
// saved and restored around the copy.
__device__ __forceinline__ void bdma16(const i32x4& srd, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_nop 0\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(srd), "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds))
      : "memory");
}
__device__ __forceinline__ void bdma4(const i32x4& srd, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds\n\ts_nop 0\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(srd), "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds))
      : "memory");
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left at their maxima; gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Row of accumulator element i for lane l (see the layout note above).
__device__ __forceinline__ int acc_row(int i, int lane) {
  return ((i >> 2) << 3) + ((lane >> 5) << 2) + (i & 3);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Fill kernel (used instead of memset so every clear is an ordinary launch).
__global__ void fill_i32_kernel(int32_t* p, int32_t v, int64_t n);

}  // namespace msa
