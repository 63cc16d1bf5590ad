// Shared device helpers for the gfx950 kernels of libmla.
#pragma once
#include <type_traits>
#include <utility>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// Calls f(std::integral_constant<int, I>{}) for I = 0 .. N-1: loop indices that
// are compile-time constants, so register arrays are never indexed at run time.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define MLA_LOG2E 1.4426950408889634f
#define MLA_LN2 0.6931471805599453f

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (the hardware conversion; NaN
// stays NaN).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint16_t float_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return (uint32_t)float_to_f16_bits(lo) | ((uint32_t)float_to_f16_bits(hi) << 16);
}

// two floats to packed bf16 (one v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Load element i of a tensor stored as bf16 or fp32, as float.
template <mla_dtype DT>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (DT == MLA_BF16) {
    return bf16_bits_to_float(static_cast<const uint16_t*>(p)[i]);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

template <mla_dtype DT>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float v) {
  if constexpr (DT == MLA_BF16) {
    static_cast<uint16_t*>(p)[i] = float_to_bf16_bits(v);
  } else {
    static_cast<float*>(p)[i] = v;
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max of two / three floats in one instruction: fmaxf would first quiet each
// input (an extra instruction per operand); the scores here are never
// signalling NaNs.
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Wave-wide (64 lanes) reductions through cross-lane moves.
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Reduce a value with the one held by lane l ^ 32.  permlane32_swap returns,
// in its two results, the lane's own value and its partner's (in an order
// that depends on the half), so a symmetric operation over both is exact.
__device__ __forceinline__ float half_pair_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_pair_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- direct global->LDS copies and wait counters (gfx950) ------------------
typedef int i32x4_t __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

// Buffer load of `size` bytes per lane straight into LDS at lds + size * lane
// (LLVM intrinsic llvm.amdgcn.raw.buffer.load.lds).  The byte address is
// voffset + soffset + offset from the resource base; addresses at or past the
// resource's byte range read as zero.
extern "C" __device__ void mla_raw_buffer_load_lds(i32x4_t rsrc, LDS_AS void* lds, int size, int voffset,
                                                   int soffset, int offset,
                                                   int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// The same 16-byte buffer->LDS copy issued as inline assembly: M0 holds the
// LDS address of lane 0's destination (lane l writes at M0 + 16 l); the byte
// address is voffset (per lane) + soffset (uniform) from the resource base.  The
// compiler does not see these as LDS writes, so it adds no waits of its own
// before later LDS reads (it would otherwise wait for every copy in flight
// before reading any LDS array it cannot prove disjoint); the caller orders
// them with s_waitcnt vmcnt and a workgroup barrier.  Copies past the
// resource's byte range read as zero.
__device__ __forceinline__ void lds_dma_b128(i32x4_t rsrc, uint32_t lds_addr, int voffset, int soffset = 0) {
  int saved;    // M0 is restored, so the compiler's own uses of it are unaffected
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voffset), "s"(rsrc), "s"(soffset)
      : "memory");
}

// The same copy with the non-temporal hint (data read once: it should not
// displace what the CU's neighbours read again from L2).
__device__ __forceinline__ void lds_dma_b128_nt(i32x4_t rsrc, uint32_t lds_addr, int voffset, int soffset = 0) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen nt lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voffset), "s"(rsrc), "s"(soffset)
      : "memory");
}

// Buffer resource for `bytes` bytes at `base` (gfx9 data-format word).
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
  uint64_t p = reinterpret_cast<uint64_t>(base);
  i32x4_t r = {(int)(uint32_t)p, (int)(uint32_t)(p >> 32), (int)bytes, 0x00020000};
  return r;
}

// The same resource forced into scalar registers (for values the compiler
// cannot prove uniform; the caller guarantees they are).
__device__ __forceinline__ i32x4_t make_rsrc_uniform(const void* base, uint32_t bytes) {
  i32x4_t r = make_rsrc(base, bytes);
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(r[i]);
  return r;
}

// Orders the LDS accesses of the lanes of one wave: the wave's LDS operations
// issued so far are complete, and the compiler moves no memory access across.
// Needed where a lane reads what another lane of its wave wrote: without it the
// compiler may hoist a lane's read above that lane's own, non-overlapping
// writes, and the read then misses another lane's write.
__device__ __forceinline__ void lds_wave_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// s_waitcnt vmcnt(n), leaving the other counters unconstrained
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
