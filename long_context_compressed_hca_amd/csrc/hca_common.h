// hca_common.h - device-side building blocks shared by the HCA kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "hca_kernels.h"

namespace hca {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> packed bfloat16 pair (lo in bits 0..15), nearest even: one
// v_cvt_pk_bf16_f32 (the same rounding as f32_to_bf16_bits for every
// non-NaN input; a NaN stays a NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  typedef __attribute__((ext_vector_type(2))) float f32x2_t;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// ---------------------------------------------------------------- LDS DMA
// global -> LDS copy of 16 bytes per lane: lane i's 16 bytes land at
// lds_row + 16*i, whatever global address lane i supplies.  lds_row must be
// the same for every lane of the wave.
__device__ __forceinline__ void dma16(const void* gsrc, lds_void* lds_row) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_row, 16, 0, 0);
}

// Buffer descriptor of `bytes` bytes at `base` (raw, stride 0, 32-bit data
// format, the gfx9 default for untyped buffer access).  Loads at offsets
// >= bytes are range checked by the hardware and return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// buffer -> LDS copy of 16 bytes per lane through a descriptor: lane i's 16
// bytes (from byte offset voff of the buffer) land at lds_row + 16*i.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, int voff, lds_void* lds_row) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_row, 16, voff, 0, 0, 0);
}

// buffer store of 16 bytes per lane at byte offset voff of the buffer; stores at
// offsets >= the descriptor's size are dropped by the hardware range check.
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
__device__ __forceinline__ void store16_buf(__amdgpu_buffer_rsrc_t r, int voff, u32x4 data) {
  __builtin_amdgcn_raw_buffer_store_b128(data, r, voff, 0, 0);
}

// s_waitcnt vmcnt(0): wait for this wave's outstanding vector-memory loads,
// including LDS DMA (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; expcnt and lgkmcnt left at their "no wait" maxima).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier without the memory fence of __syncthreads() (which waits
// for every outstanding vector-memory operation, in-flight LDS copies
// included).  The caller orders memory itself: each wave waits (vmcnt) for
// the copies the other waves will read, and LDS reads before the barrier are
// consumed (lgkmcnt waits) before it.  The asm statements keep the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace hca
