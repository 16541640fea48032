// Device-side building blocks for the gfx950 attention kernels: vector types,
// MFMA wrappers, 16-byte loads/stores, bf16 packing and cross-half reductions.
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16): lane l holds row l%32, k-slots 8*(l/32) .. +7
//   B (16 x 32): lane l holds column l%32, k-slots 8*(l/32) .. +7
//   D (32 x 32): lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
// Only the pairing of A's and B's k-slots matters for a product, so a kernel
// may assign any key/feature order to the slots as long as both operands
// agree.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st8(void* p, const u32x2& v) { *reinterpret_cast<u32x2*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Round two floats to bf16 (nearest-even; one v_cvt_pk_bf16_f32) packed low|high.
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

// Value of the other half-wave's lane (l ^ 32) combined with this lane's value.
__device__ __forceinline__ float half_swap_max(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)p[0]), __builtin_bit_cast(float, (unsigned)p[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Low / high bf16 halves of two words, packed (word a -> low half, word b -> high half).
__device__ __forceinline__ unsigned lo_lo(unsigned a, unsigned b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ unsigned hi_hi(unsigned a, unsigned b) { return (a >> 16) | (b & 0xffff0000u); }

}  // namespace fa
