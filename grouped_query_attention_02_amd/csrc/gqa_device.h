// gqa_device.h - gfx950 device helpers shared by the GQA kernels (internal).
//
// MFMA operand layouts used throughout (wave64, v_mfma_f32_32x32x16_bf16):
//   A (32 x 16): lane l holds row (l % 32) and 8 consecutive k slots of half (l / 32).
//   B (16 x 32): lane l holds column (l % 32) and the same 8 k slots of half (l / 32).
//   C (32 x 32): lane l holds column (l % 32), rows 8*(r/4) + 4*(l/32) + (r%4), r = 0..15.
// Because A and B map k slots identically, any assignment of the contraction index
// to (half, slot) gives the same product as long as both operands use it; the
// kernels exploit that to feed the score accumulators straight into the next
// product without a trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(const bf16x8& a, const bf16x8& b,
                                                     const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32_32x32x2(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Eight fp32 -> eight bf16 in one MFMA operand.
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3, float a4,
                                              float a5, float a6, float a7) {
  u32x4 u;
  u[0] = pack_bf16x2(a0, a1);
  u[1] = pack_bf16x2(a2, a3);
  u[2] = pack_bf16x2(a4, a5);
  u[3] = pack_bf16x2(a6, a7);
  return as_bf16x8(u);
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane (l ^ 32).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// max / sum of x over the lane pair (l, l ^ 32), with one v_permlane32_swap.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-uniform "any lane true".
__device__ __forceinline__ bool wave_any(bool p) { return __any(p); }

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ldg8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

__device__ __forceinline__ u32x4 zero_u32x4() {
  u32x4 z = {0u, 0u, 0u, 0u};
  return z;
}

}  // namespace gqa
