// Device helpers shared by the gfx950 kernels: vector types, bf16 conversion,
// MFMA wrappers and wavefront shuffles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rpkv_internal.h"

namespace rpkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// MFMA operand layouts (checked on gfx950 hardware):
//  32x32x16: A[m][k] in lane m + 32*(k/8), element k%8; B[k][n] in lane
//            n + 32*(k/8), element k%8; C[m][n] in lane n + 32*((m/4)%2),
//            element (m/8)*4 + m%4.
//  16x16x32: A[m][k] in lane m + 16*(k/8), element k%8; B[k][n] in lane
//            n + 16*(k/8), element k%8; C[m][n] in lane n + 16*(m/4),
//            element m%4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16 with round-to-nearest-even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 2^x and log2(x) on the hardware transcendental unit.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// The two halves of a wavefront exchanged (lane l gets lane l ^ 32) and
// combined: gfx950's v_permlane32_swap, a VALU instruction (no LDS round
// trip).  The swap of v with itself leaves {v[l % 32], v[l % 32 + 32]} in
// the pair on every lane.
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int32_t clamp_page(int32_t pg, int64_t num_pages) {
  return pg < 0 ? 0 : (pg >= num_pages ? (int32_t)(num_pages - 1) : pg);
}

constexpr float kNegInf = -__builtin_inff();

}  // namespace rpkv
