// Device-side building blocks shared by the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

constexpr int WAVE = 64;

// ---------------------------------------------------------------------------------------
// order-preserving 32-bit key of an fp32 score: a > b  <=>  key(a) > key(b) as unsigned.
// -0.0 is mapped to +0.0 first so the two zeros tie (they compare equal as floats).
// Finite scores map to keys >= 0x00800000, so a threshold of 0 admits every score.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b << 1) == 0u) b = 0u;  // +-0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---------------------------------------------------------------------------------------
// wave64 helpers
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// number of set bits of `mask` in lanes below the calling lane
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    uint32_t t = __shfl_up(v, off, WAVE);
    if (l >= off) v += t;
  }
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, WAVE));
  return v;
}

// exchange with lane ^ 32 / lane ^ 16 using the gfx950 permlane swaps (no LDS traffic)
__device__ __forceinline__ float xor32(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  // after the swap, element 0 holds (lower lanes: own value; upper: lower's value) and
  // element 1 holds (lower lanes: upper's value; upper: own value)
  return __uint_as_float(lane_id() < 32 ? r[1] : r[0]);
}
__device__ __forceinline__ float xor16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(((lane_id() >> 4) & 1) ? r[0] : r[1]);
}

// ---------------------------------------------------------------------------------------
// MFMA wrappers
// ---------------------------------------------------------------------------------------
// D = A(16x128 fp8 e4m3) * B(128x16 fp8 e4m3) + C, fp32.  Lane l holds row/col l%16 and
// the 32 contraction elements of group l/16 for A and B; C/D: col l%16, rows 4*(l/16)+i.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D = A(16x32 bf16) * B(32x16 bf16) + C, fp32.  Lane l: row/col l%16, contraction
// elements 8*(l/16) .. +7; C/D: col l%16, rows 4*(l/16)+i.
__device__ __forceinline__ v4f mfma_bf16_16x16x32(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 -> bf16 round-to-nearest-even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

}  // namespace dsa
