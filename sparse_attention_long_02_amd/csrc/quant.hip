// FP8 E4M3FN row quantiser for the indexer operands (dsa_fp8_quantize_rows) and the
// indexer key-cache append (dsa_kcache_append).
//
// The indexer runs on FP8 operands with fp32 scales (53ai.com V3.2-Exp summary, section
// 创新架构; juhe.plus explainer, section 第一步：Lightning Indexer; yunpan.plus, section 1.1
// DSA).  Quantisation of a row (a key: 128 values; a query token: its 64 heads x 128 values,
// one scale for the whole token):
//     scale = amax / 448  (fp32, correctly rounded; 1 where the row is all zero)
//     code  = E4M3FN(x / scale)  (x / scale in fp32, correctly rounded; then round to the
//             nearest E4M3FN value, ties to even mantissa, saturating at +-448)
// E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, subnormals at exponent
// field 0 (m/8 * 2^-6), no infinities, S.1111.111 is NaN (never produced here).
//
// One wave per row: a pass for amax (wave-wide max), then a pass that encodes (the row is
// read twice; the second read is served by the cache).  Rows of a width in whole groups of
// 8 with aligned starts go 8 values per lane per access; others one value at a time.  HBM-bound: per row, width x input
// bytes read + width code bytes and 4 x repeat scale bytes written.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr float E4M3_MAX = 448.f;

// Round-to-nearest-even E4M3FN code of a finite fp32 value, saturating at +-448.
__device__ __forceinline__ uint32_t e4m3fn_encode(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fminf(__uint_as_float(bits & 0x7FFFFFFFu), E4M3_MAX);
  uint32_t code;
  if (a < 0.015625f) {  // below the smallest normal 2^-6: multiples of 2^-9 (exact scaling)
    const uint32_t m = (uint32_t)__builtin_rintf(a * 512.f);  // 0..8, ties to even
    code = m;                                                // m == 8 is the code of 2^-6
  } else {
    const uint32_t ab = __float_as_uint(a);
    uint32_t e = (ab >> 23) - 127u + 7u;   // biased E4M3 exponent, 1..15
    uint32_t r = (ab >> 20) & 7u;          // the three kept mantissa bits
    const uint32_t rem = ab & 0xFFFFFu;    // the dropped ones
    if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
    if (r == 8u) {
      r = 0u;
      ++e;
    }
    code = (e << 3) | r;  // a <= 448 keeps this <= 0x7E
  }
  return code | sign;
}

__device__ __forceinline__ float load_x(const void* x, int32_t dtype, int64_t i) {
  return dtype == DSA_BF16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[i])
                           : reinterpret_cast<const float*>(x)[i];
}

// Eight consecutive values from element offset i (16-byte aligned for bf16, 32 for fp32).
__device__ __forceinline__ void load8(const void* x, int32_t dtype, int64_t i, float* v) {
  if (dtype == DSA_BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + i);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Rows of group b: source row b * n_per + i, destination row b * dst_stride + base + i with
// base = pos ? pos[b] : 0; destination rows outside [0, dst_per) of their group are skipped.
__global__ __launch_bounds__(256) void fp8_quant_rows_kernel(const void* __restrict__ x, int32_t dtype,
                                                             int64_t n_per, int64_t width, int64_t ld_x,
                                                             const int32_t* __restrict__ pos, int64_t dst_per, int64_t dst_stride,
                                                             uint8_t* __restrict__ codes, int64_t ld_c,
                                                             float* __restrict__ scale, int64_t scale_stride,
                                                             int32_t repeat, bool vec) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t b = blockIdx.y;
  if (i >= n_per) return;
  const int64_t base = pos ? (int64_t)pos[b] : 0;
  const int64_t drow = base + i;
  if (drow < 0 || drow >= dst_per) return;
  const int64_t src = (b * n_per + i) * ld_x;
  const int64_t dst = b * dst_stride + drow;

  if (vec) {  // 8 values per lane per access (16-byte loads, 8-byte code stores)
    float amax = 0.f;
    for (int64_t j0 = 8 * lane; j0 < width; j0 += 8 * WAVE) {
      float v[8];
      load8(x, dtype, src + j0, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
    amax = wave_max(amax);
    const float s = amax > 0.f ? __fdiv_rn(amax, E4M3_MAX) : 1.f;
    uint8_t* crow = codes + dst * ld_c;
    for (int64_t j0 = 8 * lane; j0 < width; j0 += 8 * WAVE) {
      float v[8];
      load8(x, dtype, src + j0, v);
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0 |= e4m3fn_encode(__fdiv_rn(v[e], s)) << (8 * e);
        w1 |= e4m3fn_encode(__fdiv_rn(v[4 + e], s)) << (8 * e);
      }
      *reinterpret_cast<uint2*>(crow + j0) = make_uint2(w0, w1);
    }
    for (int r = lane; r < repeat; r += WAVE) scale[dst * scale_stride + r] = s;
    return;
  }

  float amax = 0.f;
  for (int64_t j = lane; j < width; j += WAVE) amax = fmaxf(amax, fabsf(load_x(x, dtype, src + j)));
  amax = wave_max(amax);
  const float s = amax > 0.f ? __fdiv_rn(amax, E4M3_MAX) : 1.f;

  uint8_t* crow = codes + dst * ld_c;
  // four consecutive codes per lane and store
  for (int64_t j0 = 4 * lane; j0 < width; j0 += 4 * WAVE) {
    uint32_t word = 0;
    const int n = width - j0 < 4 ? (int)(width - j0) : 4;
    for (int e = 0; e < n; ++e) word |= e4m3fn_encode(__fdiv_rn(load_x(x, dtype, src + j0 + e), s)) << (8 * e);
    if (n == 4 && (((uintptr_t)(crow + j0)) & 3u) == 0u) {
      *reinterpret_cast<uint32_t*>(crow + j0) = word;
    } else {
      for (int e = 0; e < n; ++e) crow[j0 + e] = (uint8_t)(word >> (8 * e));
    }
  }
  for (int r = lane; r < repeat; r += WAVE) scale[dst * scale_stride + r] = s;
}

hipError_t launch_fp8_quant_rows(const QuantArgs& a, hipStream_t st) {
  // the vector path needs every row start 16-byte aligned (inputs) and 8-byte aligned
  // (codes), and a width in whole groups of 8
  const int64_t esz = a.dtype == DSA_BF16 ? 2 : 4;
  const bool vec = a.width % 8 == 0 && ((uintptr_t)a.x & 15u) == 0 && (a.ld_x * esz) % 16 == 0 &&
                   ((uintptr_t)a.codes & 7u) == 0 && a.ld_codes % 8 == 0;
  dim3 grid((unsigned)((a.n_per + 3) / 4), (unsigned)a.groups);
  hipLaunchKernelGGL(fp8_quant_rows_kernel, grid, dim3(256), 0, st, a.x, a.dtype, a.n_per, a.width, a.ld_x,
                     a.pos, a.dst_per, a.dst_stride ? a.dst_stride : a.dst_per, a.codes, a.ld_codes, a.scale, a.scale_stride, a.repeat, vec);
  return hipGetLastError();
}

}  // namespace dsa
