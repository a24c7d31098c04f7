// Lightning-indexer tile arithmetic for the FP8 path (H_I = 64 heads x d_I = 128).
//
// The index score of query t and key s is
//     I[t,s] = k_scale[s] * sum_j c[t,j] * ReLU(q8[t,j,:] . k8[s,:]),  c = w * q_scale
// the weighted sum over indexer heads of ReLU'd FP8 dot products (the indexer is
// multi-head, uses ReLU and runs in FP8: 53ai.com V3.2-Exp report summary, section
// 创新架构; juhe.plus explainer, section 第一步：Lightning Indexer).  Pulling the positive
// per-row scales out of the ReLU is exact in real arithmetic.
//
// How the terms are formed (the same in every kernel, so scores are bit-identical
// whichever kernel produces them):
//   * the 64 heads are the M dimension of four 16x16x128 FP8 MFMAs (A = a query's head
//     rows), the keys are N (B = 16 keys x 128 bytes).  The MFMA's block scales multiply
//     every product by 2^-25, exactly (powers of two), so each head dot x lies in
//     (-0.77, 0.77) whatever the FP8 codes (|x| <= 448^2 * 128 * 2^-25);
//   * ReLU: pairs of head dots are packed to f16 (round to nearest even) by one conversion
//     whose output clamp to [0, 1] is the ReLU, as every head dot lies below 1 in magnitude
//     (one VALU op per pair of head values);
//   * the weighted head sum runs on the matrix core: per "head half" (32 heads) a
//     16x16x32 f16 MFMA whose A operand holds the half's normalised weights
//     c' = c / max|c| (f16) in every row and whose B operand is the ReLU'd values, so every
//     lane receives the half's sum for its key (l % 16) in fp32;
//   * the two head halves are added; the result is scaled by max|c| * 2^25 and by k_scale.
// Relative error of a term: <= 2^-11 (f16 rounding of the head dot) + 2^-11 (f16 weight);
// f16 subnormals below 2^-14 (head dots below 2^11 in code units) carry an absolute error
// of at most 1 code unit.
#pragma once

#include "dsa_device.h"

namespace dsa {

constexpr int IDX_HEADS = 64;
constexpr int IDX_DIM = 128;
constexpr int KEY_TILE = 64;  // keys per tile


// E8M0 block scales: 2^-13 on the query side, 2^-12 on the key side
constexpr uint32_t SCALE_Q = 0x72727272u, SCALE_K = 0x73737373u;
constexpr float UNSCALE = 33554432.0f;  // 2^25

__device__ __forceinline__ v4f mfma_fp8_scaled(v8i a, v8i b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, SCALE_Q, 0,
                                                          SCALE_K);
}

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// One query row's operands for one head half (head blocks 2hh, 2hh+1): the FP8 A operands
// and the A operand of the head-sum MFMA (contraction slot e of lane group g = head
// 32hh + 16(e/4) + 4g + e%4, the head whose ReLU'd value that lane packs in slot e).
struct IdxHalf {
  v8i a[2];
  v8h wa;
};

// Per-row weight normaliser: cs = max_j |w_j q_scale_j| * 2^25 (0 if all weights vanish),
// from lane j's head weight and query scale.
__device__ __forceinline__ float row_cmax_of(float w_l, float qs_l) {
  float m = fabsf(__fmul_rn(w_l, qs_l));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, WAVE));
  return m;
}
__device__ __forceinline__ float row_cmax(const float* __restrict__ qs, const float* __restrict__ w) {
  const int l = lane_id();
  return row_cmax_of(w[l], qs[l]);
}

// f16 head weight (w * q_scale) / max|c|: rounded to fp32, then to f16.  The empty asm keeps
// the compiler from fusing the two roundings into one mixed-precision FMA (which rounds
// differently now and then, and every kernel must produce the same weights).
__device__ __forceinline__ _Float16 head_weight_f16(float w, float qs, float inv) {
  float p = __fmul_rn(__fmul_rn(w, qs), inv);
  asm volatile("" : "+v"(p));
  return (_Float16)p;
}

// The head whose weight lane l packs in slot e of head half hh.
__device__ __forceinline__ int slot_head(int hh, int e, int l) {
  return 32 * hh + 16 * (e >> 2) + 4 * (l >> 4) + (e & 3);
}

// A operands of head half hh: head blocks 2hh, 2hh+1.
__device__ __forceinline__ void load_idx_half_a(IdxHalf& Q, const uint8_t* __restrict__ q8, int hh) {
  const int l = lane_id();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int hb = 2 * hh + k;
    const int head = 16 * hb + (l & 15);
    const v4i* p = reinterpret_cast<const v4i*>(q8 + head * IDX_DIM + 32 * (l >> 4));
    const v4i lo = p[0], hi = p[1];
    Q.a[k] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// Every weight and scale a lane needs is loaded before the first is used: the empty asm in
// head_weight_f16() keeps the scheduler from moving a later load above it, and loads
// interleaved with the conversions would each wait out their own latency.
__device__ __forceinline__ void load_idx_half(IdxHalf& Q, const uint8_t* __restrict__ q8,
                                              const float* __restrict__ qs, const float* __restrict__ w,
                                              int hh, float cmax) {
  const int l = lane_id();
  float wh[8], sh[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    wh[e] = w[slot_head(hh, e, l)];
    sh[e] = qs[slot_head(hh, e, l)];
  }
  load_idx_half_a(Q, q8, hh);
  const float inv = cmax > 0.f ? 1.f / cmax : 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) Q.wa[e] = head_weight_f16(wh[e], sh[e], inv);
}

// ReLU'd f16 B operand of the head-sum MFMA from the two FP8 MFMA results of a head half
// (slot e = head block e/4, MFMA row 4g + e%4).  min(max(., 0), 1) of the converted pair
// compiles to v_cvt_pk_f16_f32 with its clamp bit, which on this part gives exactly the
// ReLU of values below 1 in magnitude, the sign of zero included (v_cvt_pkrtz_f16_f32's
// clamp does not: negative inputs keep their sign there).
__device__ __forceinline__ v8h relu_pack(v4f x0, v4f x1) {
  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  typedef float f2v __attribute__((ext_vector_type(2)));
  const h2v zero = h2v{(_Float16)0.f, (_Float16)0.f};
  const h2v one = h2v{(_Float16)1.f, (_Float16)1.f};
  auto relu = [&](float a, float b) {
    return __builtin_elementwise_min(__builtin_elementwise_max(__builtin_convertvector(f2v{a, b}, h2v), zero), one);
  };
  const h2v r0 = relu(x0[0], x0[1]);
  const h2v r1 = relu(x0[2], x0[3]);
  const h2v r2 = relu(x1[0], x1[1]);
  const h2v r3 = relu(x1[2], x1[3]);
  return v8h{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// The head half's weighted ReLU sum for key l % 16 of the fragment, in every lane (element 0).
__device__ __forceinline__ float head_half_sum(const IdxHalf& Q, v4f x0, v4f x1) {
  const v4f d = __builtin_amdgcn_mfma_f32_16x16x32_f16(Q.wa, relu_pack(x0, x1), v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  return d[0];
}

// Final score from the two head-half totals.
__device__ __forceinline__ float finish_score(float t0, float t1, float cmax, float kscale) {
  return __fmul_rn(__fmul_rn(__fadd_rn(t0, t1), __fmul_rn(cmax, UNSCALE)), kscale);
}

// ---------------------------------------------------------------------------------------
// single-wave scoring of one query row against 64 keys (the score-writing kernels)
// ---------------------------------------------------------------------------------------
struct IdxRow {
  IdxHalf h[2];
  float cmax;
};

// (all of the row's loads in flight at once, then the normaliser and the f16 weights)
__device__ __forceinline__ void load_idx_row(IdxRow& R, const uint8_t* __restrict__ q8,
                                             const float* __restrict__ qs, const float* __restrict__ w) {
  const int l = lane_id();
  const float w_l = w[l], qs_l = qs[l];
  float wh[2][8], sh[2][8];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      wh[hh][e] = w[slot_head(hh, e, l)];
      sh[hh][e] = qs[slot_head(hh, e, l)];
    }
  load_idx_half_a(R.h[0], q8, 0);
  load_idx_half_a(R.h[1], q8, 1);
  R.cmax = row_cmax_of(w_l, qs_l);
  const float inv = R.cmax > 0.f ? 1.f / R.cmax : 0.f;
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) R.h[hh].wa[e] = head_weight_f16(wh[hh][e], sh[hh][e], inv);
}

// Waits (here, once) until a query row's operand loads have landed.
__device__ __forceinline__ void idx_row_landed(IdxRow& R) {
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int k = 0; k < 2; ++k) asm volatile("" : "+v"(R.h[hh].a[k]));
}

// B operand of fragment f (keys 16f .. 16f+15) from a 64-key LDS tile stored as 64 rows of
// 128 bytes whose 16-byte units are XOR-swizzled by (row & 7).
__device__ __forceinline__ v8i lds_key_fragment(const uint8_t* tile, int f) {
  const int l = lane_id();
  const int row = 16 * f + (l & 15);
  const int c0 = (2 * (l >> 4)) ^ (row & 7);
  const int c1 = (2 * (l >> 4) + 1) ^ (row & 7);
  const v4i lo = *reinterpret_cast<const v4i*>(tile + row * IDX_DIM + 16 * c0);
  const v4i hi = *reinterpret_cast<const v4i*>(tile + row * IDX_DIM + 16 * c1);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// B operand of fragment f straight from global memory (keys key0 + 16f + lane%16,
// clamped to n_k - 1 so the read stays in bounds; key j is row j * stride).
__device__ __forceinline__ v8i global_key_fragment(const uint8_t* __restrict__ k8, int64_t key0,
                                                   int f, int64_t n_k, int stride = 1) {
  const int l = lane_id();
  int64_t key = key0 + 16 * f + (l & 15);
  key = (key < n_k ? key : n_k - 1) * stride;
  // plain loads: the two halves of a lane's 32 bytes come from two instructions that each
  // touch half of every row, and the second must find the row in L2 (with streaming loads
  // it was fetched from HBM twice)
  const v4i* p = reinterpret_cast<const v4i*>(k8 + key * IDX_DIM + 32 * (l >> 4));
  const v4i lo = p[0];
  const v4i hi = p[1];
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Score of key (key0 + lane) of a 64-key tile given the four fragments' B operands: lane l
// takes fragment l/16's sums (every lane of a fragment's head-sum MFMA holds key l % 16).
__device__ __forceinline__ float score_tile64(const IdxRow& R, const v8i* b, float kscale) {
  v4f x[4][2][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      x[f][hh][0] = mfma_fp8_scaled(R.h[hh].a[0], b[f]);
      x[f][hh][1] = mfma_fp8_scaled(R.h[hh].a[1], b[f]);
    }
  float t[4][2];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) t[f][hh] = head_half_sum(R.h[hh], x[f][hh][0], x[f][hh][1]);
  const int fl = lane_id() >> 4;
  const float t0 = fl == 0 ? t[0][0] : fl == 1 ? t[1][0] : fl == 2 ? t[2][0] : t[3][0];
  const float t1 = fl == 0 ? t[0][1] : fl == 1 ? t[1][1] : fl == 2 ? t[2][1] : t[3][1];
  return finish_score(t0, t1, R.cmax, kscale);
}

// Cooperative copy of one 64-key tile (8 KB) into LDS by a 256-thread block:
// two 16-byte units per thread, swizzled as lds_key_fragment() expects.
struct KeyTileRegs {
  v4i c[2];
};
__device__ __forceinline__ void load_key_tile_regs(KeyTileRegs& R, const uint8_t* __restrict__ k8,
                                                   int64_t key0, int64_t n_k, int tid) {
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int u = tid + 256 * r;
    int64_t key = key0 + (u >> 3);
    key = key < n_k ? key : n_k - 1;
    R.c[r] = *reinterpret_cast<const v4i*>(k8 + key * IDX_DIM + 16 * (u & 7));
  }
}
__device__ __forceinline__ void store_key_tile_lds(const KeyTileRegs& R, uint8_t* tile, int tid) {
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int u = tid + 256 * r;
    const int row = u >> 3, c = u & 7;
    *reinterpret_cast<v4i*>(tile + row * IDX_DIM + 16 * (c ^ (row & 7))) = R.c[r];
  }
}

}  // namespace dsa
