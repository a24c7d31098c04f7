// Lightning-indexer tile arithmetic for the FP8 path (H_I = 64 heads x d_I = 128).
//
// The index score of query t and key s is
//     I[t,s] = k_scale[s] * sum_j c[t,j] * ReLU(q8[t,j,:] . k8[s,:]),  c = w * q_scale
// i.e. the weighted sum over indexer heads of ReLU'd FP8 dot products (the indexer is
// multi-head, uses ReLU and runs in FP8: 53ai.com V3.2-Exp report summary, section
// 创新架构; juhe.plus explainer, section 第一步：Lightning Indexer).  Pulling the positive
// per-row scales out of the ReLU is exact in real arithmetic.
//
// One wave scores one query against 64 keys at a time:
//   * the 64 heads are the M dimension of four 16x16x128 FP8 MFMAs (A = the query's head
//     rows, loaded once), the keys are N (B = 16 keys x 128 bytes per fragment);
//   * each lane then holds 4 heads x 1 key per MFMA and folds ReLU and c into a running
//     fp32 sum over its 16 heads;
//   * a reduce-scatter over the four 16-lane groups (two permlane swaps) leaves lane l
//     with the full head sum for key l of the 64-key tile.
// Every kernel that produces scores goes through score_tile64(), so scores are
// bit-identical whichever kernel computes them.
#pragma once

#include "dsa_device.h"

namespace dsa {

constexpr int IDX_HEADS = 64;
constexpr int IDX_DIM = 128;
constexpr int KEY_TILE = 64;  // keys scored per wave step

// per-wave query state: A operands of the 4 head blocks and the 16 head weights c this
// lane folds (heads 16*hb + 4*(lane/16) + i)
struct IdxQuery {
  v8i a[4];
  float c[16];
};

// q8: the query's [64][128] FP8 codes; qs, w: its 64 scales and weights.
__device__ __forceinline__ void load_idx_query(IdxQuery& Q, const uint8_t* __restrict__ q8,
                                               const float* __restrict__ qs,
                                               const float* __restrict__ w) {
  const int l = lane_id();
  const int g = l >> 4;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int head = 16 * hb + (l & 15);
    const v4i* p = reinterpret_cast<const v4i*>(q8 + head * IDX_DIM + 32 * g);
    v4i lo = p[0], hi = p[1];
    Q.a[hb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h2 = 16 * hb + 4 * g + i;
      Q.c[4 * hb + i] = __fmul_rn(w[h2], qs[h2]);
    }
  }
}

// Partial head sum (this lane's 16 heads) for the key this lane holds in fragment b.
__device__ __forceinline__ float fold_fragment(const IdxQuery& Q, v8i b) {
  v4f acc[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) acc[hb] = mfma_fp8_16x16x128(Q.a[hb], b, v4f{0.f, 0.f, 0.f, 0.f});
  float p = 0.f;
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) p = __fmaf_rn(Q.c[4 * hb + i], fmaxf(acc[hb][i], 0.f), p);
  return p;
}

// Given the partial sums of 4 consecutive 16-key fragments, return the full head sum
// of key (lane) of the 64-key tile.
__device__ __forceinline__ float reduce_scatter4(float p0, float p1, float p2, float p3) {
  // lanes 0-31 collect fragments 0,1 and lanes 32-63 fragments 2,3 (pairs g, g+2)
  auto r02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
  auto r13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
  const float qa = __fadd_rn(__uint_as_float(r02[0]), __uint_as_float(r02[1]));
  const float qb = __fadd_rn(__uint_as_float(r13[0]), __uint_as_float(r13[1]));
  // rows (16-lane groups) 0..3 end with fragments 0..3 (pairs g, g+1)
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(qa), __float_as_uint(qb), false, false);
  return __fadd_rn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// B operand of fragment f (keys 16f .. 16f+15) from a 64-key LDS tile stored as
// 64 rows of 128 bytes whose 16-byte chunks are XOR-swizzled by (row & 7).
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
// clamped to n_k - 1 so the read stays in bounds).
__device__ __forceinline__ v8i global_key_fragment(const uint8_t* __restrict__ k8, int64_t key0,
                                                   int f, int64_t n_k) {
  const int l = lane_id();
  int64_t key = key0 + 16 * f + (l & 15);
  key = key < n_k ? key : n_k - 1;
  const v4i* p = reinterpret_cast<const v4i*>(k8 + key * IDX_DIM + 32 * (l >> 4));
  const v4i lo = __builtin_nontemporal_load(p);
  const v4i hi = __builtin_nontemporal_load(p + 1);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Score of key (key0 + lane) given the four fragments' B operands and that key's scale.
__device__ __forceinline__ float score_tile64(const IdxQuery& Q, v8i b0, v8i b1, v8i b2, v8i b3,
                                             float kscale) {
  const float p0 = fold_fragment(Q, b0);
  const float p1 = fold_fragment(Q, b1);
  const float p2 = fold_fragment(Q, b2);
  const float p3 = fold_fragment(Q, b3);
  return __fmul_rn(reduce_scatter4(p0, p1, p2, p3), kscale);
}

// Cooperative copy of one 64-key tile (8 KB) into LDS by a 256-thread block:
// two 16-byte chunks per thread, swizzled as lds_key_fragment() expects.
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
