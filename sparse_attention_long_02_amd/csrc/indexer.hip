// Lightning-indexer kernels that write scores to memory (dsa_indexer, decode).
//
// Two launch shapes share the tile arithmetic of indexer_tile.h, so their scores are
// bit-identical to each other and to what the fused prefill kernel ranks:
//   * idx_scores_fp8_rows:  4 query rows per 256-thread block (one per wave); key tiles
//     are staged once in LDS and read by all four waves.  Blocks are issued
//     longest-row-first to balance the causal triangle.
//   * idx_scores_fp8_split: one query row, its keys split across blocks and waves, key
//     fragments read straight from HBM (decode: one query per sequence, the key cache is
//     streamed exactly once).
// idx_scores_f32 is the plain fp32 variant (any H_I, d_I) for the fp32 configuration.
#include "dsa_kernels.h"
#include "indexer_tile.h"

namespace dsa {

__global__ __launch_bounds__(256) void idx_scores_fp8_rows(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, const float* __restrict__ w, int64_t n_q, int64_t n_k,
    const int32_t* __restrict__ q_pos, int64_t pos_offset, int64_t row_begin, int64_t n_rows,
    float* __restrict__ scores, int64_t ld) {
  __shared__ __align__(16) uint8_t tiles[2][KEY_TILE * IDX_DIM];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int64_t grp = (int64_t)gridDim.x - 1 - blockIdx.x;  // last rows first
  const int64_t i = grp * 4 + wv;
  const bool active = i < n_rows;
  const int64_t pos0 = (q_pos ? (int64_t)q_pos[b] : 0) + pos_offset + row_begin;
  const int64_t pos = pos0 + i;
  const int64_t i_last = (grp * 4 + 3 < n_rows) ? grp * 4 + 3 : n_rows - 1;
  int64_t n_vis = pos0 + i_last + 1;
  n_vis = n_vis < n_k ? n_vis : n_k;
  n_vis = n_vis > 0 ? n_vis : 0;
  const int ntiles = (int)((n_vis + KEY_TILE - 1) / KEY_TILE);

  const int64_t row = row_begin + i;
  const uint8_t* kb8 = k8 + (int64_t)b * n_k * IDX_DIM;
  const float* ksb = ks + (int64_t)b * n_k;
  IdxRow Q;
  if (active) {
    const int64_t qrow = (int64_t)b * n_q + row;
    load_idx_row(Q, q8 + qrow * IDX_HEADS * IDX_DIM, qs + qrow * IDX_HEADS, w + qrow * IDX_HEADS);
  }
  float* srow = scores + ((int64_t)b * n_rows + (active ? i : 0)) * ld;

  KeyTileRegs R;
  if (ntiles > 0) {
    load_key_tile_regs(R, kb8, 0, n_k, tid);
    store_key_tile_lds(R, tiles[0], tid);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < ntiles) load_key_tile_regs(R, kb8, (int64_t)(t + 1) * KEY_TILE, n_k, tid);
    if (active) {
      const int64_t key = (int64_t)t * KEY_TILE + lane;
      const float ksc = ksb[key < n_k ? key : n_k - 1];
      const v8i bf[4] = {lds_key_fragment(tiles[cur], 0), lds_key_fragment(tiles[cur], 1),
                         lds_key_fragment(tiles[cur], 2), lds_key_fragment(tiles[cur], 3)};
      const float s = score_tile64(Q, bf, ksc);
      if (key < n_k) srow[key] = key <= pos ? s : -INFINITY;
    }
    if (t + 1 < ntiles) store_key_tile_lds(R, tiles[cur ^ 1], tid);
    __syncthreads();
  }
  if (active)
    for (int64_t key = (int64_t)ntiles * KEY_TILE + lane; key < n_k; key += KEY_TILE) srow[key] = -INFINITY;
}

// grid: x = key splits of SPLIT_TILES tiles, y = row, z = sequence
constexpr int SPLIT_TILES = 32;  // 2048 keys per block, 8 tiles per wave

__global__ __launch_bounds__(256) void idx_scores_fp8_split(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, const float* __restrict__ w, int64_t n_q, int64_t n_k,
    const int32_t* __restrict__ q_pos, int64_t pos_offset, int64_t row_begin, int64_t n_rows,
    float* __restrict__ scores, int64_t ld) {
  const int b = blockIdx.z;
  const int64_t i = blockIdx.y;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pos = (q_pos ? (int64_t)q_pos[b] : 0) + pos_offset + row_begin + i;
  const int64_t row = row_begin + i;
  const int64_t qrow = (int64_t)b * n_q + row;
  const uint8_t* kb8 = k8 + (int64_t)b * n_k * IDX_DIM;
  const float* ksb = ks + (int64_t)b * n_k;
  float* srow = scores + ((int64_t)b * n_rows + i) * ld;
  const int64_t t0 = (int64_t)blockIdx.x * SPLIT_TILES;
  int64_t n_vis = pos + 1 < n_k ? pos + 1 : n_k;
  n_vis = n_vis > 0 ? n_vis : 0;
  const int64_t vis_tiles = (n_vis + KEY_TILE - 1) / KEY_TILE;

  const int64_t all_tiles = (n_k + KEY_TILE - 1) / KEY_TILE;
  const int64_t t_end = t0 + SPLIT_TILES < all_tiles ? t0 + SPLIT_TILES : all_tiles;
  const int64_t t_vis = t_end < vis_tiles ? t_end : vis_tiles;
  // tiles wholly beyond the query's position
  for (int64_t t = (t0 > t_vis ? t0 : t_vis) + wv; t < t_end; t += 4) {
    const int64_t key = t * KEY_TILE + lane;
    if (key < n_k) srow[key] = -INFINITY;
  }
  // visible tiles of this wave: t0 + wv, t0 + wv + 4, ...; each tile's key fragments are
  // loaded one tile ahead, while the previous tile is scored
  int64_t t = t0 + wv;
  if (t >= t_vis) return;
  IdxRow Q;
  load_idx_row(Q, q8 + qrow * IDX_HEADS * IDX_DIM, qs + qrow * IDX_HEADS, w + qrow * IDX_HEADS);
  v8i bf[4];
  float ksc;
  {
    const int64_t key0 = t * KEY_TILE, key = key0 + lane;
#pragma unroll
    for (int f = 0; f < 4; ++f) bf[f] = global_key_fragment(kb8, key0, f, n_k);
    ksc = ksb[key < n_k ? key : n_k - 1];
  }
  for (; t < t_vis; t += 4) {
    const int64_t tn = t + 4;
    v8i bn[4] = {bf[0], bf[1], bf[2], bf[3]};
    float kn = ksc;
    if (tn < t_vis) {
      const int64_t key0 = tn * KEY_TILE, key = key0 + lane;
#pragma unroll
      for (int f = 0; f < 4; ++f) bn[f] = global_key_fragment(kb8, key0, f, n_k);
      kn = ksb[key < n_k ? key : n_k - 1];
    }
    const int64_t key = t * KEY_TILE + lane;
    const float sc = score_tile64(Q, bf, ksc);
    if (key < n_k) srow[key] = key <= pos ? sc : -INFINITY;
#pragma unroll
    for (int f = 0; f < 4; ++f) bf[f] = bn[f];
    ksc = kn;
  }
}

// fp32 indexer: one thread per (row, key).
__global__ __launch_bounds__(256) void idx_scores_f32(
    const float* __restrict__ q, const float* __restrict__ qs, const float* __restrict__ kk,
    const float* __restrict__ ks, const float* __restrict__ w, int64_t n_q, int64_t n_k,
    const int32_t* __restrict__ q_pos, int64_t pos_offset, int H_I, int d_I, int64_t row_begin, int64_t n_rows,
    float* __restrict__ scores, int64_t ld) {
  const int b = blockIdx.z;
  const int64_t i = blockIdx.y;
  const int64_t key = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (key >= n_k) return;
  const int64_t pos = (q_pos ? (int64_t)q_pos[b] : 0) + pos_offset + row_begin + i;
  float* srow = scores + ((int64_t)b * n_rows + i) * ld;
  if (key > pos) {
    srow[key] = -INFINITY;
    return;
  }
  const int64_t qrow = (int64_t)b * n_q + row_begin + i;
  const float* qr = q + qrow * H_I * d_I;
  const float* kr = kk + ((int64_t)b * n_k + key) * d_I;
  float acc = 0.f;
  for (int j = 0; j < H_I; ++j) {
    float dot = 0.f;
    for (int d = 0; d < d_I; ++d) dot = __fmaf_rn(qr[j * d_I + d], kr[d], dot);
    const float c = __fmul_rn(w[qrow * H_I + j], qs[qrow * H_I + j]);
    acc = __fmaf_rn(c, fmaxf(dot, 0.f), acc);
  }
  srow[key] = __fmul_rn(acc, ks[(int64_t)b * n_k + key]);
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t st) {
  if (a.dtype == DSA_F32) {
    dim3 grid((unsigned)((a.n_k + 255) / 256), (unsigned)a.n_rows, (unsigned)a.B);
    hipLaunchKernelGGL(idx_scores_f32, grid, dim3(256), 0, st, (const float*)a.q_idx, a.q_scale,
                       (const float*)a.k_idx, a.k_scale, a.w, a.n_q, a.n_k, a.q_pos, a.pos_offset, a.H_I, a.d_I,
                       a.row_begin, a.n_rows, a.scores, a.ld_scores);
  } else if (a.n_rows * a.B <= 512) {
    dim3 grid((unsigned)((a.n_k + SPLIT_TILES * KEY_TILE - 1) / (SPLIT_TILES * KEY_TILE)),
              (unsigned)a.n_rows, (unsigned)a.B);
    hipLaunchKernelGGL(idx_scores_fp8_split, grid, dim3(256), 0, st, (const uint8_t*)a.q_idx, a.q_scale,
                       (const uint8_t*)a.k_idx, a.k_scale, a.w, a.n_q, a.n_k, a.q_pos, a.pos_offset, a.row_begin,
                       a.n_rows, a.scores, a.ld_scores);
  } else {
    dim3 grid((unsigned)((a.n_rows + 3) / 4), (unsigned)a.B);
    hipLaunchKernelGGL(idx_scores_fp8_rows, grid, dim3(256), 0, st, (const uint8_t*)a.q_idx, a.q_scale,
                       (const uint8_t*)a.k_idx, a.k_scale, a.w, a.n_q, a.n_k, a.q_pos, a.pos_offset, a.row_begin,
                       a.n_rows, a.scores, a.ld_scores);
  }
  return hipGetLastError();
}

}  // namespace dsa
