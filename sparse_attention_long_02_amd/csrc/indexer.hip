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
    const float* __restrict__ ks, const float* __restrict__ w, int64_t n_q, int64_t n_k, int64_t kbs,
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
  const uint8_t* kb8 = k8 + (int64_t)b * kbs * IDX_DIM;
  const float* ksb = ks + (int64_t)b * kbs;
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

// Key fragment f of the tile at launch key key0 and the scale of launch key `key` (clamped to
// n_keys - 1; launch key j is cache token j * stride of sequence b), from the contiguous
// per-sequence cache (kbs rows apart) or, PAGED, through the page table.
// Paged: with stride 1 a 64-key tile (key0 a multiple of 64) is one page, whose first pool
// row `row0` the caller looks up once per tile; strided keys look up their own pages.
template <bool PAGED>
__device__ __forceinline__ int64_t split_key_row(const PageTable& pt, int b, int64_t key, int64_t key0,
                                                 int64_t row0, int stride) {
  return stride == 1 ? row0 + (key - key0) : paged_row(pt, b, key * stride);
}
template <bool PAGED>
__device__ __forceinline__ v8i split_key_fragment(const uint8_t* __restrict__ k8, const PageTable& pt, int b,
                                                  int64_t kbs, int64_t key0, int f, int64_t n_keys, int stride,
                                                  int64_t row0) {
  if constexpr (!PAGED) {
    return global_key_fragment(k8 + (int64_t)b * kbs * IDX_DIM, key0, f, n_keys, stride);
  } else {
    const int l = lane_id();
    int64_t key = key0 + 16 * f + (l & 15);
    key = key < n_keys ? key : n_keys - 1;
    const v4i* p = reinterpret_cast<const v4i*>(k8 + split_key_row<PAGED>(pt, b, key, key0, row0, stride) * IDX_DIM +
                                                32 * (l >> 4));
    const v4i lo = p[0];
    const v4i hi = p[1];
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}
template <bool PAGED>
__device__ __forceinline__ float split_key_scale(const float* __restrict__ ks, const PageTable& pt, int b,
                                                 int64_t kbs, int64_t key, int64_t key0, int64_t n_keys, int stride,
                                                 int64_t row0) {
  key = key < n_keys ? key : n_keys - 1;
  if constexpr (!PAGED) return ks[(int64_t)b * kbs + key * stride];
  else return ks[split_key_row<PAGED>(pt, b, key, key0, row0, stride)];
}
// pool row of the first key of the tile at key0 (stride 1), looked up once per tile
template <bool PAGED>
__device__ __forceinline__ int64_t split_tile_row(const PageTable& pt, int b, int64_t key0, int stride) {
  if constexpr (!PAGED) return 0;
  else return stride == 1 ? paged_row(pt, b, key0) : 0;
}
// The same in two steps: the table entry of the tile at key0 (clamped to the last key, so the
// load stays inside the table whatever key0 is), and later the tile's first pool row from it.
template <bool PAGED>
__device__ __forceinline__ int32_t split_tile_entry(const PageTable& pt, int b, int64_t key0, int64_t n_keys,
                                                    int stride) {
  if constexpr (!PAGED) return 0;
  else return stride == 1 ? page_entry(pt, b, key0 < n_keys ? key0 : n_keys - 1) : 0;
}
template <bool PAGED>
__device__ __forceinline__ int64_t split_entry_row(const PageTable& pt, int32_t entry, int64_t key0, int stride) {
  if constexpr (!PAGED) return 0;
  else return stride == 1 ? page_entry_row(pt, entry, key0) : 0;
}

// grid: x = key splits of SPLIT_TILES tiles, y = row, z = sequence.
// Store mode: the row's scores of keys 0, S, 2S, ... (S = key_stride) go to columns 0, 1,
// 2, ... of its score row, -inf for keys past its position.  Filter mode (FILTER): nothing
// is stored; every wave keeps its own segment of DEC_SEG slots of the row's candidate list:
// the keys it scores above thr[b * n_rows + i], as (fp32 score bits, key index) pairs in
// ascending key order at cand + ((b * n_rows + i) * n_segs + seg) * DEC_SEG, seg =
// 4 blockIdx.x + wave (slots past DEC_SEG are counted, not stored), and their number at
// cnt[(b * n_rows + i) * n_segs + seg].  No atomics: a wave's slots come from a ballot and
// its running count.  With redo non-null only rows whose redo byte is set run.

template <bool FILTER, bool PAGED>
__global__ __launch_bounds__(256) void idx_scores_fp8_split(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, const float* __restrict__ w, int64_t n_q, int64_t n_k, int64_t kbs,
    const int32_t* __restrict__ q_pos, int64_t pos_offset, int64_t row_begin, int64_t n_rows,
    float* __restrict__ scores, int64_t ld, int key_stride_arg, const float* __restrict__ thr,
    uint2* __restrict__ cand, uint32_t* __restrict__ cnt, const uint8_t* __restrict__ redo, PageTable pt) {
  const int b = blockIdx.z;
  const int64_t i = blockIdx.y;
  const int64_t rid = (int64_t)b * n_rows + i;
  if (redo && !redo[rid]) return;  // uniform over the block
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pos = (q_pos ? (int64_t)q_pos[b] : 0) + pos_offset + row_begin + i;
  const int64_t row = row_begin + i;
  const int64_t qrow = (int64_t)b * n_q + row;
  float* srow = scores + rid * ld;
  const int64_t t0 = (int64_t)blockIdx.x * SPLIT_TILES;
  // the filter always runs over every key: a compile-time stride of 1 leaves one load path
  // in its loop (with the strided path beside it the compiler drains every tile's loads
  // before the previous tile is scored, which defeats the read-ahead)
  const int key_stride = FILTER ? 1 : key_stride_arg;
  // launch keys: key j is cache row j * key_stride; the row sees those at or below pos
  const int64_t n_keys = (n_k + key_stride - 1) / key_stride;
  int64_t lim = pos < n_k - 1 ? pos : n_k - 1;
  const int64_t n_vis = lim >= 0 ? lim / key_stride + 1 : 0;
  const int64_t vis_tiles = (n_vis + KEY_TILE - 1) / KEY_TILE;

  const int64_t all_tiles = (n_keys + KEY_TILE - 1) / KEY_TILE;
  const int64_t t_end = t0 + SPLIT_TILES < all_tiles ? t0 + SPLIT_TILES : all_tiles;
  const int64_t t_vis = t_end < vis_tiles ? t_end : vis_tiles;
  if (!FILTER) {  // tiles wholly beyond the query's position
    for (int64_t t = (t0 > t_vis ? t0 : t_vis) + wv; t < t_end; t += 4) {
      const int64_t key = t * KEY_TILE + lane;
      if (key < n_keys) srow[key] = -INFINITY;
    }
  }
  // visible tiles of this wave: t0 + wv, t0 + wv + 4, ...; each tile's key fragments are
  // loaded one tile ahead, while the previous tile is scored.  The two tiles in flight live
  // in two register buffers used in turn (the loop is unrolled by two): copying a tile's
  // registers from one buffer to the other would make the wave wait for its loads at the
  // copy, which is what the read-ahead exists to avoid.
  int64_t t = t0 + wv;
  const int64_t seg = rid * (4 * (int64_t)gridDim.x) + 4 * blockIdx.x + wv;
  if (t >= t_vis) {
    if (FILTER && lane == 0) cnt[seg] = 0u;
    return;
  }
  struct TileBuf {
    v8i b[4];
    float ks;
  };
  // paged, stride 1: the page entries of the tiles to be loaded, also two in turn; a tile's
  // entry is loaded one step before its fragments, ahead of that step's loads, so that no
  // load waits for a lookup (the memory counter drains in order)
  auto load_tile = [&](TileBuf& B, int64_t tile, int32_t entry) {
    const int64_t key0 = tile * KEY_TILE, key = key0 + lane;
    const int64_t row0 = split_entry_row<PAGED>(pt, entry, key0, key_stride);
#pragma unroll
    for (int f = 0; f < 4; ++f) B.b[f] = split_key_fragment<PAGED>(k8, pt, b, kbs, key0, f, n_keys, key_stride, row0);
    B.ks = split_key_scale<PAGED>(ks, pt, b, kbs, key, key0, n_keys, key_stride, row0);
  };
  // Every step issues the same loads: past the last visible tile the next tile is the last
  // one again (a re-read from cache, never scored).  With the loads conditional, the compiler
  // sizes each wait for the path that issued none and so waits for the tile just issued.
  auto clamp_tile = [&](int64_t x) { return x < t_vis ? x : t_vis - 1; };
  auto entry_of = [&](int64_t x) {
    return split_tile_entry<PAGED>(pt, b, clamp_tile(x) * KEY_TILE, n_keys, key_stride);
  };
  // the first tile's loads go out before the query row's, so both are in flight at once
  TileBuf A, B;
  load_tile(A, t, entry_of(t));
  int32_t e0 = 0, e1 = entry_of(t + 4);
  IdxRow Q;
  load_idx_row(Q, q8 + qrow * IDX_HEADS * IDX_DIM, qs + qrow * IDX_HEADS, w + qrow * IDX_HEADS);
  float T = 0.f;
  uint2* crow = nullptr;
  uint32_t ccount = 0;  // wave-uniform
  if (FILTER) {
    T = thr[rid];
    crow = cand + seg * DEC_SEG;
  }
  // the query's operands have landed before the loop: otherwise the compiler, merging the
  // loop's entry with its back edge, takes them as still in flight in every iteration and
  // makes each tile's first MFMAs wait for the loads issued just before them
  idx_row_landed(Q);
  auto score = [&](const TileBuf& C, int64_t tile) {
    const int64_t key = tile * KEY_TILE + lane;
    const float sc = score_tile64(Q, C.b, C.ks);
    if (FILTER) {
      const bool pass = key < n_vis && sc > T;
      const uint64_t m = ballot(pass);
      const uint32_t slot = ccount + lanes_below(m);
      if (pass && slot < (uint32_t)DEC_SEG) crow[slot] = make_uint2(__float_as_uint(sc), (uint32_t)key);
      ccount += (uint32_t)__popcll((unsigned long long)m);
    } else if (key < n_keys) {
      srow[key] = key < n_vis ? sc : -INFINITY;
    }
  };
  for (;;) {
    e0 = entry_of(t + 8);
    load_tile(B, clamp_tile(t + 4), e1);
    score(A, t);
    t += 4;
    if (t >= t_vis) break;
    e1 = entry_of(t + 8);
    load_tile(A, clamp_tile(t + 4), e0);
    score(B, t);
    t += 4;
    if (t >= t_vis) break;
  }
  if (FILTER && lane == 0) cnt[seg] = ccount;
}

hipError_t launch_idx_split(const SplitIdxArgs& a, hipStream_t st) {
  const int64_t n_keys = (a.n_k + a.key_stride - 1) / a.key_stride;
  dim3 grid((unsigned)((n_keys + SPLIT_TILES * KEY_TILE - 1) / (SPLIT_TILES * KEY_TILE)), (unsigned)a.n_rows,
            (unsigned)a.B);
  const int64_t kbs = a.k_bstride ? a.k_bstride : a.n_k;
  const bool paged = a.pages.table != nullptr;
  auto kern = a.cand ? (paged ? idx_scores_fp8_split<true, true> : idx_scores_fp8_split<true, false>)
                     : (paged ? idx_scores_fp8_split<false, true> : idx_scores_fp8_split<false, false>);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, a.q8, a.qs, a.k8, a.ks, a.w, a.n_q, a.n_k, kbs, a.q_pos,
                     a.pos_offset, a.row_begin, a.n_rows, a.cand ? nullptr : a.scores, a.cand ? (int64_t)0 : a.ld,
                     a.cand ? 1 : (int)a.key_stride, a.thr, a.cand, a.cnt, a.redo, a.pages);
  return hipGetLastError();
}

// fp32 indexer: one thread per (row, key).
__global__ __launch_bounds__(256) void idx_scores_f32(
    const float* __restrict__ q, const float* __restrict__ qs, const float* __restrict__ kk,
    const float* __restrict__ ks, const float* __restrict__ w, int64_t n_q, int64_t n_k, int64_t kbs,
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
  const float* kr = kk + ((int64_t)b * kbs + key) * d_I;
  float acc = 0.f;
  for (int j = 0; j < H_I; ++j) {
    float dot = 0.f;
    for (int d = 0; d < d_I; ++d) dot = __fmaf_rn(qr[j * d_I + d], kr[d], dot);
    const float c = __fmul_rn(w[qrow * H_I + j], qs[qrow * H_I + j]);
    acc = __fmaf_rn(c, fmaxf(dot, 0.f), acc);
  }
  srow[key] = __fmul_rn(acc, ks[(int64_t)b * kbs + key]);
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t st) {
  const int64_t kbs = a.k_bstride ? a.k_bstride : a.n_k;
  if (a.dtype == DSA_F32) {
    dim3 grid((unsigned)((a.n_k + 255) / 256), (unsigned)a.n_rows, (unsigned)a.B);
    hipLaunchKernelGGL(idx_scores_f32, grid, dim3(256), 0, st, (const float*)a.q_idx, a.q_scale,
                       (const float*)a.k_idx, a.k_scale, a.w, a.n_q, a.n_k, kbs, a.q_pos, a.pos_offset, a.H_I, a.d_I,
                       a.row_begin, a.n_rows, a.scores, a.ld_scores);
  } else if (a.n_rows * a.B <= 512) {
    SplitIdxArgs sa{(const uint8_t*)a.q_idx, a.q_scale, (const uint8_t*)a.k_idx, a.k_scale, a.w, a.B, a.n_q, a.n_k,
                    a.q_pos, a.pos_offset, a.row_begin, a.n_rows, a.scores, a.ld_scores, 1, nullptr, nullptr,
                    nullptr, nullptr, a.k_bstride};
    return launch_idx_split(sa, st);
  } else {
    dim3 grid((unsigned)((a.n_rows + 3) / 4), (unsigned)a.B);
    hipLaunchKernelGGL(idx_scores_fp8_rows, grid, dim3(256), 0, st, (const uint8_t*)a.q_idx, a.q_scale,
                       (const uint8_t*)a.k_idx, a.k_scale, a.w, a.n_q, a.n_k, kbs, a.q_pos, a.pos_offset, a.row_begin,
                       a.n_rows, a.scores, a.ld_scores);
  }
  return hipGetLastError();
}

}  // namespace dsa
