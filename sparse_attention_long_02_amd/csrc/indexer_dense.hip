// FP8 lightning-indexer scores of blocks of 16 query rows, for the threshold-filtered
// selection of prefill rows (and, with a key stride, the key sample that sets the
// thresholds).  Two modes:
//   * store: the scores of a row (every key, or every S-th key) go to a padded workspace
//     row; the selection uses it only for the 1-in-32 key sample;
//   * filter: the scores are compared with the row's threshold and only the keys at or
//     above it leave the chip, appended to the row's candidate list in ascending key order.
//
// The score of query t and key s is the weighted sum over the 64 indexer heads of ReLU'd
// FP8 dot products (53ai.com V3.2-Exp summary, section 创新架构; juhe.plus explainer,
// section 第一步：Lightning Indexer), formed exactly as in indexer_tile.h so that every
// kernel produces the same bits.  Only the grouping differs, chosen so that the matrix
// cores do nearly all the work:
//   * a block of 4 waves owns 16 consecutive query rows, 4 per wave, all 64 heads of each
//     (the A operands of 16 FP8 MFMAs per 16-key fragment, 128 registers);
//   * a 64-key tile is scored as 4 fragments.  Fragment f takes the tile's keys 4c + f
//     (c = 0..15), so after the four fragments lane c of each lane group holds 4 adjacent
//     keys and writes them with one 16-byte store;
//   * the weighted head sums of the 4 rows run as two chains (one per head half) of four
//     16x16x32 f16 MFMAs.  The A operand of row j carries that row's weights in output rows
//     4j .. 4j+3 and zeros elsewhere, so lane group g ends the chain holding row g's sum;
//     the zero rows add exact zeros, so each sum is the same single MFMA sum as in the
//     other kernels;
//   * key tiles (8 KB + 64 key scales) arrive by direct global->LDS loads into a ring of
//     DN_SLOTS slots, DN_SLOTS-2 tiles ahead; one block barrier per tile.
// Rows and columns of the workspace are padded (rows to 16 per block, columns to whole
// 64-key tiles), so every store is in bounds and every wave issues exactly one store per
// tile; the explicit load waits below count on that.
#include "dsa_kernels.h"
#include "indexer_tile.h"
#include "lds_dma.h"

namespace dsa {

constexpr int DN_WAVES = 4;
constexpr int DN_SLOTS = 6;
constexpr int DN_TILE_BYTES = KEY_TILE * IDX_DIM;            // 8192
constexpr int DN_SLOT_BYTES = DN_TILE_BYTES + KEY_TILE * 4;  // + the tile's key scales

typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));

// LDS layout of a tile: row rho (0..63) holds key 4 (rho % 16) + rho / 16 of the tile, its
// 16-byte unit u stored at unit u ^ (rho & 7); the 64 key scales follow in key order.
// Wave w loads rows 16w .. 16w+15 (two 1 KB direct loads); wave 3 also loads the scales.
struct DenseDma {
  uint32_t off[2];  // byte offset of this lane's unit within its key row, plus 128 * key
};
__device__ __forceinline__ DenseDma dense_dma_lane(int wv, int lane) {
  DenseDma d;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rho = 16 * wv + 8 * i + (lane >> 3);
    const int key = 4 * (rho & 15) + (rho >> 4);
    d.off[i] = (uint32_t)(key * IDX_DIM + 16 * ((lane & 7) ^ (rho & 7)));
  }
  return d;
}
// Key j of the launch is cache row j * stride; keys past n_keys - 1 (the last one the
// launch may read) read that key (their scores are masked).  kb / ksb: the sequence's rows,
// or (PAGED) the page pools, whose rows the table gives.
template <bool PAGED>
__device__ __forceinline__ void dense_tile_load(uint32_t slot, const uint8_t* __restrict__ kb,
                                                const float* __restrict__ ksb, int64_t key0, int64_t n_keys,
                                                int64_t stride, const DenseDma& d, int wv, int lane,
                                                const PageTable& pt, int b) {
  // paged, stride 1: the tile is one page, looked up once (strided keys look up their own)
  int64_t first = 0, base = 0;
  if (PAGED && stride == 1) base = paged_tile_base(pt, b, key0, n_keys - 1, first);
  auto row_of = [&](int64_t kc) -> int64_t {
    if constexpr (!PAGED) return kc;
    else return stride == 1 ? base + (kc - first) : paged_row(pt, b, kc);
  };
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t key = key0 + (d.off[i] >> 7);
    const int64_t kc = (key < n_keys ? key : n_keys - 1) * stride;
    dma16_vaddr(kb + row_of(kc) * IDX_DIM + (d.off[i] & 127u), slot + 2048 * wv + 1024 * i);
  }
  if (wv == 3) {
    const int64_t key = key0 + lane;
    const int64_t kc = (key < n_keys ? key : n_keys - 1) * stride;
    dma4_vaddr(ksb + row_of(kc), slot + DN_TILE_BYTES);
  }
}

// B operand of fragment f: LDS rows 16f + c (keys 4c + f), contraction bytes 32g .. 32g+31.
__device__ __forceinline__ v8i dense_fragment(const uint8_t* tile, int f, int lane) {
  typedef __attribute__((address_space(3))) const v4i lds_v4i;
  typedef __attribute__((address_space(3))) const uint8_t lds_u8;
  const int rho = 16 * f + (lane & 15);
  const int g = lane >> 4;
  const lds_u8* row = (lds_u8*)tile + rho * IDX_DIM;
  const v4i lo = *(lds_v4i*)(row + 16 * ((2 * g) ^ (rho & 7)));
  const v4i hi = *(lds_v4i*)(row + 16 * ((2 * g + 1) ^ (rho & 7)));
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// grid.x = B * n_grp (16-row groups, longest first within each sequence); 256 threads.
// Row i (0 <= i < n_rows) of sequence b is query row row_begin + i, at position
// (q_pos ? q_pos[b] : 0) + row_begin + i.  Launch key j is cache row j * stride and the row
// sees it when j * stride <= min(position, n_k - 1).
// Store mode: the row's scores go to row b * 16 n_grp + i of `scores` (ld floats apart, ld
// a multiple of 64 covering the tiles the row needs); keys it does not see score -inf.
// Filter mode: see DenseIdxArgs.
template <bool FILTER, bool PAGED>
__global__ __launch_bounds__(DN_WAVES * 64, 2) void idx_dense_fp8_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, const float* __restrict__ w, int B, int64_t n_q, int64_t n_k, int64_t kbs,
    const int32_t* __restrict__ q_pos, int64_t row_begin, int64_t n_rows, int64_t n_grp, int stride,
    float* __restrict__ scores, int64_t ld, const float* __restrict__ thr, uint2* __restrict__ cand,
    uint32_t* __restrict__ cnt, PageTable pt) {
  __shared__ __align__(16) uint8_t ring[DN_SLOTS * DN_SLOT_BYTES];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int b = (int)(blockIdx.x % B);
  const int64_t grp = n_grp - 1 - (int64_t)(blockIdx.x / B);
  const int64_t pos0 = (q_pos ? (int64_t)q_pos[b] : 0) + row_begin;
  const int64_t i0 = 16 * grp;
  const int64_t i_last = i0 + 15 < n_rows ? i0 + 15 : n_rows - 1;
  // launch keys 0 .. n_keys - 1 exist; the group's last row sees n_vis of them
  const int64_t n_keys = (n_k + stride - 1) / stride;
  int64_t lim_last = pos0 + i_last < n_k - 1 ? pos0 + i_last : n_k - 1;
  const int64_t n_vis = lim_last >= 0 ? lim_last / stride + 1 : 0;
  const int ntiles = (int)((n_vis + KEY_TILE - 1) / KEY_TILE);

  const uint8_t* kb = PAGED ? k8 : k8 + (size_t)b * kbs * IDX_DIM;
  const float* ksb = PAGED ? ks : ks + (size_t)b * kbs;
  const uint32_t ring0 = lds_addr(ring);
  const DenseDma dl = dense_dma_lane(wv, lane);
#pragma unroll
  for (int t = 0; t < DN_SLOTS - 2; ++t)
    if (t < ntiles)
      dense_tile_load<PAGED>(ring0 + t * DN_SLOT_BYTES, kb, ksb, (int64_t)t * KEY_TILE, n_keys, stride, dl, wv,
                             lane, pt, b);

  // this wave's rows i0 + 4wv + j; padding rows score the last real row
  const int g = lane >> 4, c = lane & 15, rq = c >> 2;
  v8i A[4][4];
  v8h_t W[2][4];
  float cmx = 0.f;
  int64_t lim = -1;
  auto row_of = [&](int j) {
    const int64_t i = i0 + 4 * wv + j;
    return (int64_t)b * n_q + row_begin + (i < n_rows ? i : n_rows - 1);
  };
  // every load first (A operands, the four rows' normaliser inputs, and the weights and
  // scales of this lane's row rq), then the arithmetic: the empty asm in head_weight_f16()
  // keeps loads from moving above it, so loads placed between the conversions would each
  // wait out their own latency
  float wl[4], sl[4], wh[2][8], sh[2][8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t qrow = row_of(j);
    wl[j] = w[qrow * IDX_HEADS + lane];
    sl[j] = qs[qrow * IDX_HEADS + lane];
  }
  {
    const int64_t qrow = row_of(rq);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        wh[hh][e] = w[qrow * IDX_HEADS + slot_head(hh, e, lane)];
        sh[hh][e] = qs[qrow * IDX_HEADS + slot_head(hh, e, lane)];
      }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint8_t* qr = q8 + row_of(j) * IDX_HEADS * IDX_DIM;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const v4i* p = reinterpret_cast<const v4i*>(qr + (16 * hb + c) * IDX_DIM + 32 * g);
      const v4i lo = p[0], hi = p[1];
      A[j][hb] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  float cm_own = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i = i0 + 4 * wv + j;
    const float cm = row_cmax_of(wl[j], sl[j]);
    if (rq == j) cm_own = cm;
    if (g == j) {
      cmx = __fmul_rn(cm, UNSCALE);
      const int64_t p = pos0 + i;
      const int64_t lk = p < n_k - 1 ? p : n_k - 1;
      lim = lk >= 0 ? lk / stride : -1;
    }
  }
  {
    const float inv = cm_own > 0.f ? 1.f / cm_own : 0.f;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const _Float16 wt = head_weight_f16(wh[hh][e], sh[hh][e], inv);
#pragma unroll
        for (int j = 0; j < 4; ++j) W[hh][j][e] = rq == j ? wt : (_Float16)0.f;
      }
  }
  const int64_t my_row = (int64_t)b * 16 * n_grp + i0 + 4 * wv + g;
  float* srow = scores + my_row * ld + 4 * c;
  // filter mode: this lane's row's threshold; the wave's four rows' lists and counts (the
  // counts are wave-uniform, one per 16-lane group)
  float thr_f = 0.f;
  uint32_t cnt_g[4] = {0u, 0u, 0u, 0u};
  uint2* wlist = nullptr;
  if constexpr (FILTER) {
    const int64_t i = i0 + 4 * wv + g;
    thr_f = thr[(int64_t)b * 16 * n_grp + (i < n_rows ? i : n_rows - 1)];
    wlist = cand + ((int64_t)b * 16 * n_grp + i0 + 4 * wv) * SEL_CAND_PITCH;
  }
  const uint32_t row_off = (uint32_t)g * SEL_CAND_PITCH;
  // A tile's scores are compared with the threshold when the tile is done; appending the
  // keys that pass runs one tile later, between the next tile's matrix-core products, so
  // its scan / store chain overlaps them.  Keys 4c + f of the tile (row g of the wave) are
  // appended in (c, f) order, i.e. ascending: a lane's first slot follows the row's earlier
  // hits and the hits of the lanes below it in its 16-lane group (a scan within the DPP
  // row).  Every lane stores four times per tile, lanes without a key to append into their
  // row's scratch slot, so each wave issues exactly four stores per tile and the load
  // waits below can count them.
  auto append_tile = [&](const float (&sc)[4], uint32_t hit, uint32_t key32) {
    const uint32_t h = (uint32_t)__builtin_popcount(hit);
    uint32_t incl = h;
    incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x111, 0xF, 0xF, true);  // row_shr:1
    incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x112, 0xF, 0xF, true);  // row_shr:2
    incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x114, 0xF, 0xF, true);  // row_shr:4
    incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x118, 0xF, 0xF, true);  // row_shr:8
    const uint32_t base = g == 0 ? cnt_g[0] : g == 1 ? cnt_g[1] : g == 2 ? cnt_g[2] : cnt_g[3];
    const uint32_t first = row_off + base + incl - h;
    const uint32_t end = row_off + (uint32_t)SEL_CAND_CAP;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint32_t o = first + (uint32_t)__builtin_popcount(hit & ((1u << f) - 1u));
      const bool ok = ((hit >> f) & 1u) && o < end;
      wlist[ok ? o : end] = make_uint2(__float_as_uint(sc[f]), key32 + f);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) cnt_g[q] += (uint32_t)__builtin_amdgcn_readlane((int)incl, 16 * q + 15);
  };
  const int32_t lim32 = (int32_t)lim;
  // the previous tile's pending append (none before tile 0)
  float psc[4] = {0.f, 0.f, 0.f, 0.f};
  uint32_t phit = 0;
  constexpr int STORES = FILTER ? 4 : 1;

  // one 64-key tile: scores, then the store (store mode) or the compare (filter mode)
  auto tile_step = [&](int t) {
    const uint8_t* tile = ring + (t % DN_SLOTS) * DN_SLOT_BYTES;
    float v[4];
    // each fragment's B operand is read from LDS one fragment ahead
    v8i bnext = dense_fragment(tile, 0, lane);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const v8i bf = bnext;
      if (f < 3) bnext = dense_fragment(tile, f + 1, lane);
      v4f d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4f x0 = mfma_fp8_scaled(A[j][0], bf);
        const v4f x1 = mfma_fp8_scaled(A[j][1], bf);
        const v4f x2 = mfma_fp8_scaled(A[j][2], bf);
        const v4f x3 = mfma_fp8_scaled(A[j][3], bf);
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(W[0][j], relu_pack(x0, x1), d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(W[1][j], relu_pack(x2, x3), d1, 0, 0, 0);
      }
      v[f] = __fadd_rn(d0[0], d1[0]);
      if constexpr (FILTER)
        if (f == 0) append_tile(psc, phit, (uint32_t)(4 * c + (t - 1) * KEY_TILE));
    }
    __builtin_amdgcn_s_setprio(0);
    typedef __attribute__((address_space(3))) const v4f lds_v4f;
    const v4f kscale = *(lds_v4f*)((__attribute__((address_space(3))) const uint8_t*)tile + DN_TILE_BYTES + 16 * c);
    const int64_t key = (int64_t)t * KEY_TILE + 4 * c;
    if constexpr (!FILTER) {
      v4f o;
#pragma unroll
      for (int f = 0; f < 4; ++f)
        o[f] = key + f <= lim ? __fmul_rn(__fmul_rn(v[f], cmx), kscale[f]) : -INFINITY;
      *reinterpret_cast<v4f*>(srow + (int64_t)t * KEY_TILE) = o;
    } else {
      phit = 0;
      const int32_t vis = lim32 - (int32_t)key;  // filter mode: fewer than 2^31 keys
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        psc[f] = __fmul_rn(__fmul_rn(v[f], cmx), kscale[f]);
        phit |= (uint32_t)((f <= vis) & (psc[f] > thr_f)) << f;
      }
    }
  };

  // Two tiles per block barrier.  At each step the slots of the previous step's two tiles are
  // refilled with the tiles four ahead (the ring holds the step's two tiles and four in
  // flight).
  for (int t = 0; t < ntiles; t += 2) {
    // tiles t and t+1 have landed once at most the loads of tiles t+2 and t+3 and the stores
    // of the two steps since their own loads (STORES per tile) are outstanding
    // (vector-memory operations complete in issue order); outside the steady state wait
    // for everything
    if (t >= 4 && t + 3 < ntiles) {
      if (wv == 3) VMCNT(2 * 3 + 4 * STORES);
      else VMCNT(2 * 2 + 4 * STORES);
    } else {
      VMCNT(0);
    }
    LGKM0();
    block_barrier();
    // into the slots of tiles t-2 and t-1, which every wave is done with
    if (t + 4 < ntiles)
      dense_tile_load<PAGED>(ring0 + ((t + 4) % DN_SLOTS) * DN_SLOT_BYTES, kb, ksb, (int64_t)(t + 4) * KEY_TILE,
                             n_keys, stride, dl, wv, lane, pt, b);
    if (t + 5 < ntiles)
      dense_tile_load<PAGED>(ring0 + ((t + 5) % DN_SLOTS) * DN_SLOT_BYTES, kb, ksb, (int64_t)(t + 5) * KEY_TILE,
                             n_keys, stride, dl, wv, lane, pt, b);
    const int t_end = t + 2 < ntiles ? t + 2 : ntiles;
#pragma nounroll
    for (int u = t; u < t_end; ++u) tile_step(u);
  }
  if constexpr (FILTER) {
    if (ntiles > 0) append_tile(psc, phit, (uint32_t)(4 * c + (ntiles - 1) * KEY_TILE));
    const int64_t i = i0 + 4 * wv + g;
    const uint32_t total = g == 0 ? cnt_g[0] : g == 1 ? cnt_g[1] : g == 2 ? cnt_g[2] : cnt_g[3];
    if (c == 0 && i < n_rows) cnt[my_row] = total;
  }
}

hipError_t launch_idx_dense(const DenseIdxArgs& a, hipStream_t st) {
  const int64_t n_grp = (a.n_rows + 15) / 16;
  if (n_grp <= 0) return hipSuccess;
  if (a.key_stride < 1 || (a.cand && a.key_stride != 1)) return hipErrorInvalidValue;
  const bool paged = a.pages.table != nullptr;
  const int64_t kbs = a.k_bstride ? a.k_bstride : a.n_k;
  if (a.cand) {
    auto kern = paged ? idx_dense_fp8_kernel<true, true> : idx_dense_fp8_kernel<true, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.B * n_grp)), dim3(DN_WAVES * 64), 0, st, a.q8, a.qs, a.k8, a.ks, a.w,
                       (int)a.B, a.n_q, a.n_k, kbs, a.q_pos, a.row_begin, a.n_rows, n_grp, 1, nullptr, (int64_t)0,
                       a.thr, a.cand, a.cnt, a.pages);
  } else {
    auto kern = paged ? idx_dense_fp8_kernel<false, true> : idx_dense_fp8_kernel<false, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.B * n_grp)), dim3(DN_WAVES * 64), 0, st, a.q8, a.qs, a.k8, a.ks, a.w,
                       (int)a.B, a.n_q, a.n_k, kbs, a.q_pos, a.row_begin, a.n_rows, n_grp, a.key_stride, a.scores,
                       a.ld, nullptr, nullptr, nullptr, a.pages);
  }
  return hipGetLastError();
}

}  // namespace dsa
