// Fused lightning indexer + streaming top-k for prefill (query t at position t).
//
// The indexer's L x L score matrix is never stored.  Each wave owns one query row and
// scores its visible keys 64 at a time (indexer_tile.h); every score immediately meets
// the row's streaming selection state in LDS:
//   * a candidate buffer (order-preserving key + index) that stays sorted by key index,
//     because keys arrive in ascending order and appends keep lane order;
//   * a threshold thr: once the buffer has been cut to exactly k entries, v* = the k-th
//     largest key so far, and a later key can only enter with a strictly larger key
//     (on a tie it has the larger index, and the lower index wins);
//   * when the buffer is nearly full, a wave-local radix select (4 x 8-bit digits over
//     an LDS histogram) finds v* and an in-place stable compaction keeps exactly the
//     top-k so far.
// At the end the buffer holds the row's selection in ascending key order.  Rows whose
// position is below k keep every key and are written by a separate fill kernel.
//
// Selection rule: top-k by index score with ties to the lower key index (juhe.plus
// explainer, section 第二步：Fine-grained Token Selection; 53ai.com V3.2-Exp summary,
// section 创新架构).
#include "dsa_kernels.h"
#include "indexer_tile.h"

namespace dsa {

constexpr int CAND = 4096;  // candidate slots per row

struct RowSelect {
  uint32_t* key;  // [CAND]
  int32_t* idx;   // [CAND]
  uint32_t* hist; // [256]
};

// Radix select of the k-th largest key among key[0..n) (n > k), then stable in-place
// compaction to exactly k entries.  Wave-local; returns v*.
__device__ uint32_t select_compact(const RowSelect& R, int n, int k) {
  const int lane = lane_id();
  uint32_t prefix = 0, pmask = 0;
  uint32_t rem = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) R.hist[lane + 64 * j] = 0;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < n; i += WAVE) {
      const uint32_t u = R.key[i];
      if ((u & pmask) == prefix) atomicAdd(&R.hist[(u >> shift) & 255u], 1u);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    // lane owns bins 255-4*lane .. 252-4*lane (descending)
    uint32_t h[4], local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = R.hist[255 - 4 * lane - j];
      local += h[j];
    }
    uint32_t c = wave_incl_scan(local) - local;
    uint32_t digit = 0, above = 0;
    bool found = false;
    if (c < rem && c + local >= rem) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!found && c + h[j] >= rem) {
          found = true;
          digit = 255u - 4u * lane - j;
          above = c;
        }
        c += h[j];
      }
    }
    const uint64_t fm = ballot(found);
    const int src = __ffsll((unsigned long long)fm) - 1;
    digit = __shfl(digit, src, WAVE);
    above = __shfl(above, src, WAVE);
    rem -= above;
    prefix |= digit << shift;
    pmask |= 0xFFu << shift;
  }
  // keep key > v*, and the first `rem` keys equal to v* (lowest indices)
  uint32_t kept = 0, eq_seen = 0;
  for (int base = 0; base < n; base += WAVE) {
    const int i = base + lane;
    const bool in = i < n;
    const uint32_t u = in ? R.key[i] : 0u;
    const int32_t id = in ? R.idx[i] : -1;
    const bool eq = in && u == prefix;
    const uint64_t me = ballot(eq);
    const bool keep = (in && u > prefix) || (eq && eq_seen + lanes_below(me) < rem);
    const uint64_t mk = ballot(keep);
    if (keep) {
      const uint32_t dst = kept + lanes_below(mk);
      R.key[dst] = u;
      R.idx[dst] = id;
    }
    kept += (uint32_t)__popcll((unsigned long long)mk);
    eq_seen += (uint32_t)__popcll((unsigned long long)me);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  return prefix;
}

// grid.x = row groups of 4 over rows [row_lo, L), last rows first
__global__ __launch_bounds__(256, 1) void prefill_idx_topk_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, const float* __restrict__ w, int64_t L, int64_t row_lo, int k,
    int32_t* __restrict__ idx) {
  __shared__ __align__(16) uint8_t tiles[2][KEY_TILE * IDX_DIM];
  __shared__ uint32_t ckey[4][CAND];
  __shared__ int32_t cidx[4][CAND];
  __shared__ uint32_t hist[4][256];

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int64_t n_rows = L - row_lo;
  const int64_t grp = (int64_t)gridDim.x - 1 - blockIdx.x;
  const int64_t i = grp * 4 + wv;
  const bool active = i < n_rows;
  const int64_t row = row_lo + i;  // == its position
  const int64_t i_last = (grp * 4 + 3 < n_rows) ? grp * 4 + 3 : n_rows - 1;
  const int64_t n_vis = row_lo + i_last + 1;  // <= L
  const int ntiles = (int)((n_vis + KEY_TILE - 1) / KEY_TILE);

  IdxQuery Q;
  if (active) load_idx_query(Q, q8 + row * IDX_HEADS * IDX_DIM, qs + row * IDX_HEADS, w + row * IDX_HEADS);
  RowSelect R{ckey[wv], cidx[wv], hist[wv]};
  int cnt = 0;
  uint32_t thr = 0;

  KeyTileRegs TR;
  load_key_tile_regs(TR, k8, 0, L, tid);
  store_key_tile_lds(TR, tiles[0], tid);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    if (t + 1 < ntiles) load_key_tile_regs(TR, k8, (int64_t)(t + 1) * KEY_TILE, L, tid);
    if (active) {
      const int64_t key = (int64_t)t * KEY_TILE + lane;
      const float ksc = ks[key < L ? key : L - 1];
      const float s = score_tile64(Q, lds_key_fragment(tiles[cur], 0), lds_key_fragment(tiles[cur], 1),
                                   lds_key_fragment(tiles[cur], 2), lds_key_fragment(tiles[cur], 3), ksc);
      const uint32_t u = score_key(s);
      const bool pass = key <= row && u > thr;
      const uint64_t m = ballot(pass);
      if (m) {
        if (pass) {
          const int off = cnt + (int)lanes_below(m);
          R.key[off] = u;
          R.idx[off] = (int32_t)key;
        }
        cnt += __popcll((unsigned long long)m);
        if (cnt > CAND - KEY_TILE) {
          __builtin_amdgcn_s_waitcnt(0xc07f);
          __builtin_amdgcn_wave_barrier();
          thr = select_compact(R, cnt, k);
          cnt = k;
        }
      }
    }
    if (t + 1 < ntiles) store_key_tile_lds(TR, tiles[cur ^ 1], tid);
    __syncthreads();
  }
  if (active) {
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    if (cnt > k) {
      select_compact(R, cnt, k);
      cnt = k;
    }
    int32_t* out = idx + row * (int64_t)k;
    for (int j = lane; j < k; j += WAVE) out[j] = j < cnt ? R.idx[j] : -1;
  }
}

// rows [0, n) keep every visible key: idx[t] = 0..t, -1 padded
__global__ __launch_bounds__(256) void prefill_fill_kernel(int64_t n, int k, int32_t* __restrict__ idx) {
  const int64_t t = blockIdx.x;
  if (t >= n) return;
  int32_t* out = idx + t * (int64_t)k;
  for (int j = threadIdx.x; j < k; j += 256) out[j] = j <= t ? j : -1;
}

hipError_t launch_prefill_topk(const PrefillTopkArgs& a, hipStream_t st) {
  const int64_t row_lo = a.k < a.L ? a.k : a.L;
  if (row_lo > 0)
    hipLaunchKernelGGL(prefill_fill_kernel, dim3((unsigned)row_lo), dim3(256), 0, st, row_lo, a.k, a.idx);
  const int64_t n_rows = a.L - row_lo;
  if (n_rows > 0) {
    dim3 grid((unsigned)((n_rows + 3) / 4));
    hipLaunchKernelGGL(prefill_idx_topk_kernel, grid, dim3(256), 0, st, a.q8, a.qs, a.k8, a.ks, a.w, a.L,
                       row_lo, a.k, a.idx);
  }
  return hipGetLastError();
}

}  // namespace dsa
