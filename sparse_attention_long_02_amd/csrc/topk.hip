// Fine-grained token selection over materialised scores (dsa_topk, decode).
//
// The kept set of a row is the top-k keys by (score desc, key index asc) among the keys
// the query may see (juhe.plus explainer, section 第二步：Fine-grained Token Selection).
// One 512-thread block owns one row:
//   1. exact radix select of the k-th largest order-preserving key, three passes over
//      the row with digits of 12, 12 and 8 bits (LDS histograms); this yields the
//      boundary key v* and how many keys equal to v* are kept (the lowest indices);
//   2. one more pass marks the kept keys in an LDS bitmap (and the ties at v* in a
//      second bitmap, of which only the first `take` bits survive);
//   3. a block-wide prefix count over the bitmap words writes the indices in ascending
//      order, -1 padded.  Everything is integer work on the fp32 bit patterns, so the
//      result is exactly the full-sort definition.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int TK_THREADS = 512;
constexpr int TK_WAVES = TK_THREADS / WAVE;
constexpr int TK_WORDS = (int)(TOPK_MAX_N / 32);
constexpr int TK_BINS = 4096;

// exclusive scan over the block; returns the prefix and writes the block total
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wtot, uint32_t& total) {
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == WAVE - 1) wtot[wv] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < TK_WAVES; ++i) {
    const uint32_t t = wtot[i];
    before += i < wv ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
}

__global__ __launch_bounds__(TK_THREADS) void topk_rows_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t n_rows, int64_t n_k,
    const int32_t* __restrict__ q_pos, int64_t pos_offset, int64_t row_begin, int k,
    int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[TK_BINS];
  __shared__ uint32_t sel[TK_WORDS];
  __shared__ uint32_t tie[TK_WORDS];
  __shared__ uint32_t wtot[TK_WAVES];
  __shared__ uint32_t s_digit, s_above;

  const int tid = threadIdx.x;
  const int64_t i = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t pos = (q_pos ? (int64_t)q_pos[b] : 0) + pos_offset + row_begin + i;
  int64_t n = pos + 1 < n_k ? pos + 1 : n_k;
  n = n > 0 ? n : 0;
  const float* srow = scores + ((int64_t)b * n_rows + i) * ld;
  int32_t* out = idx + ((int64_t)b * n_rows + i) * k;

  if (n <= k) {  // every visible key is kept
    for (int j = tid; j < k; j += TK_THREADS) out[j] = j < n ? j : -1;
    return;
  }

  // ---- 1. radix select: digits [31:20], [19:8], [7:0]
  uint32_t prefix = 0, pmask = 0;
  uint32_t rem = (uint32_t)k;
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
  for (int r = 0; r < 3; ++r) {
    const int shift = shifts[r];
    const uint32_t dmask = (1u << widths[r]) - 1u;
    const int nb = 1 << widths[r];
    for (int j = tid; j < nb; j += TK_THREADS) hist[j] = 0;
    __syncthreads();
    for (int64_t s = tid; s < n; s += TK_THREADS) {
      const uint32_t u = score_key(srow[s]);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread t owns the bins nb-1-t*per .. (descending); cumulative count from the top
    const int per = nb / TK_THREADS > 0 ? nb / TK_THREADS : 1;
    uint32_t local = 0;
    const int top = nb - 1 - tid * per;
    if (tid * per < nb)
      for (int j = 0; j < per; ++j) local += hist[top - j];
    uint32_t total;
    uint32_t c = block_excl_scan(local, wtot, total);
    if (tid * per < nb && c < rem && c + local >= rem) {
      for (int j = 0; j < per; ++j) {
        const uint32_t h = hist[top - j];
        if (c + h >= rem) {
          s_digit = (uint32_t)(top - j);
          s_above = c;
          break;
        }
        c += h;
      }
    }
    __syncthreads();
    const uint32_t d = s_digit;
    rem -= s_above;
    prefix |= d << shift;
    pmask |= dmask << shift;
    __syncthreads();
  }
  const uint32_t vstar = prefix;  // k-th largest key; `rem` keys equal to it are kept

  // ---- 2. mark kept keys and ties
  const int64_t nw = (n + 31) / 32;
  for (int64_t j = tid; j < nw; j += TK_THREADS) {
    sel[j] = 0;
    tie[j] = 0;
  }
  __syncthreads();
  for (int64_t s = tid; s < n; s += TK_THREADS) {
    const uint32_t u = score_key(srow[s]);
    if (u > vstar) atomicOr(&sel[s >> 5], 1u << (s & 31));
    else if (u == vstar) atomicOr(&tie[s >> 5], 1u << (s & 31));
  }
  __syncthreads();

  // ---- 3. keep the first `rem` ties, then write the kept indices in ascending order
  const int64_t wpt = (nw + TK_THREADS - 1) / TK_THREADS;
  const int64_t w0 = tid * wpt;
  const int64_t w1 = w0 + wpt < nw ? w0 + wpt : nw;
  uint32_t tcount = 0;
  for (int64_t j = w0; j < w1; ++j) tcount += __popc(tie[j]);
  uint32_t tot;
  uint32_t tbefore = block_excl_scan(tcount, wtot, tot);
  for (int64_t j = w0; j < w1; ++j) {
    uint32_t m = tie[j];
    while (m) {
      const uint32_t bit = m & (0u - m);
      if (tbefore < rem) sel[j] |= bit;
      ++tbefore;
      m ^= bit;
    }
  }
  uint32_t scount = 0;
  for (int64_t j = w0; j < w1; ++j) scount += __popc(sel[j]);
  uint32_t o = block_excl_scan(scount, wtot, tot);
  for (int64_t j = w0; j < w1; ++j) {
    uint32_t m = sel[j];
    while (m) {
      const int bitpos = __ffs(m) - 1;
      if (o < (uint32_t)k) out[o] = (int32_t)(j * 32 + bitpos);
      ++o;
      m &= m - 1;
    }
  }
  for (int64_t j = (int64_t)tot + tid; j < k; j += TK_THREADS) out[j] = -1;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  dim3 grid((unsigned)a.n_rows, (unsigned)a.B);
  hipLaunchKernelGGL(topk_rows_kernel, grid, dim3(TK_THREADS), 0, st, a.scores, a.ld_scores,
                     a.n_rows, a.n_k, a.q_pos, a.pos_offset, a.row_begin, a.k, a.idx);
  return hipGetLastError();
}

}  // namespace dsa
