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
constexpr int TK_WORDS = (int)(TOPK_MAX_N / 32);
constexpr int TK_BINS = 4096;

// exclusive scan over a block of NT threads; returns the prefix and writes the block total
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wtot, uint32_t& total) {
  constexpr int NW = NT / WAVE;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const uint32_t incl = wave_incl_scan(v);
  if (lane == WAVE - 1) wtot[wv] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t t = wtot[i];
    before += i < wv ? t : 0u;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
}

// Block-wide choice of the digit holding the rem-th largest key from a histogram of nb
// bins (thread t owns bins nb-1-t*per .. downward).  Returns the digit; `above` = keys in
// higher bins.
template <int NT>
__device__ __forceinline__ uint32_t pick_digit(const uint32_t* hist, int nb, uint32_t rem, uint32_t* wtot,
                                               uint32_t* s_digit, uint32_t* s_above, uint32_t& above) {
  const int tid = threadIdx.x;
  const int per = nb / NT > 0 ? nb / NT : 1;
  uint32_t local = 0;
  const int top = nb - 1 - tid * per;
  if (tid * per < nb)
    for (int j = 0; j < per; ++j) local += hist[top - j];
  uint32_t total;
  uint32_t c = block_excl_scan<NT>(local, wtot, total);
  if (tid * per < nb && c < rem && c + local >= rem) {
    for (int j = 0; j < per; ++j) {
      const uint32_t h = hist[top - j];
      if (c + h >= rem) {
        *s_digit = (uint32_t)(top - j);
        *s_above = c;
        break;
      }
      c += h;
    }
  }
  __syncthreads();
  above = *s_above;
  const uint32_t d = *s_digit;
  __syncthreads();
  return d;
}

// Exact radix select over the visible part of a score row: the k-th largest key v* and
// how many keys equal to v* are kept (digits of 12, 12 and 8 bits, LDS histograms).
template <int NT>
__device__ void select_row(const float* __restrict__ srow, int64_t n, int k, uint32_t* hist, uint32_t* wtot,
                           uint32_t* s_digit, uint32_t* s_above, uint32_t& vstar, uint32_t& rem) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  rem = (uint32_t)k;
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
  for (int r = 0; r < 3; ++r) {
    const int shift = shifts[r];
    const uint32_t dmask = (1u << widths[r]) - 1u;
    const int nb = 1 << widths[r];
    for (int j = tid; j < nb; j += NT) hist[j] = 0;
    __syncthreads();
    for (int64_t s = tid; s < n; s += NT) {
      const uint32_t u = score_key(srow[s]);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1u);
    }
    __syncthreads();
    uint32_t above;
    const uint32_t d = pick_digit<NT>(hist, nb, rem, wtot, s_digit, s_above, above);
    rem -= above;
    prefix |= d << shift;
    pmask |= dmask << shift;
  }
  vstar = prefix;
}

// Exact radix select of the rank-th largest of n keys held in LDS (8-bit digits).
template <int NT>
__device__ uint32_t select_lds(const uint32_t* keys, int n, uint32_t rank, uint32_t* hist, uint32_t* wtot,
                               uint32_t* s_digit, uint32_t* s_above, uint32_t& rem) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  rem = rank;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int j = tid; j < 256; j += NT) hist[j] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t u = keys[i];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    uint32_t above;
    const uint32_t d = pick_digit<NT>(hist, 256, rem, wtot, s_digit, s_above, above);
    rem -= above;
    prefix |= d << shift;
    pmask |= 255u << shift;
  }
  return prefix;
}

// Keep the first `rem` ties (lowest positions), then write the kept positions in ascending
// order, -1 padded.  sel / tie: bitmaps over the row's n positions.
template <int NT>
__device__ void write_kept(uint32_t* sel, const uint32_t* tie, int64_t n, uint32_t rem, int k, int32_t* out,
                           uint32_t* wtot) {
  const int tid = threadIdx.x;
  const int64_t nw = (n + 31) / 32;
  const int64_t wpt = (nw + NT - 1) / NT;
  const int64_t w0 = tid * wpt;
  const int64_t w1 = w0 + wpt < nw ? w0 + wpt : nw;
  uint32_t tcount = 0;
  for (int64_t j = w0; j < w1; ++j) tcount += __popc(tie[j]);
  uint32_t tot;
  uint32_t tbefore = block_excl_scan<NT>(tcount, wtot, tot);
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
  uint32_t o = block_excl_scan<NT>(scount, wtot, tot);
  for (int64_t j = w0; j < w1; ++j) {
    uint32_t m = sel[j];
    while (m) {
      const int bitpos = __ffs(m) - 1;
      if (o < (uint32_t)k) out[o] = (int32_t)(j * 32 + bitpos);
      ++o;
      m &= m - 1;
    }
  }
  for (int64_t j = (int64_t)tot + tid; j < k; j += NT) out[j] = -1;
}

// mark every visible key > v* in sel and every key == v* in tie (bitmaps zeroed first)
template <int NT>
__device__ void mark_row(const float* __restrict__ srow, int64_t n, uint32_t vstar, uint32_t* sel, uint32_t* tie) {
  const int tid = threadIdx.x;
  const int64_t nw = (n + 31) / 32;
  for (int64_t j = tid; j < nw; j += NT) {
    sel[j] = 0;
    tie[j] = 0;
  }
  __syncthreads();
  for (int64_t s = tid; s < n; s += NT) {
    const uint32_t u = score_key(srow[s]);
    if (u > vstar) atomicOr(&sel[s >> 5], 1u << (s & 31));
    else if (u == vstar) atomicOr(&tie[s >> 5], 1u << (s & 31));
  }
  __syncthreads();
}

__device__ __forceinline__ void row_geometry(int64_t n_rows, int64_t n_k, const int32_t* q_pos, int64_t pos_offset,
                                             int64_t row_begin, int k, int64_t ld, const float* scores,
                                             int32_t* idx, int64_t& n, const float*& srow, int32_t*& out) {
  const int64_t i = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t pos = (q_pos ? (int64_t)q_pos[b] : 0) + pos_offset + row_begin + i;
  n = pos + 1 < n_k ? pos + 1 : n_k;
  n = n > 0 ? n : 0;
  srow = scores + ((int64_t)b * n_rows + i) * ld;
  out = idx + ((int64_t)b * n_rows + i) * k;
}

// One 512-thread block per row (rows of any length):
//   1. exact radix select of v* over the whole row;  2. mark kept keys and ties in LDS
//   bitmaps;  3. ascending write.
__global__ __launch_bounds__(TK_THREADS) void topk_rows_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t n_rows, int64_t n_k,
    const int32_t* __restrict__ q_pos, int64_t pos_offset, int64_t row_begin, int k,
    int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[TK_BINS];
  __shared__ uint32_t sel[TK_WORDS];
  __shared__ uint32_t tie[TK_WORDS];
  __shared__ uint32_t wtot[TK_THREADS / WAVE];
  __shared__ uint32_t s_digit, s_above;
  int64_t n;
  const float* srow;
  int32_t* out;
  row_geometry(n_rows, n_k, q_pos, pos_offset, row_begin, k, ld, scores, idx, n, srow, out);
  const int tid = threadIdx.x;
  if (n <= k) {  // every visible key is kept
    for (int j = tid; j < k; j += TK_THREADS) out[j] = j < n ? j : -1;
    return;
  }
  uint32_t vstar, rem;
  select_row<TK_THREADS>(srow, n, k, hist, wtot, &s_digit, &s_above, vstar, rem);
  mark_row<TK_THREADS>(srow, n, vstar, sel, tie);
  write_kept<TK_THREADS>(sel, tie, n, rem, k, out, wtot);
}

// Long rows with a small k: one 1024-thread block per row.
//   1. a threshold T from 4096 evenly spaced samples of the row (the sample key of rank
//      about twice the k-th key's expected rank), so that roughly 2k keys exceed it;
//   2. one pass appends the keys > T (key, position) to an LDS candidate buffer;
//   3. if at least k and at most TL_CAP keys exceed T, the k-th largest key is > T, so
//      v* and every key equal to it are among the candidates: the exact select runs on
//      them alone.  Otherwise (an unlucky sample, heavy ties) the exact full-row select
//      runs instead.  Either way the result is the exact top-k.
constexpr int TL_THREADS = 1024;
constexpr int TL_SAMPLES = 4096;
constexpr int TL_CAP = 8192;
constexpr int TL_BATCH = 8;
constexpr int TL_MIN_N = 16384;  // rows at least this long (and k <= TL_CAP / 4) use it

__global__ __launch_bounds__(TL_THREADS) void topk_long_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t n_rows, int64_t n_k,
    const int32_t* __restrict__ q_pos, int64_t pos_offset, int64_t row_begin, int k,
    int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[TK_BINS];
  __shared__ uint32_t sel[TK_WORDS];
  __shared__ uint32_t tie[TK_WORDS];
  __shared__ uint32_t ckey[TL_CAP];  // samples first, then candidate keys
  __shared__ int32_t cpos[TL_CAP];
  __shared__ uint32_t wtot[TL_THREADS / WAVE];
  __shared__ uint32_t s_digit, s_above, s_cnt;
  int64_t n;
  const float* srow;
  int32_t* out;
  row_geometry(n_rows, n_k, q_pos, pos_offset, row_begin, k, ld, scores, idx, n, srow, out);
  const int tid = threadIdx.x;
  if (n <= k) {
    for (int j = tid; j < k; j += TL_THREADS) out[j] = j < n ? j : -1;
    return;
  }
  // 1. threshold from the samples
  for (int j = tid; j < TL_SAMPLES; j += TL_THREADS) ckey[j] = score_key(srow[((int64_t)j * n) / TL_SAMPLES]);
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  const int64_t expect = ((int64_t)k * TL_SAMPLES + n - 1) / n;  // sample rank of the k-th key
  const uint32_t srank = (uint32_t)min<int64_t>(TL_SAMPLES, 2 * expect + 16);
  uint32_t srem;
  const uint32_t T = select_lds<TL_THREADS>(ckey, TL_SAMPLES, srank, hist, wtot, &s_digit, &s_above, srem);
  // 2. candidates: keys > T (TL_BATCH independent loads in flight per thread)
  for (int64_t s0 = 0; s0 < n; s0 += (int64_t)TL_THREADS * TL_BATCH) {
    float v[TL_BATCH];
#pragma unroll
    for (int q = 0; q < TL_BATCH; ++q) {
      const int64_t s = s0 + (int64_t)q * TL_THREADS + tid;
      v[q] = s < n ? srow[s] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < TL_BATCH; ++q) {
      const int64_t s = s0 + (int64_t)q * TL_THREADS + tid;
      const uint32_t u = score_key(v[q]);
      const bool pass = s < n && u > T;
      const uint64_t m = ballot(pass);
      uint32_t base = 0;
      if ((tid & 63) == 0 && m) base = atomicAdd(&s_cnt, (uint32_t)__popcll((unsigned long long)m));
      base = __shfl(base, 0, WAVE);
      if (pass) {
        const uint32_t slot = base + lanes_below(m);
        if (slot < (uint32_t)TL_CAP) {
          ckey[slot] = u;
          cpos[slot] = (int32_t)s;
        }
      }
    }
  }
  __syncthreads();
  const uint32_t nc = s_cnt;
  uint32_t vstar, rem;
  if (nc < (uint32_t)k || nc > (uint32_t)TL_CAP) {
    // 3b. the threshold did not bracket the k-th key: exact select over the whole row
    select_row<TL_THREADS>(srow, n, k, hist, wtot, &s_digit, &s_above, vstar, rem);
    mark_row<TL_THREADS>(srow, n, vstar, sel, tie);
  } else {
    // 3a. exact select among the candidates, then mark them
    vstar = select_lds<TL_THREADS>(ckey, (int)nc, (uint32_t)k, hist, wtot, &s_digit, &s_above, rem);
    const int64_t nw = (n + 31) / 32;
    for (int64_t j = tid; j < nw; j += TL_THREADS) {
      sel[j] = 0;
      tie[j] = 0;
    }
    __syncthreads();
    for (int c = tid; c < (int)nc; c += TL_THREADS) {
      const uint32_t u = ckey[c];
      const int32_t sp = cpos[c];
      if (u > vstar) atomicOr(&sel[sp >> 5], 1u << (sp & 31));
      else if (u == vstar) atomicOr(&tie[sp >> 5], 1u << (sp & 31));
    }
    __syncthreads();
  }
  write_kept<TL_THREADS>(sel, tie, n, rem, k, out, wtot);
}

// ---------------------------------------------------------------------------------------
// Ordered-candidate top-k (rows of any length, k <= TO_CAP / 2).  One 512-thread block per
// row and about 33 KB of LDS, so four blocks share a CU and keep 128 KB of score loads in
// flight:
//   1. a threshold T: a row of at most TO_CAP keys takes every key; a longer row takes the
//      sample key of rank about 1.5 k * TO_CAP / n among TO_CAP evenly spaced samples, so
//      that about 1.5 k keys exceed it;
//   2. one pass over the row collects the keys > T, with their positions, in ascending
//      position order: each thread reads TO_PER consecutive scores and a block scan of the
//      per-thread counts places them;
//   3. if at least k and at most TO_CAP keys exceed T, the k-th largest key v* and every
//      key equal to it are among the candidates: a radix select over the candidates gives
//      v* and how many keys equal to v* are kept (the lowest positions), and an ordered
//      pass over the candidates writes the kept positions ascending;
//   4. otherwise (an unlucky sample, heavy ties) the exact select runs over the whole row
//      and the ordered pass runs over the row itself.
// The result is the full-sort definition either way.
// ---------------------------------------------------------------------------------------
constexpr int TO_THREADS = 512;
constexpr int TO_CAP = 4096;
constexpr int TO_PER = 8;
constexpr int TO_STEP = TO_THREADS * TO_PER;

// scores p0 .. p0+TO_PER-1 of a row (positions >= n read as -inf and are never taken)
__device__ __forceinline__ void load_run(const float* __restrict__ srow, int64_t p0, int64_t n, bool vec,
                                         float v[TO_PER]) {
  if (vec && p0 + TO_PER <= n) {
    const float4* p = reinterpret_cast<const float4*>(srow + p0);
#pragma unroll
    for (int q = 0; q < TO_PER / 4; ++q) {
      const float4 x = p[q];
      v[4 * q] = x.x;
      v[4 * q + 1] = x.y;
      v[4 * q + 2] = x.z;
      v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < TO_PER; ++e) v[e] = p0 + e < n ? srow[p0 + e] : -INFINITY;
  }
}

// Keys > T (every key if `all`) in ascending position order into ckey/cpos (slots past
// TO_CAP are counted, not stored).  Returns the count.
__device__ uint32_t collect_ordered(const float* __restrict__ srow, int64_t n, bool vec, bool all, uint32_t T,
                                    uint32_t* ckey, int32_t* cpos, uint32_t* wtot) {
  const int tid = threadIdx.x;
  uint32_t nc = 0;
  for (int64_t s0 = 0; s0 < n; s0 += TO_STEP) {
    const int64_t p0 = s0 + (int64_t)TO_PER * tid;
    float v[TO_PER];
    load_run(srow, p0, n, vec, v);
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < TO_PER; ++e) m |= (uint32_t)((p0 + e < n) & (all | (score_key(v[e]) > T))) << e;
    uint32_t tot;
    uint32_t slot = nc + block_excl_scan<TO_THREADS>((uint32_t)__popc(m), wtot, tot);
#pragma unroll
    for (int e = 0; e < TO_PER; ++e)
      if ((m >> e) & 1u) {
        if (slot < (uint32_t)TO_CAP) {
          ckey[slot] = score_key(v[e]);
          cpos[slot] = (int32_t)(p0 + e);
        }
        ++slot;
      }
    nc += tot;
  }
  __syncthreads();
  return nc;
}

// Kept candidates (keys > v*, then the first `rem` keys equal to v* in position order)
// written ascending to out, -1 padded to k.
__device__ void write_from_candidates(const uint32_t* ckey, const int32_t* cpos, uint32_t nc, uint32_t vstar,
                                      uint32_t rem, int k, int32_t* __restrict__ out, uint32_t* wtot) {
  const uint32_t tid = threadIdx.x;
  const uint32_t m = (nc + TO_THREADS - 1) / TO_THREADS;
  const uint32_t j0 = min(tid * m, nc), j1 = min(j0 + m, nc);
  uint32_t ties = 0;
  for (uint32_t j = j0; j < j1; ++j) ties += ckey[j] == vstar;
  uint32_t tt;
  const uint32_t tb = block_excl_scan<TO_THREADS>(ties, wtot, tt);
  uint32_t kc = 0, tr = tb;
  for (uint32_t j = j0; j < j1; ++j) {
    const uint32_t u = ckey[j];
    kc += (u > vstar) | ((u == vstar) & (tr < rem));
    tr += u == vstar;
  }
  uint32_t tot;
  uint32_t o = block_excl_scan<TO_THREADS>(kc, wtot, tot);
  tr = tb;
  for (uint32_t j = j0; j < j1; ++j) {
    const uint32_t u = ckey[j];
    const bool keep = (u > vstar) | ((u == vstar) & (tr < rem));
    tr += u == vstar;
    if (keep) {
      if (o < (uint32_t)k) out[o] = cpos[j];
      ++o;
    }
  }
  for (int64_t j = (int64_t)tot + tid; j < k; j += TO_THREADS) out[j] = -1;
}

// Exact radix select of the k-th largest key of a whole row (8-bit digits, four passes).
__device__ uint32_t select_row8(const float* __restrict__ srow, int64_t n, bool vec, int k, uint32_t* hist,
                                uint32_t* wtot, uint32_t* s_digit, uint32_t* s_above, uint32_t& rem) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  rem = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int j = tid; j < 256; j += TO_THREADS) hist[j] = 0;
    __syncthreads();
    for (int64_t s0 = 0; s0 < n; s0 += TO_STEP) {
      const int64_t p0 = s0 + (int64_t)TO_PER * tid;
      float v[TO_PER];
      load_run(srow, p0, n, vec, v);
#pragma unroll
      for (int e = 0; e < TO_PER; ++e) {
        const uint32_t u = score_key(v[e]);
        if ((p0 + e < n) && (u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    uint32_t above;
    const uint32_t d = pick_digit<TO_THREADS>(hist, 256, rem, wtot, s_digit, s_above, above);
    rem -= above;
    prefix |= d << shift;
    pmask |= 255u << shift;
  }
  return prefix;
}

// The kept keys of a whole row (keys > v*, then the first `rem` equal to v*) written ascending.
__device__ void write_from_row(const float* __restrict__ srow, int64_t n, bool vec, uint32_t vstar, uint32_t rem,
                               int k, int32_t* __restrict__ out, uint32_t* wtot) {
  const int tid = threadIdx.x;
  uint32_t o_base = 0, t_base = 0;
  for (int64_t s0 = 0; s0 < n; s0 += TO_STEP) {
    const int64_t p0 = s0 + (int64_t)TO_PER * tid;
    float v[TO_PER];
    load_run(srow, p0, n, vec, v);
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < TO_PER; ++e) {
      const uint32_t u = score_key(v[e]);
      const bool in = p0 + e < n;
      gt |= (uint32_t)(in & (u > vstar)) << e;
      eq |= (uint32_t)(in & (u == vstar)) << e;
    }
    uint32_t tt;
    const uint32_t tb = t_base + block_excl_scan<TO_THREADS>((uint32_t)__popc(eq), wtot, tt);
    // ties of this thread that are still within the first `rem`
    const uint32_t take = tb < rem ? min((uint32_t)__popc(eq), rem - tb) : 0u;
    uint32_t keep = gt, left = take;
#pragma unroll
    for (int e = 0; e < TO_PER; ++e)
      if (((eq >> e) & 1u) && left) {
        keep |= 1u << e;
        --left;
      }
    uint32_t tot;
    uint32_t o = o_base + block_excl_scan<TO_THREADS>((uint32_t)__popc(keep), wtot, tot);
#pragma unroll
    for (int e = 0; e < TO_PER; ++e)
      if ((keep >> e) & 1u) {
        if (o < (uint32_t)k) out[o] = (int32_t)(p0 + e);
        ++o;
      }
    o_base += tot;
    t_base += tt;
  }
  for (int64_t j = (int64_t)o_base + tid; j < k; j += TO_THREADS) out[j] = -1;
}

// grid (n_rows, B), longest rows first.  Row i of sequence b: scores at
// scores + (b * score_rows + i) * ld, position q_pos[b] + pos_offset + row_begin + i, output
// row out_row0 + i of sequence b's out_rows rows.
__global__ __launch_bounds__(TO_THREADS) __attribute__((amdgpu_waves_per_eu(8))) void topk_ordered_kernel(
    const float* __restrict__ scores, int64_t ld, int64_t score_rows, int64_t n_rows, int64_t n_k,
    const int32_t* __restrict__ q_pos, int64_t pos_offset, int64_t row_begin, int k, int32_t* __restrict__ idx,
    int64_t out_rows, int64_t out_row0) {
  __shared__ uint32_t ckey[TO_CAP];  // samples first, then candidate keys
  __shared__ int32_t cpos[TO_CAP];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wtot[TO_THREADS / WAVE];
  __shared__ uint32_t s_digit, s_above;
  const int64_t i = n_rows - 1 - (int64_t)blockIdx.x;
  const int b = blockIdx.y;
  const int64_t pos = (q_pos ? (int64_t)q_pos[b] : 0) + pos_offset + row_begin + i;
  int64_t n = pos + 1 < n_k ? pos + 1 : n_k;
  n = n > 0 ? n : 0;
  const float* srow = scores + ((int64_t)b * score_rows + i) * ld;
  int32_t* out = idx + ((int64_t)b * out_rows + out_row0 + i) * k;
  const int tid = threadIdx.x;
  if (n <= k) {  // every visible key is kept
    for (int j = tid; j < k; j += TO_THREADS) out[j] = j < n ? j : -1;
    return;
  }
  const bool vec = ((uintptr_t)srow & 15u) == 0;
  const bool all = n <= TO_CAP;
  uint32_t T = 0;
  if (!all) {
    for (int j = tid; j < TO_CAP; j += TO_THREADS) ckey[j] = score_key(srow[((int64_t)j * n) / TO_CAP]);
    __syncthreads();
    int64_t srank = (3 * (int64_t)k * TO_CAP + n) / (2 * n);  // about 1.5 k keys above
    srank = srank < 1 ? 1 : srank > TO_CAP ? TO_CAP : srank;
    uint32_t srem;
    T = select_lds<TO_THREADS>(ckey, TO_CAP, (uint32_t)srank, hist, wtot, &s_digit, &s_above, srem);
  }
  const uint32_t nc = collect_ordered(srow, n, vec, all, T, ckey, cpos, wtot);
  uint32_t vstar, rem;
  if (nc >= (uint32_t)k && nc <= (uint32_t)TO_CAP) {
    vstar = select_lds<TO_THREADS>(ckey, (int)nc, (uint32_t)k, hist, wtot, &s_digit, &s_above, rem);
    write_from_candidates(ckey, cpos, nc, vstar, rem, k, out, wtot);
  } else {
    vstar = select_row8(srow, n, vec, k, hist, wtot, &s_digit, &s_above, rem);
    write_from_row(srow, n, vec, vstar, rem, k, out, wtot);
  }
}

hipError_t launch_topk_ordered(const TopkArgs& a, hipStream_t st) {
  if (a.n_rows <= 0 || a.B <= 0) return hipSuccess;
  dim3 grid((unsigned)a.n_rows, (unsigned)a.B);
  hipLaunchKernelGGL(topk_ordered_kernel, grid, dim3(TO_THREADS), 0, st, a.scores, a.ld_scores,
                     a.score_rows ? a.score_rows : a.n_rows, a.n_rows, a.n_k, a.q_pos, a.pos_offset, a.row_begin,
                     a.k, a.idx, a.out_rows ? a.out_rows : a.n_rows, a.out_row0);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  dim3 grid((unsigned)a.n_rows, (unsigned)a.B);
  if (a.n_k >= TL_MIN_N && a.k <= TL_CAP / 4)
    hipLaunchKernelGGL(topk_long_kernel, grid, dim3(TL_THREADS), 0, st, a.scores, a.ld_scores, a.n_rows, a.n_k,
                       a.q_pos, a.pos_offset, a.row_begin, a.k, a.idx);
  else
    hipLaunchKernelGGL(topk_rows_kernel, grid, dim3(TK_THREADS), 0, st, a.scores, a.ld_scores, a.n_rows, a.n_k,
                       a.q_pos, a.pos_offset, a.row_begin, a.k, a.idx);
  return hipGetLastError();
}

}  // namespace dsa
