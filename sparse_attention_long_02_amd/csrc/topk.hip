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

// Exact radix select of the rank-th largest of n keys held in LDS (1 <= rank <= n).  The
// bits every key shares (found by a block-wide AND / OR) are skipped; the rest are resolved
// in digits of up to 8 bits from the top.  Candidate lists span a narrow range of scores,
// so this drops a pass and, with it, a pass whose few busy bins would serialise the LDS
// atomics.  Returns v*; rem = how many keys equal to v* are kept.
template <int NT>
__device__ uint32_t select_lds(const uint32_t* keys, int n, uint32_t rank, uint32_t* hist, uint32_t* wtot,
                               uint32_t* s_digit, uint32_t* s_above, uint32_t& rem) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    hist[0] = 0xFFFFFFFFu;
    hist[1] = 0u;
  }
  __syncthreads();
  uint32_t ka = 0xFFFFFFFFu, ko = 0u;
  for (int i = tid; i < n; i += NT) {
    ka &= keys[i];
    ko |= keys[i];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ka &= (uint32_t)__shfl_xor((int)ka, off, WAVE);
    ko |= (uint32_t)__shfl_xor((int)ko, off, WAVE);
  }
  if ((tid & (WAVE - 1)) == 0) {
    atomicAnd(&hist[0], ka);
    atomicOr(&hist[1], ko);
  }
  __syncthreads();
  ka = hist[0];
  ko = hist[1];
  __syncthreads();
  rem = rank;
  const uint32_t diff = ka ^ ko;
  if (diff == 0u) return ka;  // every key is equal
  int top = 32 - __clz(diff);  // bits below `top` vary
  uint32_t pmask = top == 32 ? 0u : ~((1u << top) - 1u);
  uint32_t prefix = ka & pmask;
  while (top > 0) {
    const int width = top < 8 ? top : 8;
    const int shift = top - width;
    const int nb = 1 << width;
    const uint32_t dmask = (uint32_t)nb - 1u;
    for (int j = tid; j < nb; j += NT) hist[j] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t u = keys[i];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1u);
    }
    __syncthreads();
    uint32_t above;
    const uint32_t d = pick_digit<NT>(hist, nb, rem, wtot, s_digit, s_above, above);
    rem -= above;
    prefix |= d << shift;
    pmask |= dmask << shift;
    top = shift;
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
    int32_t* __restrict__ idx, const uint8_t* __restrict__ redo) {
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
  if (redo && !redo[(int64_t)blockIdx.y * n_rows + blockIdx.x]) return;  // uniform over the block
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

// blocks that select over an LDS candidate list
constexpr int TO_THREADS = 512;

// Kept candidates (keys > v*, then the first `rem` keys equal to v* in position order)
// written ascending to out, -1 padded to k; pos(j) is candidate j's key index.
template <typename Pos>
__device__ void write_from_candidates(const uint32_t* ckey, Pos pos, uint32_t nc, uint32_t vstar, uint32_t rem,
                                      int k, int32_t* __restrict__ out, uint32_t* wtot) {
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
      if (o < (uint32_t)k) out[o] = pos(j);
      ++o;
    }
  }
  for (int64_t j = (int64_t)tot + tid; j < k; j += TO_THREADS) out[j] = -1;
}

// ---------------------------------------------------------------------------------------
// Threshold-filtered selection.  The filtering indexer keeps, for each row, only the keys
// whose score reaches a threshold set from a systematic 1-in-SEL_SAMPLE_STRIDE key sample,
// so the row's top-k is decided from a short candidate list and no full score row is ever
// stored.  The threshold is the sample of rank r = ceil(m + 5 sqrt(m) + 5), m = k n_s / n
// (the expected number of samples among the row's top k): with r far above m the
// candidates almost always include the whole top-k, and with cap / stride samples expected
// above the cap's boundary, almost never overflow the SEL_CAND_CAP slots.  Either miss is
// detected exactly (fewer than k candidates, or more than the cap) and the row is
// recomputed by the streaming exact selection, so the result never depends on the sample.
// ---------------------------------------------------------------------------------------
constexpr int TH_THREADS = 256;
constexpr int LOAD_BATCH = 8;  // loads per thread in flight while a list is staged in LDS
constexpr int TH_MAX = (int)(TOPK_MAX_N / SEL_SAMPLE_STRIDE);

// The row's sample keys live in dynamic LDS of ceil(n_k / SEL_SAMPLE_STRIDE) words (16 KB at
// 131072 keys), so that many blocks share a CU.
template <int NT>
__global__ __launch_bounds__(NT) void sel_threshold_kernel(const float* __restrict__ samp, int64_t ld_s,
                                                                   int64_t rows_pad, int64_t n_rows, int64_t n_k,
                                                                   const int32_t* __restrict__ q_pos,
                                                                   int64_t row_begin, int k,
                                                                   float* __restrict__ thr) {
  extern __shared__ uint32_t keys[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wtot[NT / WAVE];
  __shared__ uint32_t s_digit, s_above;
  const int64_t i = n_rows - 1 - (int64_t)blockIdx.x;
  const int b = blockIdx.y;
  const int64_t pos = (q_pos ? (int64_t)q_pos[b] : 0) + row_begin + i;
  int64_t n = pos + 1 < n_k ? pos + 1 : n_k;
  n = n > 0 ? n : 0;
  float* out = thr + (int64_t)b * rows_pad + i;
  const int tid = threadIdx.x;
  if (n <= SEL_CAND_CAP) {  // the list holds every key the row sees
    if (tid == 0) *out = -INFINITY;
    return;
  }
  const int ns = (int)((n - 1) / SEL_SAMPLE_STRIDE + 1);
  const float m = (float)k * (float)ns / (float)n;
  int r = (int)ceilf(m + 5.f * sqrtf(m) + 5.f);
  r = r < ns ? r : ns;
  const float* srow = samp + ((int64_t)b * rows_pad + i) * ld_s;
  // the samples -> LDS, LOAD_BATCH loads per thread in flight before any is stored
  for (int j0 = 0; j0 < ns; j0 += LOAD_BATCH * NT) {
    float v[LOAD_BATCH];
#pragma unroll
    for (int q = 0; q < LOAD_BATCH; ++q) {
      const int j = j0 + q * NT + tid;
      v[q] = j < ns ? srow[j] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < LOAD_BATCH; ++q) {
      const int j = j0 + q * NT + tid;
      if (j < ns) keys[j] = score_key(v[q]);
    }
  }
  __syncthreads();
  uint32_t rem;
  const uint32_t T = select_lds<NT>(keys, ns, (uint32_t)r, hist, wtot, &s_digit, &s_above, rem);
  // the filter keeps the keys scoring strictly above this sample (the key is mapped back to
  // its fp32 value; a -0 sample was read as +0, and the two compare equal anyway)
  if (tid == 0) *out = __uint_as_float((T & 0x80000000u) ? (T & 0x7FFFFFFFu) : ~T);
}

__global__ __launch_bounds__(TO_THREADS) void sel_candidates_kernel(
    const uint2* __restrict__ cand, const uint32_t* __restrict__ cnt, int64_t rows_pad, int64_t n_rows, int64_t n_k,
    const int32_t* __restrict__ q_pos, int64_t row_begin, int k, int32_t* __restrict__ idx, int64_t out_rows,
    int64_t out_row0, uint8_t* __restrict__ redo) {
  // the candidates' score keys and key indices in LDS (48 KB, so three blocks share a CU):
  // the list is read from memory once
  __shared__ uint32_t ckey[SEL_CAND_CAP];
  __shared__ int32_t cidx[SEL_CAND_CAP];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wtot[TO_THREADS / WAVE];
  __shared__ uint32_t s_digit, s_above;
  const int64_t i = n_rows - 1 - (int64_t)blockIdx.x;
  const int b = blockIdx.y;
  const int64_t pos = (q_pos ? (int64_t)q_pos[b] : 0) + row_begin + i;
  int64_t n = pos + 1 < n_k ? pos + 1 : n_k;
  n = n > 0 ? n : 0;
  const int64_t orow = (int64_t)b * out_rows + out_row0 + i;
  int32_t* out = idx + orow * k;
  const int tid = threadIdx.x;
  if (n <= k) {  // every visible key is kept
    for (int j = tid; j < k; j += TO_THREADS) out[j] = j < n ? j : -1;
    if (tid == 0) redo[orow] = 0;
    return;
  }
  const int64_t r = (int64_t)b * rows_pad + i;
  const uint32_t c = cnt[r];
  if (c < (uint32_t)k || c > (uint32_t)SEL_CAND_CAP) {  // the list does not decide the row
    if (tid == 0) redo[orow] = 1;
    return;
  }
  // the list -> LDS, every load of a thread in flight before any is stored
  const uint2* cr = cand + r * SEL_CAND_PITCH;
  constexpr int PER = SEL_CAND_CAP / TO_THREADS;
  static_assert(SEL_CAND_CAP % TO_THREADS == 0, "the list splits evenly over the threads");
  uint2 e[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const uint32_t j = (uint32_t)(q * TO_THREADS + tid);
    e[q] = j < c ? cr[j] : make_uint2(0u, 0u);
  }
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const uint32_t j = (uint32_t)(q * TO_THREADS + tid);
    if (j < c) {
      ckey[j] = score_key(__uint_as_float(e[q].x));
      cidx[j] = (int32_t)e[q].y;
    }
  }
  __syncthreads();
  uint32_t rem;
  const uint32_t vstar = select_lds<TO_THREADS>(ckey, (int)c, (uint32_t)k, hist, wtot, &s_digit, &s_above, rem);
  write_from_candidates(ckey, [](uint32_t j) { return cidx[j]; }, c, vstar, rem, k, out, wtot);
  if (tid == 0) redo[orow] = 0;
}

// Decode: the top-k of each row's candidate segments (the filtering split indexer's).  When
// no segment overflowed and k <= total <= SEL_CAND_CAP, the segments hold every key above the
// threshold, and at least k of them, so v* (the k-th largest score) and every key equal to
// it are among them: the segments are packed into LDS, an exact select gives v*, and LDS
// bitmaps over the row's positions put the kept keys (and the lowest-positioned ties) in
// ascending order.  Otherwise the row is marked for the exact full-row selection.
constexpr int DC_THREADS = 1024;
constexpr int DC_MAX_SEGS = (int)(4 * (TOPK_MAX_N / (SPLIT_TILES * 64)));
__global__ __launch_bounds__(DC_THREADS) void dec_cand_topk_kernel(
    const uint2* __restrict__ cand, const uint32_t* __restrict__ cnt, int64_t n_segs, int64_t n_rows, int64_t n_k,
    const int32_t* __restrict__ q_pos, int64_t pos_offset, int k, int32_t* __restrict__ idx,
    uint8_t* __restrict__ redo) {
  __shared__ uint32_t hist[TK_BINS];
  __shared__ uint32_t sel[TK_WORDS];
  __shared__ uint32_t tie[TK_WORDS];
  __shared__ uint32_t ckey[SEL_CAND_CAP];
  __shared__ int32_t cpos[SEL_CAND_CAP];
  __shared__ uint32_t soff[DC_MAX_SEGS + 1];
  __shared__ uint32_t wtot[DC_THREADS / WAVE];
  __shared__ uint32_t s_digit, s_above, s_bad;
  const int64_t i = blockIdx.x;
  const int b = blockIdx.y;
  const int64_t rid = (int64_t)b * n_rows + i;
  const int64_t pos = (q_pos ? (int64_t)q_pos[b] : 0) + pos_offset + i;
  int64_t n = pos + 1 < n_k ? pos + 1 : n_k;
  n = n > 0 ? n : 0;
  int32_t* out = idx + rid * k;
  const int tid = threadIdx.x;
  if (n <= k) {  // every visible key is kept
    for (int j = tid; j < k; j += DC_THREADS) out[j] = j < n ? j : -1;
    if (tid == 0) redo[rid] = 0;
    return;
  }
  // segment offsets (one thread per segment), an overflowed segment or too many candidates
  // leave the row undecided
  if (tid == 0) s_bad = 0;
  __syncthreads();
  const uint32_t c_own = tid < n_segs ? cnt[rid * n_segs + tid] : 0u;
  if (c_own > (uint32_t)DEC_SEG) s_bad = 1;
  uint32_t total;
  const uint32_t off = block_excl_scan<DC_THREADS>(c_own, wtot, total);
  if (tid < n_segs) soff[tid] = off;
  if (tid == 0) soff[n_segs] = total;
  __syncthreads();
  if (s_bad || total < (uint32_t)k || total > (uint32_t)SEL_CAND_CAP) {
    if (tid == 0) redo[rid] = 1;
    return;
  }
  // the segments -> LDS, packed; LOAD_BATCH loads per thread in flight before any is stored
  const uint2* cr = cand + rid * n_segs * DEC_SEG;
  constexpr int SEG_STEP = DC_THREADS / DEC_SEG;
  const uint32_t j = (uint32_t)(tid % DEC_SEG);
  for (int64_t sg0 = tid / DEC_SEG; sg0 < n_segs; sg0 += (int64_t)LOAD_BATCH * SEG_STEP) {
    uint2 e[LOAD_BATCH];
    uint32_t o[LOAD_BATCH];
    bool have[LOAD_BATCH];
#pragma unroll
    for (int q = 0; q < LOAD_BATCH; ++q) {
      const int64_t sgi = sg0 + (int64_t)q * SEG_STEP;
      o[q] = sgi < n_segs ? soff[sgi] : 0u;
      have[q] = sgi < n_segs && j < soff[sgi + 1] - o[q];
      e[q] = have[q] ? cr[sgi * DEC_SEG + j] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int q = 0; q < LOAD_BATCH; ++q)
      if (have[q]) {
        ckey[o[q] + j] = score_key(__uint_as_float(e[q].x));
        cpos[o[q] + j] = (int32_t)e[q].y;
      }
  }
  const int64_t nw = (n + 31) / 32;
  for (int64_t j = tid; j < nw; j += DC_THREADS) {
    sel[j] = 0;
    tie[j] = 0;
  }
  __syncthreads();
  uint32_t rem;
  const uint32_t vstar = select_lds<DC_THREADS>(ckey, (int)total, (uint32_t)k, hist, wtot, &s_digit, &s_above, rem);
  for (uint32_t j = tid; j < total; j += DC_THREADS) {
    const uint32_t u = ckey[j];
    const int32_t sp = cpos[j];
    if (u > vstar) atomicOr(&sel[sp >> 5], 1u << (sp & 31));
    else if (u == vstar) atomicOr(&tie[sp >> 5], 1u << (sp & 31));
  }
  __syncthreads();
  write_kept<DC_THREADS>(sel, tie, n, rem, k, out, wtot);
  if (tid == 0) redo[rid] = 0;
}

hipError_t launch_dec_cand_topk(const DecCandArgs& a, hipStream_t st) {
  if (a.n_rows <= 0 || a.B <= 0) return hipSuccess;
  if (a.n_k > TOPK_MAX_N || a.n_segs > DC_MAX_SEGS || a.n_segs > DC_THREADS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dec_cand_topk_kernel, dim3((unsigned)a.n_rows, (unsigned)a.B), dim3(DC_THREADS), 0, st, a.cand,
                     a.cnt, a.n_segs, a.n_rows, a.n_k, a.q_pos, a.pos_offset, a.k, a.idx, a.redo);
  return hipGetLastError();
}

hipError_t launch_sel_threshold(const SelThresholdArgs& a, hipStream_t st) {
  if (a.n_rows <= 0 || a.B <= 0) return hipSuccess;
  if ((a.n_k + SEL_SAMPLE_STRIDE - 1) / SEL_SAMPLE_STRIDE > TH_MAX || a.ld_s < sel_sample_ld(a.n_k))
    return hipErrorInvalidValue;
  const size_t lds = (size_t)((a.n_k + SEL_SAMPLE_STRIDE - 1) / SEL_SAMPLE_STRIDE) * sizeof(uint32_t);
  // few rows (decode): one 1024-thread block per row, so the select's passes run 4x wider
  if (a.n_rows * a.B < 512)
    hipLaunchKernelGGL(sel_threshold_kernel<1024>, dim3((unsigned)a.n_rows, (unsigned)a.B), dim3(1024), lds, st,
                       a.samp, a.ld_s, a.rows_pad, a.n_rows, a.n_k, a.q_pos, a.row_begin, a.k, a.thr);
  else
    hipLaunchKernelGGL(sel_threshold_kernel<TH_THREADS>, dim3((unsigned)a.n_rows, (unsigned)a.B), dim3(TH_THREADS), lds,
                       st, a.samp, a.ld_s, a.rows_pad, a.n_rows, a.n_k, a.q_pos, a.row_begin, a.k, a.thr);
  return hipGetLastError();
}

hipError_t launch_sel_candidates(const SelCandArgs& a, hipStream_t st) {
  if (a.n_rows <= 0 || a.B <= 0) return hipSuccess;
  if (a.k > SEL_CAND_CAP) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sel_candidates_kernel, dim3((unsigned)a.n_rows, (unsigned)a.B), dim3(TO_THREADS), 0, st, a.cand,
                     a.cnt, a.rows_pad, a.n_rows, a.n_k, a.q_pos, a.row_begin, a.k, a.idx, a.out_rows, a.out_row0,
                     a.redo);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  dim3 grid((unsigned)a.n_rows, (unsigned)a.B);
  if (a.n_k >= TL_MIN_N && a.k <= TL_CAP / 4)
    hipLaunchKernelGGL(topk_long_kernel, grid, dim3(TL_THREADS), 0, st, a.scores, a.ld_scores, a.n_rows, a.n_k,
                       a.q_pos, a.pos_offset, a.row_begin, a.k, a.idx, a.redo);
  else if (a.redo)
    return hipErrorInvalidValue;  // the row-skipping variant exists for long rows only
  else
    hipLaunchKernelGGL(topk_rows_kernel, grid, dim3(TK_THREADS), 0, st, a.scores, a.ld_scores, a.n_rows, a.n_k,
                       a.q_pos, a.pos_offset, a.row_begin, a.k, a.idx);
  return hipGetLastError();
}

}  // namespace dsa
