// Fused lightning indexer + streaming top-k for prefill (query t at position t).
//
// The indexer's L x L score matrix is never stored.  Rows are scored 64 keys at a time
// (indexer_tile.h); every score immediately meets the row's streaming selection state in
// LDS:
//   * a candidate buffer (order-preserving key + index) that stays sorted by key index,
//     because keys arrive in ascending order and appends keep lane order;
//   * a threshold thr: a later key enters only if its key is > thr;
//   * when the buffer is nearly full it is cut: a wave-local radix descent (8-bit digits
//     over an LDS histogram, starting at the highest bit where the candidates can differ)
//     finds the bin holding the k-th largest key, and an in-place stable compaction keeps
//     the keys >= that bin's lower edge, which becomes the new bound (thr = edge - 1).  If
//     that would free too little room (many equal keys), the exact selection runs instead:
//     v* = the k-th largest key exactly, keep exactly the top k so far, thr = v* (a later
//     key equal to v* has a larger index, and on a tie the lower index wins).
// At the end an exact selection leaves the row's top k, in ascending key order.
// Rows whose position is below k keep every key and are written by a separate fill kernel.
//
// Selection rule: top-k by index score with ties to the lower key index (juhe.plus
// explainer, section 第二步：Fine-grained Token Selection; 53ai.com V3.2-Exp summary,
// section 创新架构).
#include "dsa_kernels.h"
#include "indexer_tile.h"

namespace dsa {

constexpr int CAND = 3072;  // candidate slots per row

// Per-row selection state of the fused kernel, at file scope so the compiler can tell it
// apart from the key tiles that direct loads are still writing (accesses to these arrays
// then never wait for the tile loads).
__shared__ uint32_t s_ckey[4][CAND];
__shared__ int32_t s_cidx[4][CAND];
__shared__ uint32_t s_hist[4][256];

// LDS increment without a return value, written as the instruction itself: the compiler
// would otherwise drain every in-flight direct load before each atomic (it cannot tell that
// the histogram and the tile buffers do not overlap).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const uint8_t*)p);
}
__device__ __forceinline__ void lds_inc(uint32_t* p) {
  asm volatile("ds_add_u32 %0, %1" ::"v"(lds_addr(p)), "v"(1u) : "memory");
}
// 4-byte LDS store written as the instruction itself (same reason as lds_inc).  Completion
// is left to the s_waitcnt lgkmcnt(0) that precedes every block barrier; a later LDS read
// by the same wave is ordered after it by the LDS queue.
__device__ __forceinline__ void lds_store(void* p, float v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
// LDS reads that complete inside the same asm block (same reason as lds_inc: a plain read
// of the tile ring or of the exchange buffers would first wait for every tile load in flight).
__device__ __forceinline__ v4i lds_read16_sync(const void* p) {
  v4i r;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(lds_addr(p)) : "memory");
  return r;
}
__device__ __forceinline__ float lds_read4_sync(const void* p) {
  float r;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(lds_addr(p)) : "memory");
  return r;
}
__device__ __forceinline__ void lds_read4x2_sync(const void* p0, const void* p1, float& a, float& b) {
  asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(a), "=&v"(b)
               : "v"(lds_addr(p0)), "v"(lds_addr(p1))
               : "memory");
}

constexpr int SEL_BATCH = 8;   // entries per lane in flight per pass step
constexpr int CUT_SLACK = 256; // a cut may keep at most this many keys below the k-th largest

// One radix digit of the k-th largest key among s_ckey[r][0..n): histogram (8-bit digits
// at `shift`) of the keys whose bits under `pmask` equal `prefix`, then the digit d where
// the count from the top reaches `rem`.  Returns d; `above` = keys in higher bins, `binc` =
// keys in bin d.
__device__ __forceinline__ uint32_t digit_step(int r, int n, int shift, uint32_t dmask, uint32_t pmask,
                                               uint32_t prefix, uint32_t rem, uint32_t& above, uint32_t& binc) {
  const int lane = lane_id();
  const uint32_t* key = s_ckey[r];
  uint32_t* hist = s_hist[r];
  *reinterpret_cast<v4i*>(hist + 4 * lane) = v4i{0, 0, 0, 0};
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  for (int base = 0; base < n; base += WAVE * SEL_BATCH) {
    uint32_t u[SEL_BATCH];
#pragma unroll
    for (int m = 0; m < SEL_BATCH; ++m) {
      const int i = base + WAVE * m + lane;
      u[m] = key[i < n ? i : 0];
    }
#pragma unroll
    for (int m = 0; m < SEL_BATCH; ++m)
      if ((base + WAVE * m + lane < n) & ((u[m] & pmask) == prefix)) lds_inc(&hist[(u[m] >> shift) & dmask]);
  }
  __builtin_amdgcn_wave_barrier();
  // lane owns bins 255-4*lane .. 252-4*lane (descending)
  const v4i hv = lds_read16_sync(hist + 252 - 4 * lane);
  const uint32_t h[4] = {(uint32_t)hv[3], (uint32_t)hv[2], (uint32_t)hv[1], (uint32_t)hv[0]};
  const uint32_t local = h[0] + h[1] + h[2] + h[3];
  uint32_t c = wave_incl_scan(local) - local;
  uint32_t digit = 0, ab = 0, bc = 0;
  bool found = false;
  if (c < rem && c + local >= rem) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!found && c + h[j] >= rem) {
        found = true;
        digit = 255u - 4u * lane - j;
        ab = c;
        bc = h[j];
      }
      c += h[j];
    }
  }
  const uint64_t fm = ballot(found);
  const int src = fm ? __ffsll((unsigned long long)fm) - 1 : 0;
  above = __shfl(ab, src, WAVE);
  binc = __shfl(bc, src, WAVE);
  return __shfl(digit, src, WAVE);
}

// Stable in-place compaction of s_ckey/s_cidx[r][0..n): keeps the keys > gt and the first
// `rem_eq` keys equal to `eq` (in buffer order, i.e. lowest key index first).  All entries
// of a batch are read before any is written, and an entry only moves down, so no unread
// entry is overwritten.  Returns the number kept.
__device__ __forceinline__ int compact_keep(int r, int n, uint32_t gt, uint32_t eq, uint32_t rem_eq) {
  const int lane = lane_id();
  uint32_t* key = s_ckey[r];
  int32_t* id = s_cidx[r];
  uint32_t kept = 0, eq_seen = 0;
  for (int base = 0; base < n; base += WAVE * SEL_BATCH) {
    uint32_t u[SEL_BATCH];
    int32_t ix[SEL_BATCH];
#pragma unroll
    for (int m = 0; m < SEL_BATCH; ++m) {
      const int i = base + WAVE * m + lane;
      u[m] = key[i < n ? i : 0];
      ix[m] = id[i < n ? i : 0];
    }
#pragma unroll
    for (int m = 0; m < SEL_BATCH; ++m) {
      const bool in = base + WAVE * m + lane < n;
      const bool is_eq = in & (u[m] == eq);
      const uint64_t me = ballot(is_eq);
      const bool keep = (in & (u[m] > gt)) | (is_eq & (eq_seen + lanes_below(me) < rem_eq));
      const uint64_t mk = ballot(keep);
      if (keep) {
        const uint32_t dst = kept + lanes_below(mk);
        key[dst] = u[m];
        id[dst] = ix[m];
      }
      kept += (uint32_t)__popcll((unsigned long long)mk);
      eq_seen += (uint32_t)__popcll((unsigned long long)me);
    }
  }
  __builtin_amdgcn_wave_barrier();
  return (int)kept;
}

// Exact selection: radix select of v* = the k-th largest key among s_ckey[r][0..n) (n > k),
// then stable compaction to exactly k entries (keys > v*, then the lowest-index keys equal
// to v*).  Wave-local.  The digits start at the highest bit where the keys differ (they
// share their top bits, which would pile every key into one histogram bin).  Returns v*.
__device__ uint32_t select_compact(int r, int n, int k) {
  const int lane = lane_id();
  const uint32_t* key = s_ckey[r];
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int base = 0; base < n; base += WAVE * SEL_BATCH) {
    uint32_t u[SEL_BATCH];
#pragma unroll
    for (int m = 0; m < SEL_BATCH; ++m) {
      const int i = base + WAVE * m + lane;
      u[m] = key[i < n ? i : 0];
    }
#pragma unroll
    for (int m = 0; m < SEL_BATCH; ++m) {
      const bool in = base + WAVE * m + lane < n;
      mn = in ? min(mn, u[m]) : mn;
      mx = in ? max(mx, u[m]) : mx;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, WAVE));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, WAVE));
  }
  uint32_t rem = (uint32_t)k;
  uint32_t prefix = mx;
  if (mn != mx) {
    int hi = 31 - __clz((int)(mn ^ mx));  // highest differing bit
    uint32_t pmask = hi == 31 ? 0u : ~((2u << hi) - 1u);
    prefix = mx & pmask;
    while (true) {
      const int shift = hi >= 7 ? hi - 7 : 0;
      const uint32_t dmask = (2u << (hi - shift)) - 1u;
      uint32_t above, binc;
      const uint32_t digit = digit_step(r, n, shift, dmask, pmask, prefix, rem, above, binc);
      rem -= above;
      prefix |= digit << shift;
      pmask |= dmask << shift;
      if (shift == 0) break;
      hi = shift - 1;
    }
  }
  compact_keep(r, n, prefix, prefix, rem);
  return prefix;
}

// Cut: keeps every key that can still be among the row's k best, without finding v*
// exactly.  Descends the radix digits of the k-th largest key only until its bin holds at
// most CUT_SLACK keys below it; the keys >= that bin's lower edge e are then kept (at least
// k keys are >= e, so no key below e can reach the top k).  `lo` <= every key <= `mx`.
// The buffer is compacted only if at most `max_keep` keys would remain.  Returns e, or 0
// (buffer untouched) if no such cut exists; `kept` = entries left.
__device__ uint32_t cut_candidates(int r, int n, int k, uint32_t lo, uint32_t mx, int max_keep, int& kept) {
  kept = n;
  if (lo >= mx) return 0u;
  int hi = 31 - __clz((int)(lo ^ mx));
  uint32_t pmask = hi == 31 ? 0u : ~((2u << hi) - 1u);
  uint32_t prefix = mx & pmask;
  uint32_t rem = (uint32_t)k;
  while (true) {
    const int shift = hi >= 7 ? hi - 7 : 0;
    const uint32_t dmask = (2u << (hi - shift)) - 1u;
    uint32_t above, binc;
    const uint32_t digit = digit_step(r, n, shift, dmask, pmask, prefix, rem, above, binc);
    rem -= above;
    prefix |= digit << shift;
    pmask |= dmask << shift;
    if (binc - rem <= (uint32_t)CUT_SLACK || shift == 0) {
      // keys >= the bin's lower edge: those in higher bins at every level, plus the bin
      if (prefix == 0u || (int)((uint32_t)k - rem + binc) > max_keep) return 0u;
      break;
    }
    hi = shift - 1;
  }
  kept = compact_keep(r, n, prefix - 1u, 0u, 0u);
  return prefix;
}

// ---------------------------------------------------------------------------------------
// Persistent fused kernel.  A block owns groups of 4 consecutive rows; blocks take groups
// longest-first in lockstep (group G = block + round * blocks), so the blocks on one XCD
// sweep the same key tiles at about the same time and the tiles stay in L2.  Keys are
// processed in steps of two 64-key tiles (one barrier per step):
//   * scoring waves 0-7: wave w scores key fragment f = w/2 (16 keys of each tile) for
//     head half hh = w%2 of all 4 rows: per tile 8 FP8 MFMAs and 4 head-sum MFMAs; the
//     half-totals go to LDS;
//   * owner waves 8-11: wave 8+j owns row j's selection.  At step s it takes step s-1's
//     128 scores (completed before the step's barrier), in the VALU and LDS issue slots
//     the scoring waves leave free.
// Key tiles arrive by direct global->LDS loads in a ring of three tile pairs (two steps in
// flight).  When any owner's buffer nears full, all four owners cut at the same step (one
// stall of the block instead of four).
// ---------------------------------------------------------------------------------------
constexpr int PF_SCORE_WAVES = 8;
constexpr int PF_WAVES = PF_SCORE_WAVES + 4;
constexpr int TILE_BYTES = KEY_TILE * IDX_DIM;
constexpr int STEP_KEYS = 2 * KEY_TILE;
constexpr int COMPACT_AT = CAND - 3 * STEP_KEYS;  // collective compaction trigger

#define WAIT_VM_LGKM0(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0x0 << 8))

// wave w copies LDS units 64w .. 64w+63 of a tile (key 8w + lane/8 of the tile, 16-byte
// unit lane%8 XOR-swizzled by the key's row); wave 0 also copies the tile's 64 key scales.
struct TileDma {
  int krow;          // key row within the tile
  uint32_t koff;     // byte offset of this lane's unit within a key row
};
__device__ __forceinline__ TileDma tile_dma_lane(int wv, int lane) {
  const int U = 64 * wv + lane;
  const int row = U >> 3, cp = U & 7;
  return TileDma{row, (uint32_t)(16 * (cp ^ (row & 7)))};
}
template <bool PAGED>
__device__ __forceinline__ void dma_key_tile(uint8_t* tk, float* ts, const uint8_t* __restrict__ k8,
                                             const float* __restrict__ ks, int key0, int L, const TileDma& d,
                                             int wv, int lane, const PageTable& pt, int b) {
  if constexpr (!PAGED) {
    // 32-bit offsets from the uniform bases (L * 128 < 2^32 for every supported L)
    const uint32_t key = (uint32_t)min(key0 + d.krow, L - 1);
    __builtin_amdgcn_global_load_lds(k8 + (key * IDX_DIM + d.koff), tk + 1024 * wv, 16, 0, 0);
    if (wv == 0) __builtin_amdgcn_global_load_lds(ks + (uint32_t)min(key0 + lane, L - 1), ts, 4, 0, 0);
  } else {  // k8 / ks are the page pools; the tile's keys lie on one page (one lookup)
    int64_t first = 0;
    const int64_t base = paged_tile_base(pt, b, key0, L - 1, first);
    const int64_t row = base + (min(key0 + d.krow, L - 1) - first);
    __builtin_amdgcn_global_load_lds(k8 + row * IDX_DIM + d.koff, tk + 1024 * wv, 16, 0, 0);
    if (wv == 0) __builtin_amdgcn_global_load_lds(ks + base + (min(key0 + lane, L - 1) - first), ts, 4, 0, 0);
  }
}

// wait until step s's two tiles have landed (step s+1's may still be in flight); wave 0
// issues four loads per step, the other scoring waves two.  Also drains this wave's LDS ops.
__device__ __forceinline__ void wait_step(int st, int nsteps, int wv) {
  const bool more = st + 1 < nsteps;
  if (wv == 0) {
    if (more) WAIT_VM_LGKM0(4);
    else WAIT_VM_LGKM0(0);
  } else {
    if (more) WAIT_VM_LGKM0(2);
    else WAIT_VM_LGKM0(0);
  }
}

// B operand of fragment f of a tile in the ring (the layout lds_key_fragment reads),
// fetched with both reads completing inside one asm block.
__device__ __forceinline__ v8i ring_key_fragment(const uint8_t* tile, int f, int lane) {
  const int row = 16 * f + (lane & 15);
  const int c0 = (2 * (lane >> 4)) ^ (row & 7);
  const int c1 = (2 * (lane >> 4) + 1) ^ (row & 7);
  v4i lo, hi;
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(lo), "=&v"(hi)
               : "v"(lds_addr(tile + row * IDX_DIM + 16 * c0)), "v"(lds_addr(tile + row * IDX_DIM + 16 * c1))
               : "memory");
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

struct OwnerState {
  int cnt;
  uint32_t thr;  // a key enters only if it is > thr
  uint32_t lo;   // every buffered key is >= lo
  uint32_t mx;   // this lane's largest key appended so far
  float cmax;
};

__shared__ __align__(16) int s_cnt[4];  // owners' published candidate counts
// Half-totals of a step's scores exchanged between the scoring waves and the owners
// ([step % 2][head half][row][key of the step]).
__shared__ float xbuf[2][2][4][STEP_KEYS];

// An owner's reads for one step, completing together: the half-totals of its row's scores
// of the previous step (keys lane and 64 + lane, both head halves), this step's two key
// scales, and the published counts.
__device__ __forceinline__ void owner_reads(int slot, int r, const float* ks0, const float* ks1, float x[4],
                                            float ksn[2], v4i& cnts) {
  const int l = lane_id();
  asm volatile(
      "ds_read_b32 %0, %7\n\tds_read_b32 %1, %8\n\tds_read_b32 %2, %9\n\tds_read_b32 %3, %10\n\t"
      "ds_read_b32 %4, %11\n\tds_read_b32 %5, %12\n\tds_read_b128 %6, %13\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(ksn[0]), "=&v"(ksn[1]), "=&v"(cnts)
      : "v"(lds_addr(&xbuf[slot][0][r][l])), "v"(lds_addr(&xbuf[slot][1][r][l])),
        "v"(lds_addr(&xbuf[slot][0][r][64 + l])), "v"(lds_addr(&xbuf[slot][1][r][64 + l])),
        "v"(lds_addr(ks0 + l)), "v"(lds_addr(ks1 + l)), "v"(lds_addr(s_cnt))
      : "memory");
}

// Append the owner's 64 new scores (keys key0 + lane) to its candidate buffer; keys past
// `lim` (the last key the row sees) are not taken.
__device__ __forceinline__ void owner_append(OwnerState& S, int r, float s, int key0, int lim) {
  const int lane = lane_id();
  const int key = key0 + lane;
  const uint32_t u = score_key(s);
  const bool pass = key <= lim && u > S.thr;
  const uint64_t m = ballot(pass);
  if (m) {
    if (pass) {
      const int off = S.cnt + (int)lanes_below(m);
      s_ckey[r][off] = u;
      s_cidx[r][off] = key;
      S.mx = max(S.mx, u);
    }
    S.cnt += __popcll((unsigned long long)m);
  }
}

// Cut when the buffer has no room for another step or when any owner's buffer nears full
// (all cut together).
__device__ __forceinline__ void owner_maybe_cut(OwnerState& S, int r, int k, int most) {
  if (S.cnt > CAND - STEP_KEYS || (most > COMPACT_AT && S.cnt > k + 2 * STEP_KEYS)) {
    __builtin_amdgcn_wave_barrier();
    uint32_t mx = S.mx;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, WAVE));
    int kept;
    const uint32_t e = cut_candidates(r, S.cnt, k, S.lo, mx, CAND - 2 * STEP_KEYS, kept);
    if (e != 0u) {
      S.thr = e - 1u;
      S.lo = e;
      S.cnt = kept;
    } else {  // the cut freed too little (many equal keys): select exactly
      S.thr = select_compact(r, S.cnt, k);
      S.lo = S.thr;
      S.cnt = k;
    }
  }
}

// Group G of the persistent loop: sequence b = G % B (consecutive blocks, hence each XCD's
// blocks, stay on few sequences), rows row_hi - 4 .. row_hi - 1 of it, longest first.
// Row r sits at position pos0 + r and sees keys 0 .. min(pos0 + r, n_k - 1); n_keys is what
// the group's last row sees (0 if its position is negative).
struct GroupGeom {
  int b, row_hi, pos0, n_keys;
};
__device__ __forceinline__ GroupGeom group_geom(int G, int B, int n_q, int n_k, const int32_t* __restrict__ q_pos) {
  GroupGeom g;
  g.b = G % B;
  g.row_hi = n_q - 4 * (G / B);
  g.pos0 = q_pos ? q_pos[g.b] : 0;
  const int64_t last = (int64_t)g.pos0 + g.row_hi;  // last row's position + 1
  g.n_keys = (int)(last < 0 ? 0 : last > n_k ? n_k : last);
  return g;
}

// With a redo list, a group runs only if one of its rows in [row_lo, row_end) is marked.
__device__ __forceinline__ bool group_skipped(const uint8_t* __restrict__ redo, const GroupGeom& g, int n_q,
                                              int row_lo, int row_end) {
  if (!redo) return false;
  const uint8_t* r = redo + (size_t)g.b * n_q;
  bool any = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = g.row_hi - 4 + j;
    if (row >= row_lo && row < row_end && row >= 0) any |= r[row] != 0;
  }
  return !any;
}

template <bool PAGED>
__global__ __launch_bounds__(PF_WAVES * 64, 1) void prefill_idx_topk_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, const float* __restrict__ w, const int32_t* __restrict__ q_pos, int B,
    int n_q, int n_k, int64_t kbs, int row_lo, int row_end, int k, int g_begin, int g_end,
    int32_t* __restrict__ idx, const uint8_t* __restrict__ redo, PageTable pt) {
  // ring of three tile pairs (pair p = tiles 2p, 2p+1) and their key scales
  __shared__ __align__(16) uint8_t tk0[TILE_BYTES];
  __shared__ __align__(16) uint8_t tk1[TILE_BYTES];
  __shared__ __align__(16) uint8_t tk2[TILE_BYTES];
  __shared__ __align__(16) uint8_t tk3[TILE_BYTES];
  __shared__ __align__(16) uint8_t tk4[TILE_BYTES];
  __shared__ __align__(16) uint8_t tk5[TILE_BYTES];
  __shared__ __align__(16) float ts0[KEY_TILE];
  __shared__ __align__(16) float ts1[KEY_TILE];
  __shared__ __align__(16) float ts2[KEY_TILE];
  __shared__ __align__(16) float ts3[KEY_TILE];
  __shared__ __align__(16) float ts4[KEY_TILE];
  __shared__ __align__(16) float ts5[KEY_TILE];

  uint8_t* const tks[6] = {tk0, tk1, tk2, tk3, tk4, tk5};
  float* const tss[6] = {ts0, ts1, ts2, ts3, ts4, ts5};
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;

  if (wv < PF_SCORE_WAVES) {
    // ---------------- scoring waves ----------------
    const int f = wv >> 1, hh = wv & 1;
    const TileDma dl = tile_dma_lane(wv, lane);
    for (int G = g_begin + blockIdx.x; G < g_end; G += gridDim.x) {
      const GroupGeom g = group_geom(G, B, n_q, n_k, q_pos);
      if (group_skipped(redo, g, n_q, row_lo, row_end)) continue;
      if (g.n_keys <= k) continue;  // every row keeps all it sees: the owners write it
      const int row0 = g.row_hi - 4;
      const size_t rbase = (size_t)g.b * n_q;
      const uint8_t* kb = PAGED ? k8 : k8 + (size_t)g.b * kbs * IDX_DIM;
      const float* ksb = PAGED ? ks : ks + (size_t)g.b * kbs;
      IdxHalf Qh[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // rows outside [row_lo, row_end) are not this launch's: score a valid row
        const size_t r = rbase + min(max(row0 + j, row_lo), row_end - 1);
        const float cmax = row_cmax(qs + r * IDX_HEADS, w + r * IDX_HEADS);
        load_idx_half(Qh[j], q8 + r * IDX_HEADS * IDX_DIM, qs + r * IDX_HEADS, w + r * IDX_HEADS, hh, cmax);
      }
      const int L = g.n_keys;
      const int nsteps = (L + STEP_KEYS - 1) / STEP_KEYS;
      // (a step's second tile may lie past key L-1: its loads clamp to key L-1, and the
      // owners never take a key past their row's position)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < 2 * nsteps) dma_key_tile<PAGED>(tks[j], tss[j], kb, ksb, j * KEY_TILE, L, dl, wv, lane, pt, g.b);

      for (int base = 0; base <= nsteps; base += 3) {
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) {
          const int st = base + pp;
          if (st <= nsteps) {
            if (st < nsteps) wait_step(st, nsteps, wv);
            else WAIT_VM_LGKM0(0);
            __builtin_amdgcn_s_barrier();
            if (st < nsteps) {
              if (st + 2 < nsteps) {  // into the pair of step st-1, which every wave is done with
                const int q = (pp + 2) % 3;
                dma_key_tile<PAGED>(tks[2 * q], tss[2 * q], kb, ksb, (2 * st + 4) * KEY_TILE, L, dl, wv, lane, pt,
                                    g.b);
                dma_key_tile<PAGED>(tks[2 * q + 1], tss[2 * q + 1], kb, ksb, (2 * st + 5) * KEY_TILE, L, dl, wv,
                                    lane, pt, g.b);
              }
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const v8i b = ring_key_fragment(tks[2 * pp + h], f, lane);
                v4f x[4][2];
                float t[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  x[j][0] = mfma_fp8_scaled(Qh[j].a[0], b);
                  x[j][1] = mfma_fp8_scaled(Qh[j].a[1], b);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) t[j] = head_half_sum(Qh[j], x[j][0], x[j][1]);
                // lane l holds every row's sum for key 16f + l%16; it stores row l/16's
                const int jr = lane >> 4;
                const float v = jr == 0 ? t[0] : jr == 1 ? t[1] : jr == 2 ? t[2] : t[3];
                lds_store(&xbuf[st & 1][hh][jr][64 * h + 16 * f + (lane & 15)], v);
              }
            }
          }
        }
      }
      WAIT_VM_LGKM0(0);
      __builtin_amdgcn_s_barrier();  // end of group: ring and exchange buffers free
    }
  } else {
    // ---------------- owner waves ----------------
    const int r = wv - PF_SCORE_WAVES;
    for (int G = g_begin + blockIdx.x; G < g_end; G += gridDim.x) {
      const GroupGeom g = group_geom(G, B, n_q, n_k, q_pos);
      if (group_skipped(redo, g, n_q, row_lo, row_end)) continue;
      const int my_row = g.row_hi - 4 + r;
      const bool valid = my_row >= row_lo && my_row < row_end;
      // last key this row sees (-1: none)
      const int64_t lim64 = min((int64_t)g.pos0 + my_row, (int64_t)n_k - 1);
      const int lim = (int)(lim64 < -1 ? -1 : lim64);
      int32_t* out = idx + ((size_t)g.b * n_q + max(my_row, 0)) * k;
      if (g.n_keys <= k) {  // no row sees more than k keys: keep them all
        if (valid)
          for (int j = lane; j < k; j += WAVE) out[j] = j <= lim ? j : -1;
        continue;
      }
      const size_t rq = (size_t)g.b * n_q + min(max(my_row, row_lo), row_end - 1);
      OwnerState S{0, 0u, 0u, 0u, row_cmax(qs + rq * IDX_HEADS, w + rq * IDX_HEADS)};
      if (lane == 0) lds_store(&s_cnt[r], __int_as_float(0));
      const int nsteps = (g.n_keys + STEP_KEYS - 1) / STEP_KEYS;
      float ksc[2] = {0.f, 0.f};  // key scales of the step not yet taken
      for (int base = 0; base <= nsteps; base += 3) {
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) {
          const int st = base + pp;
          if (st <= nsteps) {
            WAIT_VM_LGKM0(0);
            __builtin_amdgcn_s_barrier();
            // take step st-1; read step st's key scales (their pair is reloaded at step st+1)
            float x[4], ksn[2];
            v4i c;
            owner_reads((st - 1) & 1, r, tss[2 * pp], tss[2 * pp + 1], x, ksn, c);
            if (st >= 1 && valid) {
              const int key0 = (st - 1) * STEP_KEYS;
              owner_append(S, r, finish_score(x[0], x[1], S.cmax, ksc[0]), key0, lim);
              owner_append(S, r, finish_score(x[2], x[3], S.cmax, ksc[1]), key0 + KEY_TILE, lim);
              owner_maybe_cut(S, r, k, max(max(c[0], c[1]), max(c[2], c[3])));
              if (lane == 0) lds_store(&s_cnt[r], __int_as_float(S.cnt));
            }
            ksc[0] = ksn[0];
            ksc[1] = ksn[1];
          }
        }
      }
      WAIT_VM_LGKM0(0);
      __builtin_amdgcn_s_barrier();  // end of group
      // the final selection overlaps the scoring waves' start of the next group
      if (valid) {
        __builtin_amdgcn_wave_barrier();
        if (S.cnt > k) {
          select_compact(r, S.cnt, k);
          S.cnt = k;
        }
        for (int j = lane; j < k; j += WAVE) out[j] = j < S.cnt ? s_cidx[r][j] : -1;
      }
    }
  }
}

// rows [t0, n) of each sequence (row t at position t) keep every key they see:
// idx[b][t] = 0 .. min(t, n_k - 1), -1 padded
__global__ __launch_bounds__(256) void prefill_fill_kernel(int64_t t0, int64_t n, int64_t n_q, int64_t n_k, int k,
                                                           int32_t* __restrict__ idx) {
  const int64_t t = t0 + blockIdx.x;
  if (t >= n) return;
  const int64_t lim = t < n_k - 1 ? t : n_k - 1;
  int32_t* out = idx + ((int64_t)blockIdx.y * n_q + t) * k;
  for (int j = threadIdx.x; j < k; j += 256) out[j] = j <= lim ? j : -1;
}

hipError_t launch_prefill_topk(const PrefillTopkArgs& a, hipStream_t st) {
  // Rows [row_begin, row_end) of every sequence (row_end < 0: to n_q).  Without q_pos, row t
  // sits at position t: rows below k keep every key they see and are written by the fill
  // kernel.  With q_pos the positions live on the device, and groups whose rows see at most
  // k keys are written by the fused kernel's owners.
  const int64_t row_end = a.row_end < 0 || a.row_end > a.n_q ? a.n_q : a.row_end;
  int64_t row_lo = a.row_begin > 0 ? a.row_begin : 0;
  if (!a.q_pos) {
    const int64_t below = a.k < row_end ? a.k : row_end;  // rows [row_lo, below) keep all keys
    if (below > row_lo && !a.redo)
      hipLaunchKernelGGL(prefill_fill_kernel, dim3((unsigned)(below - row_lo), (unsigned)a.B), dim3(256), 0, st,
                         row_lo, below, a.n_q, a.n_k, a.k, a.idx);
    row_lo = below > row_lo ? below : row_lo;
  }
  if (row_end > row_lo) {
    static int n_cu = 0;
    if (n_cu == 0) {
      int dev = 0;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
        n_cu = 256;
    }
    // group G holds rows n_q - 4 (G / B) - 4 .. n_q - 4 (G / B) - 1 of sequence G % B: the
    // groups that meet rows [row_lo, row_end)
    const int64_t g_begin = a.B * ((a.n_q - row_end) / 4);
    const int64_t g_end = a.B * ((a.n_q - 1 - row_lo) / 4 + 1);
    const int64_t n_groups = g_end - g_begin;
    const int64_t blocks = n_groups < n_cu ? n_groups : n_cu;
    hipLaunchKernelGGL(a.pages.table ? prefill_idx_topk_kernel<true> : prefill_idx_topk_kernel<false>,
                       dim3((unsigned)blocks), dim3(PF_WAVES * 64), 0, st, a.q8, a.qs, a.k8, a.ks, a.w, a.q_pos,
                       (int)a.B, (int)a.n_q, (int)a.n_k, a.k_bstride ? a.k_bstride : a.n_k, (int)row_lo,
                       (int)row_end, a.k, (int)g_begin, (int)g_end, a.idx, a.redo, a.pages);
  }
  return hipGetLastError();
}

}  // namespace dsa
