// Host-side launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

// Sets the calling thread's last-error message (dsa_last_error) and returns status.
int set_error(int status, const char* fmt, ...);

struct IndexerArgs {
  const void* q_idx;
  const float* q_scale;
  const void* k_idx;
  const float* k_scale;
  const float* w;
  int64_t B, n_q, n_k;
  const int32_t* q_pos;     // [B] or null; position of row r = q_pos[b] + pos_offset + r
  int64_t pos_offset;
  int32_t H_I, d_I, dtype;
  int64_t row_begin, n_rows;
  float* scores;
  int64_t ld_scores;
  int64_t k_bstride = 0;    // key rows between sequences of k_idx / k_scale (0: n_k)
};
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t st);

// FP8 index scores of a few rows with their keys split over blocks (decode), SPLIT_TILES
// 64-key tiles per block of 4 waves.  Row i of sequence b sits at position q_pos[b] +
// pos_offset + row_begin + i.  Store mode (cand null): the scores of keys 0, S, 2S, ..
// (S = key_stride) to columns 0, 1, 2, .. of row b * n_rows + i of `scores` (ld floats
// apart), -inf past the row's position.  Filter mode: no store; each wave of each block
// writes the keys it scores above thr[b * n_rows + i] to its own segment of DEC_SEG slots
// (see dec_split_segments), as (fp32 score bits, key) pairs in ascending key order, and
// their number (which may exceed DEC_SEG) to the segment's count.  redo non-null: only rows
// whose redo byte is set run.
constexpr int SPLIT_TILES = 32;  // 2048 keys per block, 8 tiles per wave
constexpr int DEC_SEG = 64;      // candidate slots per wave segment
// candidate segments of a row in filter mode (4 per block): row r's list is at
// cand + r * segs * DEC_SEG, its counts at cnt + r * segs
inline int64_t dec_split_segments(int64_t n_k) {
  return 4 * ((n_k + SPLIT_TILES * 64 - 1) / (SPLIT_TILES * 64));
}
// Paged caches: the cached rows of sequence b, token j, live at pool row
// table[b * ld + j / PAGE_ROWS] * PAGE_ROWS + j % PAGE_ROWS (page ids outside
// [0, n_pages) are clamped into it, so a bad table cannot make a kernel read outside the
// pool).  A null table means the contiguous per-sequence layout.
constexpr int PAGE_ROWS = DSA_PAGE_ROWS;
static_assert(PAGE_ROWS == 64, "paged_row() takes the page by a shift of 6");
struct PageTable {
  const int32_t* table = nullptr;
  int64_t ld = 0;       // entries between the tables of consecutive sequences
  int64_t n_pages = 0;  // pages in the pool
};
// The table entry of the page holding token j of sequence b, as stored, and the pool row of
// token j given that entry (clamped into the pool).  Split so that a kernel can load an entry
// early and use it later.
__device__ __forceinline__ int32_t page_entry(const PageTable& pt, int b, int64_t j) {
  return pt.table[(int64_t)b * pt.ld + (j >> 6)];
}
__device__ __forceinline__ int64_t page_entry_row(const PageTable& pt, int64_t p, int64_t j) {
  p = p < 0 ? 0 : p >= pt.n_pages ? pt.n_pages - 1 : p;
  return p * PAGE_ROWS + (j & (PAGE_ROWS - 1));
}
__device__ __forceinline__ int64_t paged_row(const PageTable& pt, int b, int64_t j) {
  return page_entry_row(pt, page_entry(pt, b, j), j);
}
// A 64-key tile of consecutive tokens starting at key0 (a multiple of 64) whose keys are
// clamped to `last`: every key it reads lies on one page, found with one table lookup.
// Returns the pool row of token `first` = min(key0, start of last's page); token j of the
// tile (j in [first, first + 64)) is then at that row + (j - first).
__device__ __forceinline__ int64_t paged_tile_base(const PageTable& pt, int b, int64_t key0, int64_t last,
                                                   int64_t& first) {
  const int64_t last_page0 = last & ~(int64_t)(PAGE_ROWS - 1);
  first = key0 < last_page0 ? key0 : last_page0;
  return paged_row(pt, b, first);
}

struct SplitIdxArgs {
  const uint8_t* q8;
  const float* qs;
  const uint8_t* k8;
  const float* ks;
  const float* w;
  int64_t B, n_q, n_k;
  const int32_t* q_pos;
  int64_t pos_offset, row_begin, n_rows;
  float* scores;
  int64_t ld;
  int32_t key_stride;
  const float* thr;
  uint2* cand;
  uint32_t* cnt;
  const uint8_t* redo;
  int64_t k_bstride;
  PageTable pages = {};  // non-null table: k8 / ks are page pools (key_stride 1 or any)
};
hipError_t launch_idx_split(const SplitIdxArgs& a, hipStream_t st);

struct TopkArgs {
  const float* scores;
  int64_t ld_scores, B, n_rows, n_k;
  const int32_t* q_pos;     // position of row i = q_pos[b] + pos_offset + row_begin + i
  int64_t pos_offset;
  int64_t row_begin;
  int32_t k;
  int32_t* idx;
  int64_t score_rows = 0;  // score rows per sequence (0: n_rows)
  int64_t out_rows = 0;    // idx rows per sequence (0: n_rows); row i goes to idx row out_row0 + i
  int64_t out_row0 = 0;
  const uint8_t* redo = nullptr;  // non-null: only rows b * n_rows + i whose byte is set (long rows)
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
constexpr int64_t TOPK_MAX_N = 262144;

struct MlaArgs {
  const void* q;
  const void* kv;
  const void* v;  // may be null (V = kv[:, :d_v])
  const int32_t* idx;
  int64_t B, n_q, n_k;
  int32_t H, d_qk, d_v, k;
  float sm_scale;
  int32_t dtype;
  void* out;
  float* lse;
  void* ws;
  size_t ws_bytes;
  // element strides (0: dense): between the head rows of q, the rows of kv and v, and the
  // sequences of kv and v
  int64_t ld_q = 0, ld_kv = 0, ld_v = 0, bs_kv = 0, bs_v = 0;
  // at most this many key splits per query (0: as sparse_mla_splits chooses; 1: never split,
  // so no workspace is used)
  int32_t max_split = 0;
  // non-null table: kv is a page pool (bf16 path only; bs_kv unused)
  PageTable pages = {};
};
hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t st);
// workspace of the bf16 kernel when it splits each query's keys over several blocks
size_t sparse_mla_ws_bytes(int64_t B, int64_t n_q, int32_t H, int32_t d_v, int32_t k, int32_t dtype);
int sparse_mla_splits(int64_t B, int64_t n_q, int32_t k, int32_t dtype);

// fused FP8 indexer + streaming top-k: n_q query rows of each of B sequences against
// that sequence's n_k key rows; row r of sequence b sits at position q_pos[b] + r
// (q_pos null: r) and sees keys 0 .. min(position, n_k - 1).  Needs n_k * 128 < 2^32.
struct PrefillTopkArgs {
  const uint8_t* q8;
  const float* qs;
  const uint8_t* k8;
  const float* ks;
  const float* w;
  int64_t B, n_q, n_k;
  const int32_t* q_pos;
  int32_t k;
  int32_t* idx;
  // null: every row.  Otherwise redo[b * n_q + r] != 0 marks the rows to select (a group of
  // 4 rows runs if any of its rows is marked) and the rows below k are left alone.
  const uint8_t* redo = nullptr;
  int64_t k_bstride = 0;    // key rows between sequences of k8 / ks (0: n_k)
  // only rows [row_begin, row_end) of each sequence are selected and written (row_end < 0:
  // up to n_q)
  int64_t row_begin = 0, row_end = -1;
  PageTable pages = {};     // non-null table: k8 / ks are page pools
};
hipError_t launch_prefill_topk(const PrefillTopkArgs& a, hipStream_t st);

// dense FP8 index scores of rows row_begin .. row_begin + n_rows - 1 of each of B sequences
// (row r of sequence b at position (q_pos ? q_pos[b] : 0) + r) into a padded workspace:
// row i of sequence b at scores + (b * rows_pad + i) * ld, rows_pad = n_rows rounded up to
// 16, ld a multiple of 64 covering the keys the rows see rounded up to 64; keys past a
// row's position score -inf, columns past its last 64-key tile are not written.
//
// key_stride S > 1 scores the systematic sample of keys 0, S, 2S, ...: column j of a row
// is key j*S, visible when j*S <= the row's position (ld then covers ceil(n_k / S) columns).
//
// Filter mode (cand != null): instead of storing the scores, each row appends the keys it
// sees whose score is > thr[b * rows_pad + i], as (fp32 score bits, key index) pairs in
// ascending key order, to its SEL_CAND_PITCH-slot list at
// cand + (b * rows_pad + i) * SEL_CAND_PITCH (slots past SEL_CAND_CAP - 1 are counted, not
// stored; slot SEL_CAND_CAP is scratch), and writes the number of such keys to
// cnt[b * rows_pad + i].  key_stride must be 1.
struct DenseIdxArgs {
  const uint8_t* q8;
  const float* qs;
  const uint8_t* k8;
  const float* ks;
  const float* w;
  int64_t B, n_q, n_k;
  const int32_t* q_pos;
  int64_t row_begin, n_rows;
  float* scores;
  int64_t ld;
  int32_t key_stride = 1;
  const float* thr = nullptr;
  uint2* cand = nullptr;
  uint32_t* cnt = nullptr;
  int64_t k_bstride = 0;    // key rows between sequences of k8 / ks (0: n_k)
  PageTable pages = {};     // non-null table: k8 / ks are page pools
};
inline int64_t dense_rows_pad(int64_t n_rows) { return (n_rows + 15) / 16 * 16; }
hipError_t launch_idx_dense(const DenseIdxArgs& a, hipStream_t st);

// Threshold-filtered selection (FP8 prefill and chunks): a row keeps its candidates when at
// least k and at most SEL_CAND_CAP keys pass its threshold.
constexpr int SEL_SAMPLE_STRIDE = 32;
constexpr int SEL_CAND_CAP = 6144;
constexpr int SEL_CAND_PITCH = SEL_CAND_CAP + 8;
inline int64_t sel_sample_ld(int64_t n_k) {
  const int64_t ns = (n_k + SEL_SAMPLE_STRIDE - 1) / SEL_SAMPLE_STRIDE;
  return ns > 0 ? (ns + 63) / 64 * 64 : 64;
}

// Per row i of each sequence b (position q_pos[b] + row_begin + i, n = the keys it sees):
// thr[b * rows_pad + i] = -inf (collect every key) when n <= SEL_CAND_CAP, else the sample
// score of rank r = ceil(m + 5 sqrt(m) + 5), m = k * n_s / n, among the row's n_s visible
// samples at samp + (b * rows_pad + i) * ld_s (-0 read as +0).
struct SelThresholdArgs {
  const float* samp;
  int64_t ld_s, rows_pad, B, n_rows, n_k;
  const int32_t* q_pos;
  int64_t row_begin;
  int32_t k;
  float* thr;
};
hipError_t launch_sel_threshold(const SelThresholdArgs& a, hipStream_t st);

// Decode: per row i of sequence b (position q_pos[b] + pos_offset + i, n = the keys it sees),
// the top-k of its candidate segments (the filtering split indexer's, n_segs per row) when
// no segment overflowed and k <= their total <= SEL_CAND_CAP: ascending with ties to the
// lower key, -1 padded, to idx row b * n_rows + i (redo byte 0); every key when n <= k
// (redo 0); else nothing (redo 1).
struct DecCandArgs {
  const uint2* cand;
  const uint32_t* cnt;
  int64_t n_segs;
  int64_t B, n_rows, n_k;
  const int32_t* q_pos;
  int64_t pos_offset;
  int32_t k;
  int32_t* idx;
  uint8_t* redo;
};
hipError_t launch_dec_cand_topk(const DecCandArgs& a, hipStream_t st);

// Per row: the top-k of its candidate list when k <= cnt <= SEL_CAND_CAP (written to idx
// row out_row0 + i of sequence b's out_rows rows, ascending, -1 padded; redo byte 0), every
// key when the row sees at most k (redo 0), else nothing (redo 1: the row's candidates do
// not decide its top-k).  redo[b * out_rows + out_row0 + i].
struct SelCandArgs {
  const uint2* cand;
  const uint32_t* cnt;
  int64_t rows_pad, B, n_rows, n_k;
  const int32_t* q_pos;
  int64_t row_begin;
  int32_t k;
  int32_t* idx;
  int64_t out_rows, out_row0;
  uint8_t* redo;
};
hipError_t launch_sel_candidates(const SelCandArgs& a, hipStream_t st);

// backward of the sparse attention; dkv (and dv when v is separate, fp32 path) are
// zeroed and accumulated
struct MlaBwdArgs {
  const void* q;
  const void* kv;
  const void* v;
  const int32_t* idx;
  const void* out;
  const float* lse;
  const void* dout;
  int64_t B, n_q, n_k;
  int32_t H, d_qk, d_v, k;
  float sm_scale;
  int32_t dtype;
  void* dq;
  float* dkv;
  float* dv;
  void* ws;
};
hipError_t launch_sparse_mla_bwd(const MlaBwdArgs& a, hipStream_t st);
size_t sparse_mla_bwd_ws_bytes(int64_t B, int64_t n_q, int64_t n_k, int32_t k, int32_t dtype);

// index scores at the keys listed in idx [B, n_q, k] (-inf for ids outside [0, n_k))
struct ScoresAtArgs {
  const void* q_idx;
  const float* q_scale;
  const void* k_idx;
  const float* k_scale;
  const float* w;
  const int32_t* idx;
  int64_t B, n_q, n_k;
  int32_t H_I, d_I, k, dtype;
  float* scores;
};
hipError_t launch_indexer_scores_at(const ScoresAtArgs& a, hipStream_t st);

// indexer KL loss over each query's selected keys, given the attention lse per head
struct KlArgs {
  const void* q;
  const void* kv;
  const int32_t* idx;
  const float* lse;
  const float* scores;  // index scores of the selected keys [B, n_q, k]
  int64_t B, n_q, n_k;
  int32_t H, d_qk, k;
  float sm_scale;
  int32_t dtype;
  float* kl;     // [B, n_q]
  float* p_out;  // [B, n_q, k] or null
};
hipError_t launch_indexer_kl(const KlArgs& a, hipStream_t st);

// indexer KL loss of the dense warm-up (every key up to each row's position) for rows
// row_begin .. row_begin + n_rows - 1 of each sequence, their index scores at
// scores + (b * n_rows + i) * ld_s; writes kl [B, n_q] and the dense attention lse
// [B, n_q, H] (or not, when null) of those rows
struct KlDenseArgs {
  const void* q;
  const void* kv;
  const float* scores;
  int64_t ld_s;
  const int32_t* q_pos;
  int64_t row_begin, n_rows;
  int64_t B, n_q, n_k;
  int32_t H, d_qk;
  float sm_scale;
  int32_t dtype;
  float* kl;
  float* lse;
};
hipError_t launch_indexer_kl_dense(const KlDenseArgs& a, hipStream_t st);
constexpr int64_t KL_DENSE_F32_MAX_N = 4096;

// FP8 E4M3FN row quantiser: rows of `groups` groups; group b's row i (source row
// b * n_per + i, ld_x elements apart) goes to destination row b * dst_stride + base + i,
// base = pos ? pos[b] : 0 (rows outside [0, dst_per) skipped); its scale is written
// `repeat` times at scale[dst_row * scale_stride + r].
struct QuantArgs {
  const void* x;
  int32_t dtype;  // DSA_BF16 or DSA_F32
  int64_t groups, n_per, width, ld_x;
  const int32_t* pos;
  int64_t dst_per;
  uint8_t* codes;
  int64_t ld_codes;
  float* scale;
  int64_t scale_stride;
  int32_t repeat;
  int64_t dst_stride = 0;  // destination rows between groups (0: dst_per)
};
hipError_t launch_fp8_quant_rows(const QuantArgs& a, hipStream_t st);

}  // namespace dsa
