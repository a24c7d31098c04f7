// C ABI of libdsa: argument validation, workspace sizing and kernel dispatch.
// Every check happens on the host before anything is enqueued; no exception leaves.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>

#include "dsa_kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, ...)                                   \
  do {                                                       \
    if (!(cond)) return fail(DSA_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)
#define SUPPORT(cond, ...)                                   \
  do {                                                       \
    if (!(cond)) return fail(DSA_ERR_UNSUPPORTED, __VA_ARGS__); \
  } while (0)

int check_indexer_shape(int32_t H_I, int32_t d_I, int32_t dtype) {
  REQUIRE(H_I > 0 && d_I > 0, "H_I and d_I must be positive (got %d, %d)", H_I, d_I);
  if (dtype == DSA_FP8_E4M3) {
    SUPPORT(H_I == 64 && d_I == 128, "FP8 indexer needs H_I=64, d_I=128 (got %d, %d)", H_I, d_I);
  } else if (dtype == DSA_F32) {
    SUPPORT(H_I <= 64 && d_I <= 256, "fp32 indexer needs H_I<=64, d_I<=256 (got %d, %d)", H_I, d_I);
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "indexer dtype %d is not DSA_FP8_E4M3 or DSA_F32", dtype);
  }
  return DSA_OK;
}

int check_attn_shape(int32_t H, int32_t d_qk, int32_t d_v, int32_t k, int32_t dtype, bool has_v) {
  REQUIRE(H > 0 && d_qk > 0 && d_v > 0 && k > 0, "H, d_qk, d_v, k must be positive");
  REQUIRE(has_v || d_v <= d_qk, "d_v (%d) exceeds d_qk (%d) with V = kv[:, :d_v]", d_v, d_qk);
  if (dtype == DSA_BF16) {
    SUPPORT(H == 128 && d_qk == 576 && d_v == 512 && !has_v,
            "bf16 attention needs H=128, d_qk=576, d_v=512, V = kv[:, :512]");
    SUPPORT(k % 32 == 0 && k <= 2048, "bf16 attention needs k a multiple of 32, <= 2048 (got %d)", k);
  } else if (dtype == DSA_F32) {
    SUPPORT(H <= 64 && d_qk <= 256 && d_v <= 256 && k <= 4096,
            "fp32 attention needs H<=64, d_qk<=256, d_v<=256, k<=4096");
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "attention dtype %d is not DSA_BF16 or DSA_F32", dtype);
  }
  return DSA_OK;
}

// Element strides of the attention operands: a row stride covers the row's width; bf16
// rows start 16-byte aligned (the kernels load 16-byte units), so bf16 strides are
// multiples of 8 elements.  A sequence stride covers its n_rows rows.
int check_ld(const char* name, int64_t ld, int64_t width, int32_t dtype) {
  REQUIRE(ld >= width, "%s (%lld) must be >= the row width %lld", name, (long long)ld, (long long)width);
  if (dtype == DSA_BF16) REQUIRE(ld % 8 == 0, "%s (%lld) must be a multiple of 8 elements", name, (long long)ld);
  return DSA_OK;
}
int check_seq(const char* name, int64_t bs, int64_t n_rows, int64_t ld, int32_t dtype) {
  REQUIRE(bs >= n_rows * ld, "%s (%lld) must be >= %lld rows x %lld", name, (long long)bs, (long long)n_rows,
          (long long)ld);
  if (dtype == DSA_BF16) REQUIRE(bs % 8 == 0, "%s (%lld) must be a multiple of 8 elements", name, (long long)bs);
  return DSA_OK;
}
#define CHECK(x)            \
  do {                      \
    const int st_ = (x);    \
    if (st_) return st_;    \
  } while (0)

size_t decode_scores_bytes(int64_t B, int64_t n_k) { return (size_t)B * n_k * sizeof(float); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Decode selection workspace.  Long caches (FP8 indexer, n_k_max >= DEC_FILTER_MIN) take the
// threshold-filtered path: per sequence a 1-in-SEL_SAMPLE_STRIDE key sample's scores, a
// threshold, the candidate segments of the filtering indexer's waves with their counts, and a
// redo byte; the full score rows are written only for sequences the candidates do not decide.
constexpr int64_t DEC_FILTER_MIN = 16384;
struct DecWs {
  float* scores;
  float* samp;
  float* thr;
  uint32_t* cnt;
  uint8_t* redo;
  uint2* cand;
};
bool dec_filtered(int64_t n_k_max, int32_t idx_dtype) {
  return idx_dtype == DSA_FP8_E4M3 && n_k_max >= DEC_FILTER_MIN;
}
size_t dec_sel_bytes(int64_t B, int64_t n_k_max, int32_t idx_dtype, DecWs* out = nullptr, void* base = nullptr) {
  const size_t o_samp = align256(decode_scores_bytes(B, n_k_max));
  if (!dec_filtered(n_k_max, idx_dtype)) {
    if (out) *out = DecWs{(float*)base, nullptr, nullptr, nullptr, nullptr, nullptr};
    return o_samp;
  }
  const size_t o_thr = o_samp + align256((size_t)B * dsa::sel_sample_ld(n_k_max) * sizeof(float));
  const size_t o_cnt = o_thr + align256((size_t)B * sizeof(float));
  const size_t o_redo = o_cnt + align256((size_t)B * dsa::dec_split_segments(n_k_max) * sizeof(uint32_t));
  const int64_t segs = dsa::dec_split_segments(n_k_max);
  const size_t o_cand = o_redo + align256((size_t)B);
  const size_t total = o_cand + align256((size_t)B * segs * dsa::DEC_SEG * sizeof(uint2));
  if (out) {
    char* p = (char*)base;
    *out = DecWs{(float*)p, (float*)(p + o_samp), (float*)(p + o_thr), (uint32_t*)(p + o_cnt), (uint8_t*)(p + o_redo),
                 (uint2*)(p + o_cand)};
  }
  return total;
}


// largest key count of the fused selection (32-bit byte offsets within a sequence's keys)
constexpr int64_t FUSED_MAX_KEYS = ((int64_t)1 << 25) - 1;

// FP8 selection by threshold filtering (see topk.hip): per chunk of query rows (up to 16384
// rows over all sequences), a 1-in-SEL_SAMPLE_STRIDE key sample of every row's scores, each row's
// threshold from its sample, the filtering indexer's candidate lists, and the top-k of each
// list; then the streaming exact selection for the rows whose list did not decide them.
// Workspace: the per-row redo bytes of all rows, then one chunk's thresholds, counts,
// sample rows and candidate lists (about 1 GiB for 16384 rows of 128K keys).
struct SelWs {
  uint8_t* redo;
  float* thr;
  uint32_t* cnt;
  float* samp;
  uint2* cand;
};
static int64_t sel_chunk_rows(int64_t B, int64_t n_rows) {
  const int64_t pad = dsa::dense_rows_pad(n_rows);
  int64_t rows = 16384 / B / 16 * 16;
  rows = rows > 16 ? rows : 16;
  return pad < rows ? pad : rows;
}
static size_t sel_ws_bytes(int64_t B, int64_t n_q, int64_t n_k, SelWs* ws_out = nullptr, void* base = nullptr) {
  const int64_t rp = sel_chunk_rows(B, n_q);
  const size_t o_thr = align256((size_t)B * n_q);
  const size_t o_cnt = o_thr + align256((size_t)B * rp * 4);
  const size_t o_samp = o_cnt + align256((size_t)B * rp * 4);
  const size_t o_cand = o_samp + align256((size_t)B * rp * dsa::sel_sample_ld(n_k) * sizeof(float));
  const size_t total = o_cand + align256((size_t)B * rp * dsa::SEL_CAND_PITCH * sizeof(uint2));
  if (ws_out) {
    char* p = (char*)base;
    *ws_out = SelWs{(uint8_t*)p, (float*)(p + o_thr), (uint32_t*)(p + o_cnt), (float*)(p + o_samp),
                    (uint2*)(p + o_cand)};
  }
  return total;
}
// the filtered path covers keys up to TOPK_MAX_N (its sample select runs in LDS); longer
// contexts use the streaming exact selection alone, which needs no workspace
static bool sel_filtered(int64_t n_k) { return n_k <= dsa::TOPK_MAX_N; }
static size_t sel_bytes(int64_t B, int64_t n_q, int64_t n_k) {
  return sel_filtered(n_k) ? sel_ws_bytes(B, n_q, n_k) : 0;
}

// rows 0 .. n_q - 1 of each of B sequences (row r at position (q_pos ? q_pos[b] : 0) + r)
// (kbs: key rows between the sequences of k8 / ks; 0 means n_k)
// chunk_done (optional): called after each chunk with its rows [r0, r0 + n), once they are
// final on stream s; the chunk's undecided rows are then selected before the call instead of
// in one pass after the last chunk.
using ChunkHook = std::function<int(int64_t r0, int64_t n)>;
static int select_fp8(const uint8_t* q8, const float* qs, const uint8_t* k8, const float* ks, const float* w,
                      int64_t B, int64_t n_q, int64_t n_k, const int32_t* q_pos, int32_t k, int32_t* idx, void* ws,
                      size_t ws_bytes, hipStream_t s, int64_t kbs = 0, const ChunkHook* chunk_done = nullptr,
                      const dsa::PageTable& pages = dsa::PageTable{}) {
  SUPPORT(n_k <= FUSED_MAX_KEYS, "FP8 selection supports up to %lld keys", (long long)FUSED_MAX_KEYS);
  dsa::PrefillTopkArgs pa{q8, qs, k8, ks, w, B, n_q, n_k, q_pos, k, idx, nullptr, kbs};
  pa.pages = pages;
  if (!sel_filtered(n_k)) return hip_status(dsa::launch_prefill_topk(pa, s), "indexer/top-k launch");
  SelWs sw;
  const size_t need = sel_ws_bytes(B, n_q, n_k, &sw, ws);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "FP8 selection needs %zu workspace bytes (got %zu)", need, ws_bytes);
  REQUIRE(aligned16(ws), "workspace must be 16-byte aligned");
  const int64_t rows = sel_chunk_rows(B, n_q);
  const int64_t ld_s = dsa::sel_sample_ld(n_k);
  for (int64_t r0 = 0; r0 < n_q; r0 += rows) {
    const int64_t n = rows < n_q - r0 ? rows : n_q - r0;
    const int64_t rp = dsa::dense_rows_pad(n);
    dsa::DenseIdxArgs sa{q8, qs, k8, ks, w, B, n_q, n_k, q_pos, r0, n, sw.samp, ld_s, dsa::SEL_SAMPLE_STRIDE,
                         nullptr, nullptr, nullptr, kbs};
    sa.pages = pages;
    int st = hip_status(dsa::launch_idx_dense(sa, s), "key-sample indexer launch");
    if (st) return st;
    dsa::SelThresholdArgs ta{sw.samp, ld_s, rp, B, n, n_k, q_pos, r0, k, sw.thr};
    st = hip_status(dsa::launch_sel_threshold(ta, s), "threshold launch");
    if (st) return st;
    dsa::DenseIdxArgs fa{q8, qs, k8, ks, w, B, n_q, n_k, q_pos, r0, n, nullptr, 0, 1, sw.thr, sw.cand, sw.cnt, kbs};
    fa.pages = pages;
    st = hip_status(dsa::launch_idx_dense(fa, s), "filtering indexer launch");
    if (st) return st;
    dsa::SelCandArgs ca{sw.cand, sw.cnt, rp, B, n, n_k, q_pos, r0, k, idx, n_q, r0, sw.redo};
    st = hip_status(dsa::launch_sel_candidates(ca, s), "candidate top-k launch");
    if (st) return st;
    if (chunk_done) {
      dsa::PrefillTopkArgs pc = pa;
      pc.redo = sw.redo;
      pc.row_begin = r0;
      pc.row_end = r0 + n;
      st = hip_status(dsa::launch_prefill_topk(pc, s), "exact selection of the chunk's remaining rows");
      if (st) return st;
      st = (*chunk_done)(r0, n);
      if (st) return st;
    }
  }
  if (chunk_done) return DSA_OK;
  pa.redo = sw.redo;
  return hip_status(dsa::launch_prefill_topk(pa, s), "exact selection of the remaining rows");
}

// dense warm-up KL: query rows per pass, so that one pass's score rows take at most 2^28
// floats (1 GiB)
static int64_t kl_dense_rows(int64_t B, int64_t n_q, int64_t n_k) {
  int64_t r = ((int64_t)1 << 28) / (B * (n_k > 0 ? n_k : 1));
  r = r < 1 ? 1 : r;
  r = r < 65535 ? r : 65535;
  return r < n_q ? r : n_q;
}
static size_t kl_dense_ws_bytes(int64_t B, int64_t n_q, int64_t n_k) {
  return align256((size_t)B * kl_dense_rows(B, n_q, n_k) * n_k * sizeof(float));
}

// the fp32 chunk path ranks materialised scores; the FP8 path filters on chip
size_t chunk_scores_bytes(int64_t B, int64_t n_q, int64_t n_k, int32_t attn_dtype) {
  return attn_dtype == DSA_F32 ? align256((size_t)B * n_q * n_k * sizeof(float)) : sel_bytes(B, n_q, n_k);
}

}  // namespace

namespace dsa {
int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}
}  // namespace dsa

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG: invalid argument";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: no kernel for this dtype or shape";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
    case DSA_ERR_HIP: return "DSA_ERR_HIP: HIP runtime error";
    default: return "unknown dsa status";
  }
}

const char* dsa_last_error(void) { return g_err; }

size_t dsa_workspace_size(int32_t op, int64_t B, int64_t n_q, int64_t n_k, int32_t H, int32_t d_v,
                          int32_t k, int32_t dtype) {
  if (B <= 0 || n_q < 0 || n_k < 0 || H <= 0 || d_v <= 0 || k <= 0) return 0;
  switch (op) {
    case DSA_OP_SPARSE_MLA:
      return dsa::sparse_mla_ws_bytes(B, n_q, H, d_v, k, dtype);
    case DSA_OP_PREFILL:
      if (dtype == DSA_F32)  // fp32 path ranks materialised scores
        return align256((size_t)n_q * n_k * sizeof(float)) + dsa::sparse_mla_ws_bytes(1, n_q, H, d_v, k, dtype);
      return sel_bytes(1, n_q, n_k) + dsa::sparse_mla_ws_bytes(1, n_q, H, d_v, k, dtype);
    case DSA_OP_SELECT:
      return dtype == DSA_F32 ? align256((size_t)n_q * n_k * sizeof(float)) : sel_bytes(1, n_q, n_k);
    case DSA_OP_DECODE:
      // the attention dtype selects the pair: bf16 attention goes with the FP8 indexer
      return dec_sel_bytes(B, n_k, dtype == DSA_BF16 ? DSA_FP8_E4M3 : DSA_F32) +
             dsa::sparse_mla_ws_bytes(B, 1, H, d_v, k, dtype);
    case DSA_OP_MLA_BWD:
      return dsa::sparse_mla_bwd_ws_bytes(B, n_q, n_k, k, dtype);
    case DSA_OP_CHUNK:
      return chunk_scores_bytes(B, n_q, n_k, dtype) + dsa::sparse_mla_ws_bytes(B, n_q, H, d_v, k, dtype);
    case DSA_OP_KL_DENSE:
      return kl_dense_ws_bytes(B, n_q, n_k);
    default:
      return 0;
  }
}

int dsa_indexer(const void* q_idx, const float* q_scale, const void* k_idx, const float* k_scale,
                const float* w, int64_t B, int64_t n_q, int64_t n_k, const int32_t* q_pos, int32_t H_I,
                int32_t d_I, int32_t dtype, int64_t row_begin, int64_t n_rows, float* scores,
                int64_t ld_scores, dsa_stream_t stream) {
  REQUIRE(q_idx && q_scale && k_idx && k_scale && w && scores, "null pointer argument");
  REQUIRE(B > 0 && n_q > 0 && n_k > 0, "B, n_q, n_k must be positive");
  REQUIRE(B <= 65535, "B must be <= 65535");
  REQUIRE(row_begin >= 0 && n_rows > 0 && row_begin + n_rows <= n_q, "row range outside [0, n_q)");
  REQUIRE(n_rows <= 65535 || (n_rows + 3) / 4 <= 2147483647LL, "too many rows");
  REQUIRE(ld_scores >= n_k, "ld_scores (%lld) < n_k (%lld)", (long long)ld_scores, (long long)n_k);
  int st = check_indexer_shape(H_I, d_I, dtype);
  if (st) return st;
  if (dtype == DSA_FP8_E4M3) REQUIRE(aligned16(q_idx) && aligned16(k_idx), "FP8 operands must be 16-byte aligned");
  if (dtype == DSA_F32 || n_rows * B <= 512) REQUIRE(n_rows <= 65535, "n_rows must be <= 65535 here");
  dsa::IndexerArgs a{q_idx, q_scale, k_idx, k_scale, w, B, n_q, n_k, q_pos, 0, H_I, d_I, dtype,
                     row_begin, n_rows, scores, ld_scores};
  return hip_status(dsa::launch_indexer(a, (hipStream_t)stream), "dsa_indexer launch");
}

int dsa_topk(const float* scores, int64_t ld_scores, int64_t B, int64_t n_rows, int64_t n_k,
             const int32_t* q_pos, int64_t row_begin, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
             dsa_stream_t stream) {
  (void)ws;
  (void)ws_bytes;
  REQUIRE(scores && idx, "null pointer argument");
  REQUIRE(B > 0 && B <= 65535 && n_rows > 0 && n_k > 0 && k > 0, "B, n_rows, n_k, k must be positive");
  REQUIRE(n_rows <= 2147483647LL, "too many rows");
  REQUIRE(row_begin >= 0, "row_begin must be >= 0");
  REQUIRE(ld_scores >= n_k, "ld_scores < n_k");
  SUPPORT(n_k <= dsa::TOPK_MAX_N, "dsa_topk supports n_k <= %lld", (long long)dsa::TOPK_MAX_N);
  SUPPORT(k <= 65536, "dsa_topk supports k <= 65536");
  dsa::TopkArgs a{scores, ld_scores, B, n_rows, n_k, q_pos, 0, row_begin, k, idx};
  return hip_status(dsa::launch_topk(a, (hipStream_t)stream), "dsa_topk launch");
}

int dsa_sparse_mla(const void* q, int64_t ld_q, const void* kv, int64_t ld_kv, const void* v, int64_t ld_v,
                   const int32_t* idx, int64_t B, int64_t n_q, int64_t n_k, int32_t H, int32_t d_qk, int32_t d_v,
                   int32_t k, float sm_scale, int32_t dtype, void* out, float* lse, void* ws, size_t ws_bytes,
                   dsa_stream_t stream) {
  REQUIRE(q && kv && idx && out, "null pointer argument");
  REQUIRE(B > 0 && B <= 65535 && n_q > 0 && n_k > 0, "B, n_q, n_k must be positive");
  int st = check_attn_shape(H, d_qk, d_v, k, dtype, v != nullptr);
  if (st) return st;
  CHECK(check_ld("ld_q", ld_q, d_qk, dtype));
  CHECK(check_ld("ld_kv", ld_kv, d_qk, dtype));
  if (v) CHECK(check_ld("ld_v", ld_v, d_v, dtype));
  if (dtype == DSA_BF16) REQUIRE(aligned16(q) && aligned16(kv) && aligned16(out), "bf16 operands must be 16-byte aligned");
  REQUIRE(n_q * H <= 2147483647LL, "n_q * H too large");
  const size_t need = dsa::sparse_mla_ws_bytes(B, n_q, H, d_v, k, dtype);
  if (need && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "dsa_sparse_mla needs %zu workspace bytes (got %zu)", need, ws_bytes);
  dsa::MlaArgs a{q, kv, v, idx, B, n_q, n_k, H, d_qk, d_v, k, sm_scale, dtype, out, lse, ws, ws_bytes,
                 ld_q, ld_kv, v ? ld_v : 0, n_k * ld_kv, v ? n_k * ld_v : 0};
  return hip_status(dsa::launch_sparse_mla(a, (hipStream_t)stream), "dsa_sparse_mla launch");
}

// A second stream (default priority) per host thread and device.  The prefill runs the
// attention of each finished selection chunk on it, beside the selection of the next chunk,
// and the caller's stream waits for it before the call's work ends.  Created on first use and
// never released (like the handles of a runtime, they go with the process).
struct AuxStream {
  hipStream_t s = nullptr;
  hipEvent_t ev = nullptr;
};
static AuxStream* aux_stream() {
  constexpr int MAX_DEVICES = 64;
  thread_local AuxStream aux[MAX_DEVICES];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  AuxStream& a = aux[dev];
  if (!a.s) {
    hipStream_t st = nullptr;
    hipEvent_t ev = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
      (void)hipStreamDestroy(st);
      return nullptr;
    }
    a.s = st;
    a.ev = ev;
  }
  return &a;
}

static int select_prefill(const void* q_idx, const float* q_scale, const void* k_idx, const float* k_scale,
                          const float* w, int64_t L, int32_t H_I, int32_t d_I, int32_t k, int32_t idx_dtype,
                          int32_t* idx, void* ws, size_t ws_bytes, hipStream_t s) {
  if (idx_dtype == DSA_FP8_E4M3) {
    SUPPORT(k <= 2048, "FP8 selection keeps at most 2048 keys (k = %d)", k);
    return select_fp8((const uint8_t*)q_idx, q_scale, (const uint8_t*)k_idx, k_scale, w, 1, L, L, nullptr, k, idx,
                      ws, ws_bytes, s);
  }
  SUPPORT(L <= 16384, "fp32 prefill supports L <= 16384");
  const size_t need = align256((size_t)L * L * sizeof(float));
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "fp32 selection needs %zu workspace bytes (got %zu)", need, ws_bytes);
  REQUIRE(aligned16(ws), "workspace must be 16-byte aligned");
  float* scores = (float*)ws;
  dsa::IndexerArgs ia{q_idx, q_scale, k_idx, k_scale, w, 1, L, L, nullptr, 0, H_I, d_I, idx_dtype, 0, L, scores, L};
  int st = hip_status(dsa::launch_indexer(ia, s), "prefill indexer launch");
  if (st) return st;
  dsa::TopkArgs ta{scores, L, 1, L, L, nullptr, 0, 0, k, idx};
  return hip_status(dsa::launch_topk(ta, s), "prefill top-k launch");
}

int dsa_select_prefill(const void* q_idx, const float* q_scale, const void* k_idx, const float* k_scale,
                       const float* w, int64_t L, int32_t H_I, int32_t d_I, int32_t k, int32_t idx_dtype,
                       int32_t* idx, void* ws, size_t ws_bytes, dsa_stream_t stream) {
  REQUIRE(q_idx && q_scale && k_idx && k_scale && w && idx, "null pointer argument");
  REQUIRE(L > 0 && L <= 2147483647LL, "L must be in [1, 2^31)");
  REQUIRE(k > 0, "k must be positive");
  int st = check_indexer_shape(H_I, d_I, idx_dtype);
  if (st) return st;
  if (idx_dtype == DSA_FP8_E4M3) REQUIRE(aligned16(q_idx) && aligned16(k_idx), "FP8 operands must be 16-byte aligned");
  return select_prefill(q_idx, q_scale, k_idx, k_scale, w, L, H_I, d_I, k, idx_dtype, idx, ws, ws_bytes,
                        (hipStream_t)stream);
}

int dsa_forward_prefill(const void* q_idx, const float* q_scale, const void* k_idx, const float* k_scale,
                        const float* w, const void* q, int64_t ld_q, const void* kv, int64_t ld_kv, const void* v,
                        int64_t ld_v, int64_t L, int32_t H_I, int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v,
                        int32_t k, float sm_scale, int32_t idx_dtype, int32_t attn_dtype, int32_t* idx, void* out,
                        float* lse, void* ws, size_t ws_bytes, dsa_stream_t stream) {
  REQUIRE(q_idx && q_scale && k_idx && k_scale && w && q && kv && idx && out, "null pointer argument");
  REQUIRE(L > 0 && L <= 2147483647LL, "L must be in [1, 2^31)");
  int st = check_indexer_shape(H_I, d_I, idx_dtype);
  if (st) return st;
  st = check_attn_shape(H, d_qk, d_v, k, attn_dtype, v != nullptr);
  if (st) return st;
  CHECK(check_ld("ld_q", ld_q, d_qk, attn_dtype));
  CHECK(check_ld("ld_kv", ld_kv, d_qk, attn_dtype));
  if (v) CHECK(check_ld("ld_v", ld_v, d_v, attn_dtype));
  if (idx_dtype == DSA_FP8_E4M3) REQUIRE(aligned16(q_idx) && aligned16(k_idx), "FP8 operands must be 16-byte aligned");
  if (attn_dtype == DSA_BF16) REQUIRE(aligned16(q) && aligned16(kv) && aligned16(out), "bf16 operands must be 16-byte aligned");
  SUPPORT(idx_dtype == attn_dtype || (idx_dtype == DSA_FP8_E4M3 && attn_dtype == DSA_BF16),
          "prefill pairs an FP8 indexer with bf16 attention, or fp32 with fp32");
  SUPPORT(idx_dtype != DSA_FP8_E4M3 || k <= 2048, "FP8 selection keeps at most 2048 keys");
  const bool f32 = idx_dtype == DSA_F32;
  if (f32) SUPPORT(L <= 16384, "fp32 prefill supports L <= 16384");
  const size_t s_bytes = f32 ? align256((size_t)L * L * sizeof(float)) : sel_bytes(1, L, L);
  const size_t need = s_bytes + dsa::sparse_mla_ws_bytes(1, L, H, d_v, k, attn_dtype);
  if (need && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "dsa_forward_prefill needs %zu workspace bytes (got %zu)", need, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  // FP8 selection in several chunks: each chunk's attention runs on a second stream while the
  // next chunk is selected (the two kernels share the GPU; run back to back they take a few
  // per cent longer).  Chunk launches never split their keys, so they need no workspace.
  AuxStream* aux = nullptr;
  if (!f32 && attn_dtype == DSA_BF16 && sel_filtered(L) && sel_chunk_rows(1, L) < L) aux = aux_stream();
  if (aux) {
    bool forked = false;
    const ChunkHook mla_chunk = [&](int64_t r0, int64_t n) -> int {
      int e = hip_status(hipEventRecord(aux->ev, s), "prefill: event record");
      if (e) return e;
      e = hip_status(hipStreamWaitEvent(aux->s, aux->ev, 0), "prefill: stream wait");
      if (e) return e;
      forked = true;
      dsa::MlaArgs a{(const uint16_t*)q + r0 * H * ld_q, kv, v, idx + r0 * k, 1, n, L, H, d_qk, d_v, k, sm_scale,
                     attn_dtype, (uint16_t*)out + r0 * H * d_v, lse ? lse + r0 * H : nullptr, nullptr, 0, ld_q,
                     ld_kv, v ? ld_v : 0, L * ld_kv, v ? L * ld_v : 0};
      a.max_split = 1;
      return hip_status(dsa::launch_sparse_mla(a, aux->s), "prefill sparse attention launch (chunk)");
    };
    st = select_fp8((const uint8_t*)q_idx, q_scale, (const uint8_t*)k_idx, k_scale, w, 1, L, L, nullptr, k, idx, ws,
                    s_bytes, s, 0, &mla_chunk);
    if (forked) {
      // join, whatever happened: the caller's stream waits for every attention launch
      int e = hip_status(hipEventRecord(aux->ev, aux->s), "prefill: event record");
      if (!e) e = hip_status(hipStreamWaitEvent(s, aux->ev, 0), "prefill: stream wait");
      if (e) (void)hipStreamSynchronize(aux->s);
      if (!st) st = e;
    }
    return st;
  }
  st = select_prefill(q_idx, q_scale, k_idx, k_scale, w, L, H_I, d_I, k, idx_dtype, idx, ws, s_bytes, s);
  if (st) return st;
  dsa::MlaArgs a{q, kv, v, idx, 1, L, L, H, d_qk, d_v, k, sm_scale, attn_dtype, out, lse,
                 (char*)ws + s_bytes, ws_bytes - s_bytes, ld_q, ld_kv, v ? ld_v : 0, L * ld_kv, v ? L * ld_v : 0};
  return hip_status(dsa::launch_sparse_mla(a, s), "prefill sparse attention launch");
}

// Strides of the per-sequence caches and of q (decode and chunks).
static int check_cache_strides(int64_t n_k_max, int64_t kc_seq_stride, const void* v_cache, int64_t ld_q, int64_t ld_kv,
                        int64_t kv_seq_stride, int64_t ld_v, int64_t v_seq_stride, int32_t d_qk, int32_t d_v,
                        int32_t attn_dtype) {
  REQUIRE(kc_seq_stride >= n_k_max, "kc_seq_stride (%lld) must be >= n_k_max (%lld)", (long long)kc_seq_stride,
          (long long)n_k_max);
  CHECK(check_ld("ld_q", ld_q, d_qk, attn_dtype));
  CHECK(check_ld("ld_kv", ld_kv, d_qk, attn_dtype));
  CHECK(check_seq("kv_seq_stride", kv_seq_stride, n_k_max, ld_kv, attn_dtype));
  if (v_cache) {
    CHECK(check_ld("ld_v", ld_v, d_v, attn_dtype));
    CHECK(check_seq("v_seq_stride", v_seq_stride, n_k_max, ld_v, attn_dtype));
  }
  return DSA_OK;
}

// The decode layer once its arguments are checked: selection (filtered for long FP8 caches),
// then the split attention.  With a page table, k_cache / k_cache_scale / kv_cache are page
// pools and the sequence strides are unused.
static int decode_run(int64_t B, const int32_t* ctx_len, int64_t n_k_max, const void* q_idx, const float* q_scale,
                      const float* w, const void* k_cache, const float* k_cache_scale, int64_t kc_seq_stride,
                      const void* q, int64_t ld_q, const void* kv_cache, int64_t ld_kv, int64_t kv_seq_stride,
                      const void* v_cache, int64_t ld_v, int64_t v_seq_stride, int32_t H_I, int32_t d_I, int32_t H,
                      int32_t d_qk, int32_t d_v, int32_t k, float sm_scale, int32_t idx_dtype, int32_t attn_dtype,
                      int32_t* idx, void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t s,
                      const dsa::PageTable& pt, const char* name) {
  DecWs dw;
  const size_t s_bytes = dec_sel_bytes(B, n_k_max, idx_dtype, &dw, ws);
  const size_t need = s_bytes + dsa::sparse_mla_ws_bytes(B, 1, H, d_v, k, attn_dtype);
  if (!ws || ws_bytes < need) return fail(DSA_ERR_WORKSPACE, "%s needs %zu workspace bytes (got %zu)", name, need, ws_bytes);
  REQUIRE(aligned16(ws), "workspace must be 16-byte aligned");
  int st = DSA_OK;
  const uint8_t* q8 = (const uint8_t*)q_idx;
  const uint8_t* k8 = (const uint8_t*)k_cache;
  // the query of sequence b is its row 0, at position ctx_len[b] - 1
  if (dec_filtered(n_k_max, idx_dtype)) {
    const int64_t ld_s = dsa::sel_sample_ld(n_k_max);
    // 1. scores of every SEL_SAMPLE_STRIDE-th key; 2. each sequence's threshold (and its
    // candidate count zeroed); 3. the filtering indexer appends the keys above it; 4. the
    // top-k of each candidate list; 5. sequences whose list did not decide them: full score
    // rows and the exact row selection (both launches skip every other sequence)
    dsa::SplitIdxArgs sa{q8, q_scale, k8, k_cache_scale, w, B, 1, n_k_max, ctx_len, -1, 0, 1, dw.samp, ld_s,
                         dsa::SEL_SAMPLE_STRIDE, nullptr, nullptr, nullptr, nullptr, kc_seq_stride};
    sa.pages = pt;
    st = hip_status(dsa::launch_idx_split(sa, s), "decode key-sample indexer launch");
    if (st) return st;
    dsa::SelThresholdArgs ta{dw.samp, ld_s, 1, B, 1, n_k_max, ctx_len, -1, k, dw.thr};
    st = hip_status(dsa::launch_sel_threshold(ta, s), "decode threshold launch");
    if (st) return st;
    dsa::SplitIdxArgs fa{q8, q_scale, k8, k_cache_scale, w, B, 1, n_k_max, ctx_len, -1, 0, 1, nullptr, 0, 1,
                         dw.thr, dw.cand, dw.cnt, nullptr, kc_seq_stride};
    fa.pages = pt;
    st = hip_status(dsa::launch_idx_split(fa, s), "decode filtering indexer launch");
    if (st) return st;
    dsa::DecCandArgs ca{dw.cand, dw.cnt, dsa::dec_split_segments(n_k_max), B, 1, n_k_max, ctx_len, -1, k, idx,
                        dw.redo};
    st = hip_status(dsa::launch_dec_cand_topk(ca, s), "decode candidate top-k launch");
    if (st) return st;
    dsa::SplitIdxArgs ra{q8, q_scale, k8, k_cache_scale, w, B, 1, n_k_max, ctx_len, -1, 0, 1, dw.scores, n_k_max,
                         1, nullptr, nullptr, nullptr, dw.redo, kc_seq_stride};
    ra.pages = pt;
    st = hip_status(dsa::launch_idx_split(ra, s), "decode indexer launch (undecided sequences)");
    if (st) return st;
    dsa::TopkArgs tk{dw.scores, n_k_max, B, 1, n_k_max, ctx_len, -1, 0, k, idx, 0, 0, 0, dw.redo};
    st = hip_status(dsa::launch_topk(tk, s), "decode top-k launch (undecided sequences)");
    if (st) return st;
  } else {
    if (pt.table) {  // paged caches are FP8: the split indexer reads them through the table
      dsa::SplitIdxArgs ia{q8, q_scale, k8, k_cache_scale, w, B, 1, n_k_max, ctx_len, -1, 0, 1, dw.scores,
                           n_k_max, 1, nullptr, nullptr, nullptr, nullptr, 0};
      ia.pages = pt;
      st = hip_status(dsa::launch_idx_split(ia, s), "decode indexer launch");
    } else {
      dsa::IndexerArgs ia{q_idx, q_scale, k_cache, k_cache_scale, w, B, 1, n_k_max, ctx_len, -1, H_I, d_I,
                          idx_dtype, 0, 1, dw.scores, n_k_max, kc_seq_stride};
      st = hip_status(dsa::launch_indexer(ia, s), "decode indexer launch");
    }
    if (st) return st;
    dsa::TopkArgs ta{dw.scores, n_k_max, B, 1, n_k_max, ctx_len, -1, 0, k, idx};
    st = hip_status(dsa::launch_topk(ta, s), "decode top-k launch");
    if (st) return st;
  }
  dsa::MlaArgs a{q, kv_cache, v_cache, idx, B, 1, n_k_max, H, d_qk, d_v, k, sm_scale, attn_dtype,
                 out, lse, (char*)ws + s_bytes, ws_bytes - s_bytes, ld_q, ld_kv, v_cache ? ld_v : 0,
                 kv_seq_stride, v_cache ? v_seq_stride : 0};
  a.pages = pt;
  return hip_status(dsa::launch_sparse_mla(a, s), "decode sparse attention launch");
}

int dsa_forward_decode(int64_t B, const int32_t* ctx_len, int64_t n_k_max, const void* q_idx, const float* q_scale,
                       const float* w, const void* k_cache, const float* k_cache_scale, int64_t kc_seq_stride,
                       const void* q, int64_t ld_q, const void* kv_cache, int64_t ld_kv, int64_t kv_seq_stride,
                       const void* v_cache, int64_t ld_v, int64_t v_seq_stride, int32_t H_I, int32_t d_I, int32_t H,
                       int32_t d_qk, int32_t d_v, int32_t k, float sm_scale, int32_t idx_dtype, int32_t attn_dtype,
                       int32_t* idx, void* out, float* lse, void* ws, size_t ws_bytes, dsa_stream_t stream) {
  REQUIRE(ctx_len && q_idx && q_scale && w && k_cache && k_cache_scale && q && kv_cache && idx && out,
          "null pointer argument");
  REQUIRE(B > 0 && B <= 65535 && n_k_max > 0, "B in [1, 65535] and n_k_max > 0 required");
  int st = check_indexer_shape(H_I, d_I, idx_dtype);
  if (st) return st;
  st = check_attn_shape(H, d_qk, d_v, k, attn_dtype, v_cache != nullptr);
  if (st) return st;
  CHECK(check_cache_strides(n_k_max, kc_seq_stride, v_cache, ld_q, ld_kv, kv_seq_stride, ld_v, v_seq_stride, d_qk,
                            d_v, attn_dtype));
  SUPPORT(n_k_max <= dsa::TOPK_MAX_N, "decode supports n_k_max <= %lld", (long long)dsa::TOPK_MAX_N);
  if (idx_dtype == DSA_FP8_E4M3) REQUIRE(aligned16(q_idx) && aligned16(k_cache), "FP8 operands must be 16-byte aligned");
  if (attn_dtype == DSA_BF16) REQUIRE(aligned16(q) && aligned16(kv_cache) && aligned16(out), "bf16 operands must be 16-byte aligned");
  SUPPORT(idx_dtype == attn_dtype || (idx_dtype == DSA_FP8_E4M3 && attn_dtype == DSA_BF16),
          "decode pairs an FP8 indexer with bf16 attention, or fp32 with fp32");
  return decode_run(B, ctx_len, n_k_max, q_idx, q_scale, w, k_cache, k_cache_scale, kc_seq_stride, q, ld_q, kv_cache,
                    ld_kv, kv_seq_stride, v_cache, ld_v, v_seq_stride, H_I, d_I, H, d_qk, d_v, k, sm_scale, idx_dtype,
                    attn_dtype, idx, out, lse, ws, ws_bytes, (hipStream_t)stream, dsa::PageTable{},
                    "dsa_forward_decode");
}

int dsa_forward_decode_paged(int64_t B, const int32_t* ctx_len, int64_t n_k_max, const void* q_idx,
                             const float* q_scale, const float* w, const void* k_pool, const float* k_pool_scale,
                             const void* q, int64_t ld_q, const void* kv_pool, int64_t ld_kv,
                             const int32_t* block_table, int64_t bt_stride, int64_t n_pages, int32_t H_I,
                             int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v, int32_t k, float sm_scale,
                             int32_t idx_dtype, int32_t attn_dtype, int32_t* idx, void* out, float* lse, void* ws,
                             size_t ws_bytes, dsa_stream_t stream) {
  REQUIRE(ctx_len && q_idx && q_scale && w && k_pool && k_pool_scale && q && kv_pool && block_table && idx && out,
          "null pointer argument");
  REQUIRE(B > 0 && B <= 65535 && n_k_max > 0, "B in [1, 65535] and n_k_max > 0 required");
  SUPPORT(idx_dtype == DSA_FP8_E4M3 && attn_dtype == DSA_BF16,
          "paged decode needs an FP8 indexer and bf16 attention");
  int st = check_indexer_shape(H_I, d_I, idx_dtype);
  if (st) return st;
  st = check_attn_shape(H, d_qk, d_v, k, attn_dtype, false);
  if (st) return st;
  CHECK(check_ld("ld_q", ld_q, d_qk, attn_dtype));
  CHECK(check_ld("ld_kv", ld_kv, d_qk, attn_dtype));
  SUPPORT(n_k_max <= dsa::TOPK_MAX_N, "decode supports n_k_max <= %lld", (long long)dsa::TOPK_MAX_N);
  const int64_t pages_per_seq = (n_k_max + dsa::PAGE_ROWS - 1) / dsa::PAGE_ROWS;
  REQUIRE(bt_stride >= pages_per_seq, "bt_stride (%lld) must cover n_k_max (%lld pages of %d rows)",
          (long long)bt_stride, (long long)pages_per_seq, dsa::PAGE_ROWS);
  REQUIRE(n_pages > 0 && n_pages <= 2147483647LL / dsa::PAGE_ROWS, "n_pages must be in [1, 2^31 / %d)",
          dsa::PAGE_ROWS);
  REQUIRE(aligned16(q_idx) && aligned16(k_pool), "FP8 operands must be 16-byte aligned");
  REQUIRE(aligned16(q) && aligned16(kv_pool) && aligned16(out), "bf16 operands must be 16-byte aligned");
  dsa::PageTable pt;
  pt.table = block_table;
  pt.ld = bt_stride;
  pt.n_pages = n_pages;
  return decode_run(B, ctx_len, n_k_max, q_idx, q_scale, w, k_pool, k_pool_scale, 0, q, ld_q, kv_pool, ld_kv, 0,
                    nullptr, 0, 0, H_I, d_I, H, d_qk, d_v, k, sm_scale, idx_dtype, attn_dtype, idx, out, lse, ws,
                    ws_bytes, (hipStream_t)stream, pt, "dsa_forward_decode_paged");
}

int dsa_fp8_quantize_rows(const void* x, int32_t x_dtype, int64_t n_rows, int64_t width, int64_t ld_x,
                          uint8_t* codes, int64_t ld_codes, float* scale, int64_t scale_stride, int32_t repeat,
                          dsa_stream_t stream) {
  REQUIRE(x && codes && scale, "null pointer argument");
  REQUIRE(x_dtype == DSA_BF16 || x_dtype == DSA_F32, "x_dtype must be DSA_BF16 or DSA_F32 (got %d)", x_dtype);
  REQUIRE(n_rows > 0 && width > 0, "n_rows and width must be positive");
  REQUIRE(n_rows <= (int64_t)4 * 2147483647, "n_rows too large");
  REQUIRE(ld_x >= width && ld_codes >= width, "row strides must be >= width");
  REQUIRE(repeat >= 1 && scale_stride >= repeat, "need 1 <= repeat <= scale_stride");
  dsa::QuantArgs a{x, x_dtype, 1, n_rows, width, ld_x, nullptr, n_rows, codes, ld_codes, scale, scale_stride, repeat};
  return hip_status(dsa::launch_fp8_quant_rows(a, (hipStream_t)stream), "fp8 quantiser launch");
}

int dsa_kcache_append(const void* k_new, int32_t dtype, int64_t B, int64_t n_new, int32_t d_I, const int32_t* pos,
                      int64_t n_k_max, int64_t kc_seq_stride, uint8_t* k_cache, float* k_cache_scale,
                      dsa_stream_t stream) {
  REQUIRE(k_new && pos && k_cache && k_cache_scale, "null pointer argument");
  REQUIRE(dtype == DSA_BF16 || dtype == DSA_F32, "dtype must be DSA_BF16 or DSA_F32 (got %d)", dtype);
  REQUIRE(B > 0 && B <= 65535 && n_new > 0 && d_I > 0 && n_k_max > 0, "B in [1, 65535], n_new, d_I, n_k_max > 0");
  REQUIRE(n_new <= (int64_t)4 * 2147483647, "n_new too large");
  REQUIRE(kc_seq_stride >= n_k_max, "kc_seq_stride (%lld) must be >= n_k_max (%lld)", (long long)kc_seq_stride,
          (long long)n_k_max);
  dsa::QuantArgs a{k_new, dtype, B, n_new, d_I, d_I, pos, n_k_max, k_cache, d_I, k_cache_scale, 1, 1, kc_seq_stride};
  return hip_status(dsa::launch_fp8_quant_rows(a, (hipStream_t)stream), "key-cache append launch");
}

// The chunk layer once its arguments are checked.  With a page table (FP8 indexer, bf16
// attention), k_cache / k_cache_scale / kv_cache are page pools and the sequence strides are
// unused.
static int chunk_run(int64_t B, int64_t n_q, const int32_t* q_pos, int64_t n_k_max, const void* q_idx,
                     const float* q_scale, const float* w, const void* k_cache, const float* k_cache_scale,
                     int64_t kc_seq_stride, const void* q, int64_t ld_q, const void* kv_cache, int64_t ld_kv,
                     int64_t kv_seq_stride, const void* v_cache, int64_t ld_v, int64_t v_seq_stride, int32_t H_I,
                     int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v, int32_t k, float sm_scale,
                     int32_t idx_dtype, int32_t attn_dtype, int32_t* idx, void* out, float* lse, void* ws,
                     size_t ws_bytes, hipStream_t s, const dsa::PageTable& pt, const char* name) {
  int st = DSA_OK;
  const size_t s_bytes = chunk_scores_bytes(B, n_q, n_k_max, attn_dtype);
  const size_t need = s_bytes + dsa::sparse_mla_ws_bytes(B, n_q, H, d_v, k, attn_dtype);
  if (need && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "%s needs %zu workspace bytes (got %zu)", name, need, ws_bytes);
  if (need) REQUIRE(aligned16(ws), "workspace must be 16-byte aligned");
  if (idx_dtype == DSA_FP8_E4M3) {
    st = select_fp8((const uint8_t*)q_idx, q_scale, (const uint8_t*)k_cache, k_cache_scale, w, B, n_q, n_k_max,
                    q_pos, k, idx, ws, s_bytes, s, kc_seq_stride, nullptr, pt);
  } else {
    float* scores = (float*)ws;
    dsa::IndexerArgs ia{q_idx, q_scale, k_cache, k_cache_scale, w, B, n_q, n_k_max, q_pos, 0, H_I, d_I,
                        idx_dtype, 0, n_q, scores, n_k_max, kc_seq_stride};
    st = hip_status(dsa::launch_indexer(ia, s), "chunk indexer launch");
    if (st) return st;
    dsa::TopkArgs ta{scores, n_k_max, B, n_q, n_k_max, q_pos, 0, 0, k, idx};
    st = hip_status(dsa::launch_topk(ta, s), "chunk top-k launch");
  }
  if (st) return st;
  dsa::MlaArgs a{q, kv_cache, v_cache, idx, B, n_q, n_k_max, H, d_qk, d_v, k, sm_scale, attn_dtype,
                 out, lse, (char*)ws + s_bytes, ws_bytes - s_bytes, ld_q, ld_kv, v_cache ? ld_v : 0,
                 kv_seq_stride, v_cache ? v_seq_stride : 0};
  a.pages = pt;
  return hip_status(dsa::launch_sparse_mla(a, s), "chunk sparse attention launch");
}

int dsa_forward_chunk(int64_t B, int64_t n_q, const int32_t* q_pos, int64_t n_k_max, const void* q_idx,
                      const float* q_scale, const float* w, const void* k_cache, const float* k_cache_scale,
                      int64_t kc_seq_stride, const void* q, int64_t ld_q, const void* kv_cache, int64_t ld_kv,
                      int64_t kv_seq_stride, const void* v_cache, int64_t ld_v, int64_t v_seq_stride, int32_t H_I,
                      int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v, int32_t k, float sm_scale,
                      int32_t idx_dtype, int32_t attn_dtype, int32_t* idx, void* out, float* lse, void* ws,
                      size_t ws_bytes, dsa_stream_t stream) {
  REQUIRE(q_pos && q_idx && q_scale && w && k_cache && k_cache_scale && q && kv_cache && idx && out,
          "null pointer argument");
  REQUIRE(B > 0 && B <= 65535 && n_q > 0 && n_k_max > 0, "B in [1, 65535], n_q > 0 and n_k_max > 0 required");
  REQUIRE(n_q <= 2147483647LL && n_q * H <= 2147483647LL, "n_q too large");
  int st = check_indexer_shape(H_I, d_I, idx_dtype);
  if (st) return st;
  st = check_attn_shape(H, d_qk, d_v, k, attn_dtype, v_cache != nullptr);
  if (st) return st;
  SUPPORT(idx_dtype == attn_dtype || (idx_dtype == DSA_FP8_E4M3 && attn_dtype == DSA_BF16),
          "a chunk pairs an FP8 indexer with bf16 attention, or fp32 with fp32");
  CHECK(check_cache_strides(n_k_max, kc_seq_stride, v_cache, ld_q, ld_kv, kv_seq_stride, ld_v, v_seq_stride, d_qk,
                            d_v, attn_dtype));
  if (idx_dtype == DSA_FP8_E4M3) {
    REQUIRE(aligned16(q_idx) && aligned16(k_cache), "FP8 operands must be 16-byte aligned");
    SUPPORT(k <= 2048, "FP8 selection keeps at most 2048 keys (k = %d)", k);
    SUPPORT(n_k_max <= FUSED_MAX_KEYS, "FP8 selection supports n_k_max <= %lld", (long long)FUSED_MAX_KEYS);
    REQUIRE(B * ((n_q + 3) / 4) <= 2147483647LL, "B * n_q too large");
  } else {
    SUPPORT(n_k_max <= dsa::TOPK_MAX_N, "fp32 chunk supports n_k_max <= %lld", (long long)dsa::TOPK_MAX_N);
    SUPPORT(n_q <= 65535, "fp32 chunk supports n_q <= 65535");
  }
  if (attn_dtype == DSA_BF16) REQUIRE(aligned16(q) && aligned16(kv_cache) && aligned16(out), "bf16 operands must be 16-byte aligned");
  return chunk_run(B, n_q, q_pos, n_k_max, q_idx, q_scale, w, k_cache, k_cache_scale, kc_seq_stride, q, ld_q,
                   kv_cache, ld_kv, kv_seq_stride, v_cache, ld_v, v_seq_stride, H_I, d_I, H, d_qk, d_v, k, sm_scale,
                   idx_dtype, attn_dtype, idx, out, lse, ws, ws_bytes, (hipStream_t)stream, dsa::PageTable{},
                   "dsa_forward_chunk");
}

int dsa_forward_chunk_paged(int64_t B, int64_t n_q, const int32_t* q_pos, int64_t n_k_max, const void* q_idx,
                            const float* q_scale, const float* w, const void* k_pool, const float* k_pool_scale,
                            const void* q, int64_t ld_q, const void* kv_pool, int64_t ld_kv,
                            const int32_t* block_table, int64_t bt_stride, int64_t n_pages, int32_t H_I,
                            int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v, int32_t k, float sm_scale,
                            int32_t idx_dtype, int32_t attn_dtype, int32_t* idx, void* out, float* lse, void* ws,
                            size_t ws_bytes, dsa_stream_t stream) {
  REQUIRE(q_pos && q_idx && q_scale && w && k_pool && k_pool_scale && q && kv_pool && block_table && idx && out,
          "null pointer argument");
  REQUIRE(B > 0 && B <= 65535 && n_q > 0 && n_k_max > 0, "B in [1, 65535], n_q > 0 and n_k_max > 0 required");
  REQUIRE(n_q <= 2147483647LL && n_q * H <= 2147483647LL, "n_q too large");
  SUPPORT(idx_dtype == DSA_FP8_E4M3 && attn_dtype == DSA_BF16, "paged chunks need an FP8 indexer and bf16 attention");
  int st = check_indexer_shape(H_I, d_I, idx_dtype);
  if (st) return st;
  st = check_attn_shape(H, d_qk, d_v, k, attn_dtype, false);
  if (st) return st;
  CHECK(check_ld("ld_q", ld_q, d_qk, attn_dtype));
  CHECK(check_ld("ld_kv", ld_kv, d_qk, attn_dtype));
  SUPPORT(k <= 2048, "FP8 selection keeps at most 2048 keys (k = %d)", k);
  SUPPORT(n_k_max <= FUSED_MAX_KEYS, "FP8 selection supports n_k_max <= %lld", (long long)FUSED_MAX_KEYS);
  REQUIRE(B * ((n_q + 3) / 4) <= 2147483647LL, "B * n_q too large");
  const int64_t pages_per_seq = (n_k_max + dsa::PAGE_ROWS - 1) / dsa::PAGE_ROWS;
  REQUIRE(bt_stride >= pages_per_seq, "bt_stride (%lld) must cover n_k_max (%lld pages of %d rows)",
          (long long)bt_stride, (long long)pages_per_seq, dsa::PAGE_ROWS);
  REQUIRE(n_pages > 0 && n_pages <= 2147483647LL / dsa::PAGE_ROWS, "n_pages must be in [1, 2^31 / %d)",
          dsa::PAGE_ROWS);
  REQUIRE(aligned16(q_idx) && aligned16(k_pool), "FP8 operands must be 16-byte aligned");
  REQUIRE(aligned16(q) && aligned16(kv_pool) && aligned16(out), "bf16 operands must be 16-byte aligned");
  dsa::PageTable pt;
  pt.table = block_table;
  pt.ld = bt_stride;
  pt.n_pages = n_pages;
  return chunk_run(B, n_q, q_pos, n_k_max, q_idx, q_scale, w, k_pool, k_pool_scale, 0, q, ld_q, kv_pool, ld_kv, 0,
                   nullptr, 0, 0, H_I, d_I, H, d_qk, d_v, k, sm_scale, idx_dtype, attn_dtype, idx, out, lse, ws,
                   ws_bytes, (hipStream_t)stream, pt, "dsa_forward_chunk_paged");
}

int dsa_indexer_scores_at(const void* q_idx, const float* q_scale, const void* k_idx, const float* k_scale,
                          const float* w, const int32_t* idx, int64_t B, int64_t n_q, int64_t n_k, int32_t H_I,
                          int32_t d_I, int32_t k, int32_t dtype, float* scores, dsa_stream_t stream) {
  REQUIRE(q_idx && q_scale && k_idx && k_scale && w && idx && scores, "null pointer argument");
  REQUIRE(B > 0 && B <= 65535 && n_q > 0 && n_k > 0 && k > 0, "B in [1, 65535] and n_q, n_k, k > 0 required");
  int st = check_indexer_shape(H_I, d_I, dtype);
  if (st) return st;
  if (dtype == DSA_FP8_E4M3) {
    REQUIRE(aligned16(q_idx) && aligned16(k_idx), "FP8 operands must be 16-byte aligned");
    REQUIRE((n_q + 3) / 4 <= 2147483647LL, "n_q too large");
  } else {
    REQUIRE(n_q <= 65535, "fp32 path supports n_q <= 65535");
  }
  dsa::ScoresAtArgs a{q_idx, q_scale, k_idx, k_scale, w, idx, B, n_q, n_k, H_I, d_I, k, dtype, scores};
  return hip_status(dsa::launch_indexer_scores_at(a, (hipStream_t)stream), "dsa_indexer_scores_at launch");
}

int dsa_indexer_kl(const void* q, const void* kv, const int32_t* idx, const float* lse, const float* idx_scores,
                   int64_t B, int64_t n_q, int64_t n_k, int32_t H, int32_t d_qk, int32_t k, float sm_scale,
                   int32_t dtype, float* kl, float* p_out, dsa_stream_t stream) {
  REQUIRE(q && kv && idx && lse && idx_scores && kl, "null pointer argument");
  REQUIRE(B > 0 && B <= 65535 && n_q > 0 && n_k > 0, "B in [1, 65535] and n_q, n_k > 0 required");
  REQUIRE(n_q <= 2147483647LL, "n_q too large");
  REQUIRE(H > 0 && d_qk > 0 && k > 0, "H, d_qk, k must be positive");
  if (dtype == DSA_BF16) {
    SUPPORT(H == 128 && d_qk == 576, "bf16 KL loss needs H = 128, d_qk = 576");
    SUPPORT(k % 32 == 0 && k <= 2048, "bf16 KL loss needs k a multiple of 32, <= 2048 (got %d)", k);
    REQUIRE(aligned16(q) && aligned16(kv) && aligned16(idx) && aligned16(idx_scores),
            "bf16 path: q, kv, idx and idx_scores must be 16-byte aligned");
  } else if (dtype == DSA_F32) {
    SUPPORT(H <= 64 && d_qk <= 256 && k <= 4096, "fp32 KL loss needs H <= 64, d_qk <= 256, k <= 4096");
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "KL loss dtype %d is not DSA_BF16 or DSA_F32", dtype);
  }
  dsa::KlArgs a{q, kv, idx, lse, idx_scores, B, n_q, n_k, H, d_qk, k, sm_scale, dtype, kl, p_out};
  return hip_status(dsa::launch_indexer_kl(a, (hipStream_t)stream), "dsa_indexer_kl launch");
}

int dsa_indexer_kl_dense(const void* q_idx, const float* q_scale, const void* k_idx, const float* k_scale,
                         const float* w, const void* q, const void* kv, int64_t B, int64_t n_q, int64_t n_k,
                         const int32_t* q_pos, int32_t H_I, int32_t d_I, int32_t H, int32_t d_qk, float sm_scale,
                         int32_t idx_dtype, int32_t attn_dtype, float* kl, float* lse, void* ws, size_t ws_bytes,
                         dsa_stream_t stream) {
  REQUIRE(q_idx && q_scale && k_idx && k_scale && w && q && kv && kl, "null pointer argument");
  REQUIRE(B > 0 && B <= 65535 && n_q > 0 && n_k > 0, "B in [1, 65535] and n_q, n_k > 0 required");
  REQUIRE(n_q <= 2147483647LL && n_k <= 2147483647LL, "n_q, n_k must be < 2^31");
  CHECK(check_indexer_shape(H_I, d_I, idx_dtype));
  REQUIRE(H > 0 && d_qk > 0, "H and d_qk must be positive");
  if (attn_dtype == DSA_BF16) {
    SUPPORT(H == 128 && d_qk == 576, "bf16 dense KL loss needs H = 128, d_qk = 576");
    REQUIRE(aligned16(q) && aligned16(kv), "bf16 operands must be 16-byte aligned");
  } else if (attn_dtype == DSA_F32) {
    SUPPORT(H <= 64 && d_qk <= 256 && n_k <= dsa::KL_DENSE_F32_MAX_N,
            "fp32 dense KL loss needs H <= 64, d_qk <= 256, n_k <= %lld", (long long)dsa::KL_DENSE_F32_MAX_N);
  } else {
    return fail(DSA_ERR_UNSUPPORTED, "dense KL attention dtype %d is not DSA_BF16 or DSA_F32", attn_dtype);
  }
  if (idx_dtype == DSA_FP8_E4M3) REQUIRE(aligned16(q_idx) && aligned16(k_idx), "FP8 operands must be 16-byte aligned");
  const size_t need = kl_dense_ws_bytes(B, n_q, n_k);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "dsa_indexer_kl_dense needs %zu workspace bytes (got %zu)", need, ws_bytes);
  REQUIRE(aligned16(ws), "workspace must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  float* scores = (float*)ws;
  const int64_t rows = kl_dense_rows(B, n_q, n_k);
  for (int64_t r0 = 0; r0 < n_q; r0 += rows) {
    const int64_t nr = rows < n_q - r0 ? rows : n_q - r0;
    dsa::IndexerArgs ia{q_idx, q_scale, k_idx, k_scale, w, B, n_q, n_k, q_pos, 0, H_I, d_I, idx_dtype, r0, nr,
                        scores, n_k};
    int st = hip_status(dsa::launch_indexer(ia, s), "dense KL indexer launch");
    if (st) return st;
    dsa::KlDenseArgs ka{q, kv, scores, n_k, q_pos, r0, nr, B, n_q, n_k, H, d_qk, sm_scale, attn_dtype, kl, lse};
    st = hip_status(dsa::launch_indexer_kl_dense(ka, s), "dense KL launch");
    if (st) return st;
  }
  return DSA_OK;
}

int dsa_sparse_mla_backward(const void* q, const void* kv, const void* v, const int32_t* idx, const void* out,
                            const float* lse, const void* d_out, int64_t B, int64_t n_q, int64_t n_k, int32_t H,
                            int32_t d_qk, int32_t d_v, int32_t k, float sm_scale, int32_t dtype, void* d_q,
                            float* d_kv, float* d_v_out, void* ws, size_t ws_bytes, dsa_stream_t stream) {
  REQUIRE(q && kv && idx && lse && d_out && d_q && d_kv, "null pointer argument");
  REQUIRE(B > 0 && B <= 65535 && n_q > 0 && n_k > 0, "B in [1, 65535] and n_q, n_k > 0 required");
  REQUIRE(B * n_q <= 2147483647LL, "B * n_q too large");
  int st = check_attn_shape(H, d_qk, d_v, k, dtype, v != nullptr);
  if (st) return st;
  if (dtype == DSA_BF16) {
    REQUIRE(out, "the bf16 backward needs the forward output (out)");
    SUPPORT(n_k * 576 < (1LL << 32), "bf16 backward supports n_k * 576 < 2^32");
    REQUIRE(aligned16(q) && aligned16(kv) && aligned16(out) && aligned16(d_out) && aligned16(d_q) &&
                aligned16(idx) && aligned16(d_kv),
            "bf16 backward operands must be 16-byte aligned");
    const size_t need = dsa::sparse_mla_bwd_ws_bytes(B, n_q, n_k, k, dtype);
    if (!ws || ws_bytes < need)
      return fail(DSA_ERR_WORKSPACE, "dsa_sparse_mla_backward needs %zu workspace bytes (got %zu)", need, ws_bytes);
    REQUIRE(aligned16(ws), "workspace must be 16-byte aligned");
  } else {
    REQUIRE(!v || d_v_out, "a separate V needs d_v_out");
    SUPPORT(n_q <= 65535, "fp32 backward supports n_q <= 65535");
  }
  dsa::MlaBwdArgs a{q, kv, v, idx, out, lse, d_out, B, n_q, n_k, H, d_qk, d_v, k, sm_scale, dtype,
                    d_q, d_kv, d_v_out, ws};
  return hip_status(dsa::launch_sparse_mla_bwd(a, (hipStream_t)stream), "dsa_sparse_mla_backward launch");
}

}  // extern "C"
