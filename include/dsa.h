/*
 * dsa.h -- C ABI of libdsa: DeepSeek Sparse Attention (DSA) forward for one layer on
 * AMD Instinct MI355X (gfx950).
 *
 * DSA has three stages (described on the pages this library follows):
 *   1. lightning indexer: a multi-head ReLU scorer, run in FP8, that gives every query a
 *      score for each of its preceding tokens
 *      ("DeepSeek-V3.2-Exp 技术报告解读" (53ai.com), section 创新架构; WeChat explainer on
 *      juhe.plus, section 第一步：Lightning Indexer);
 *   2. fine-grained token selection: keep the top-k keys per query, k = 2048
 *      (juhe.plus explainer, section 第二步：Fine-grained Token Selection; paperbridge.wiki
 *      summary, section DeepSeek Sparse Attention);
 *   3. attention over the kept keys only, MLA in MQA mode: all query heads share one
 *      latent key-value row (53ai.com, section 创新架构 and Figure 1).
 *
 * Definitions used by every entry point
 * -------------------------------------
 *   index score   I[t,s] = sum_j w[t,j] * ReLU( (q8[t,j,:]*q_scale[t,j]) . (k8[s,:]*k_scale[s]) )
 *                 for keys s <= pos(t) ("preceding tokens" includes the token itself).
 *   selection     S_t = the min(k, pos(t)+1) keys s <= pos(t) ranked highest by
 *                 (I desc, s asc): ties go to the lower key index.  Written as int32 in
 *                 ascending key order, padded with -1.
 *   attention     z_s = sm_scale * q[t,h,:] . kv[s,:]      (s in S_t, every head h)
 *                 O[t,h,:] = sum_s softmax(z)_s * V[s,:],  lse[t,h] = ln sum_s exp(z_s)
 *                 V = kv[:, 0:d_v] (the latent part of the row) unless a separate v is
 *                 given.  An empty S_t gives O = 0, lse = -inf.
 *
 * Conventions
 * -----------
 *   * Every pointer argument is a DEVICE pointer unless stated otherwise; arrays are
 *     row-major with the innermost dimension contiguous.  Strides are in elements and
 *     are documented per argument: ld_scores; ld_q (between the head rows of q), ld_kv
 *     and ld_v (between key rows); and, for the per-sequence caches of decode and
 *     chunks, the sequence strides kc_seq_stride (key rows of the indexer key cache and
 *     its scales), kv_seq_stride and v_seq_stride (elements).  Every other array is
 *     dense.  A row stride must be >= the row's width, and a sequence stride must be
 *     >= rows x row stride (sequences do not overlap); bf16 row and sequence strides must
 *     be multiples of 8 elements (16-byte rows).  Violations return DSA_ERR_INVALID_ARG.
 *     The caller owns every buffer, including the workspace (size it with
 *     dsa_workspace_size); the library allocates nothing and keeps no pointer after a
 *     call returns.
 *   * All work is enqueued on `stream` (0 = the null stream); calls return before the
 *     GPU finishes.  Buffers must stay alive until the stream has passed the work.
 *   * Return value: DSA_OK (0) or a negative dsa_status.  Arguments are validated on
 *     the host before anything is enqueued; a failing call enqueues nothing, except
 *     DSA_ERR_HIP, which reports a launch failure.  dsa_last_error() gives a message
 *     for the calling thread's last failure.  No exception or abort crosses the ABI.
 *   * Device-side preconditions that are not checked: indices in idx are -1 or in
 *     [0, n_k); positions fit the key arrays; no NaN in the inputs.
 *   * dtype codes: DSA_F32 (fp32 everywhere), DSA_FP8_E4M3 (indexer operands are OCP
 *     FP8 E4M3FN codes, one byte each, with fp32 scales), DSA_BF16 (attention operands
 *     and output in bfloat16).
 *   * Supported shapes.  dtype DSA_F32: any H_I <= 64, d_I <= 256, H <= 64,
 *     d_qk <= 256, d_v <= 256, k <= 4096.  FP8 indexer: H_I = 64, d_I = 128.  BF16
 *     attention: H = 128, d_qk = 576, d_v = 512 with V = kv[:, 0:512].  Top-k:
 *     k <= 2048 (fp8/bf16 path) and n_k <= 262144.  Others: DSA_ERR_UNSUPPORTED.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* dsa_stream_t; /* a hipStream_t */

#define DSA_ABI_VERSION 2

/* Tokens per page of the paged caches (dsa_forward_decode_paged, dsa_forward_chunk_paged). */
#define DSA_PAGE_ROWS 64

enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1, /* null pointer, bad dimension, misaligned pointer */
  DSA_ERR_UNSUPPORTED = -2, /* valid request without a kernel (dtype or shape) */
  DSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than dsa_workspace_size() */
  DSA_ERR_HIP = -4          /* the HIP runtime reported an error */
};

enum dsa_dtype { DSA_F32 = 0, DSA_BF16 = 1, DSA_FP8_E4M3 = 2 };

enum dsa_op { DSA_OP_INDEXER = 0, DSA_OP_TOPK = 1, DSA_OP_SPARSE_MLA = 2,
              DSA_OP_PREFILL = 3, DSA_OP_DECODE = 4, DSA_OP_SELECT = 5, DSA_OP_CHUNK = 6,
              DSA_OP_MLA_BWD = 7, DSA_OP_KL_DENSE = 8 };

/* DSA_ABI_VERSION of the loaded library. */
int dsa_abi_version(void);

/* Static description of a status code (never NULL). */
const char* dsa_status_string(int status);

/* Message of the calling thread's most recent failing call ("" if none). */
const char* dsa_last_error(void);

/*
 * Workspace bytes an entry point needs (0 if none).  op is a dsa_op; the other
 * arguments are the ones the entry point takes (unused ones may be 0).  For
 * DSA_OP_PREFILL and DSA_OP_CHUNK pass the attention dtype (DSA_F32 selects the fp32
 * path, whose selection ranks materialised scores); for DSA_OP_SELECT pass the indexer
 * dtype.
 */
size_t dsa_workspace_size(int32_t op, int64_t B, int64_t n_q, int64_t n_k, int32_t H,
                          int32_t d_v, int32_t k, int32_t dtype);

/*
 * dsa_indexer -- lightning-indexer scores for a range of query rows (stage 1).
 *
 *   q_idx   [B, n_q, H_I, d_I]  FP8 codes (DSA_FP8_E4M3) or float (DSA_F32)
 *   q_scale [B, n_q, H_I]       fp32 scale of each query head row
 *   k_idx   [B, n_k, d_I]       FP8 codes or float
 *   k_scale [B, n_k]            fp32 scale of each key row
 *   w       [B, n_q, H_I]       fp32 head weights
 *   q_pos   [B] int32 or NULL   position of query row 0 of sequence b (NULL: all 0);
 *                               row r of sequence b sits at pos = q_pos[b] + r
 *   rows    row_begin .. row_begin + n_rows - 1 of each sequence are scored
 *   scores  [B, n_rows, ld_scores] fp32 output, ld_scores >= n_k: scores[b][i][s] =
 *           I[row_begin+i, s] for s <= pos, -inf for pos < s < n_k; columns >= n_k
 *           are not written.
 * Scores are bit-identical to the ones dsa_forward_prefill / dsa_forward_decode
 * select from.  Needs no workspace.
 */
int dsa_indexer(const void* q_idx, const float* q_scale, const void* k_idx,
                const float* k_scale, const float* w, int64_t B, int64_t n_q, int64_t n_k,
                const int32_t* q_pos, int32_t H_I, int32_t d_I, int32_t dtype,
                int64_t row_begin, int64_t n_rows, float* scores, int64_t ld_scores,
                dsa_stream_t stream);

/*
 * dsa_topk -- fine-grained token selection over materialised scores (stage 2).
 *
 *   scores [B, n_rows, ld_scores] fp32; row i of sequence b belongs to the query at
 *          pos = q_pos[b] + row_begin + i (q_pos NULL: 0) and only columns
 *          s <= min(pos, n_k - 1) are read.
 *   idx    [B, n_rows, k] int32 output: S_t in ascending order, -1 padded.
 * The result depends only on the fp32 values (+0.0 and -0.0 are equal); it is
 * bit-exact against a full sort by (score desc, index asc).  Workspace:
 * dsa_workspace_size(DSA_OP_TOPK, ...) (currently 0; pass NULL, 0).
 */
int dsa_topk(const float* scores, int64_t ld_scores, int64_t B, int64_t n_rows, int64_t n_k,
             const int32_t* q_pos, int64_t row_begin, int32_t k, int32_t* idx, void* ws,
             size_t ws_bytes, dsa_stream_t stream);

/*
 * dsa_sparse_mla -- attention of every query head over its selected keys (stage 3): the
 * core attention runs only over the k kept key-value entries, in MLA's MQA mode where one
 * latent key-value row serves every query head (paperbridge.wiki summary, section
 * DeepSeek Sparse Attention; 53ai.com V3.2-Exp summary, section 创新架构 and Figure 1).
 *
 *   q    [B, n_q, H] rows of d_qk values, ld_q elements apart (ld_q >= d_qk): element
 *        (b, t, h, d) at q[((b * n_q + t) * H + h) * ld_q + d]; bf16 or fp32 (dtype)
 *   kv   [B, n_k] rows of d_qk values, ld_kv apart: the shared key/latent rows (MQA);
 *        (b, s, d) at kv[(b * n_k + s) * ld_kv + d]
 *   v    [B, n_k] rows of d_v values, ld_v apart, or NULL: NULL means V = kv[.., 0:d_v]
 *        (ld_v is then ignored)
 *   idx  [B, n_q, k] int32   selected keys (-1 entries are ignored, anywhere)
 *   out  [B, n_q, H, d_v]    dense output, same dtype as q
 *   lse  [B, n_q, H] fp32 or NULL: natural-log sum-exp of the scaled logits
 * Workspace: dsa_workspace_size(DSA_OP_SPARSE_MLA, B, n_q, n_k, H, d_v, k, dtype).
 */
int dsa_sparse_mla(const void* q, int64_t ld_q, const void* kv, int64_t ld_kv, const void* v,
                   int64_t ld_v, const int32_t* idx, int64_t B, int64_t n_q, int64_t n_k, int32_t H,
                   int32_t d_qk, int32_t d_v, int32_t k, float sm_scale, int32_t dtype, void* out,
                   float* lse, void* ws, size_t ws_bytes, dsa_stream_t stream);

/*
 * dsa_sparse_mla_backward -- gradients of dsa_sparse_mla for the sparse training stage
 * (the main model learns on the sparse pattern: juhe.plus explainer, section
 * 阶段二：Sparse Training; 53ai.com V3.2-Exp summary, section 持续预训练).  With the
 * forward's P[h,s] = exp(sm_scale q_h . kv_s - lse_h) over each row's valid ids:
 *     dP = dO . v_s,  dZ = P (dP - dO_h . O_h),  dq_h = sm_scale sum_s dZ kv_s,
 *     dkv_s += sm_scale sum_h dZ q_h (and sum_h P dO_h on the V values)
 * summed over every query that selected s.
 *
 *   q, kv, v, idx, lse: the forward's inputs and lse; out [B, n_q, H, d_v]: its output
 *          (bf16 path; may be NULL for fp32); d_out [B, n_q, H, d_v]: gradient of out
 *   d_q    [B, n_q, H, d_qk] output, dtype of q
 *   d_kv   [B, n_k, d_qk] fp32 output, zeroed and accumulated by the call (V = kv[:, :d_v]
 *          adds its gradient here); d_v_out [B, n_k, d_v] fp32 for a separate V (fp32
 *          path), else NULL
 * dtype DSA_BF16 (H = 128, d_qk = 576, d_v = 512, V inside kv, k a multiple of 32 up to
 * 2048) or DSA_F32 (small shapes).  Workspace: dsa_workspace_size(DSA_OP_MLA_BWD, B, n_q,
 * n_k, H, d_v, k, dtype) (bf16: the transposed q and dO and the bf16 P and dZ of up to
 * 4096 queries at a time, then for up to 2048 queries at a time the fp32 d_kv
 * contributions of every (query, selected key) pair (k * 576 * 4 bytes per query), those
 * pairs' lists by key and the lists' offsets over the keys of the sequences those queries
 * belong to).  The order in which a key's contributions are summed is not fixed: d_kv is
 * reproducible to rounding, not bit for bit.
 */
int dsa_sparse_mla_backward(const void* q, const void* kv, const void* v, const int32_t* idx,
                            const void* out, const float* lse, const void* d_out, int64_t B,
                            int64_t n_q, int64_t n_k, int32_t H, int32_t d_qk, int32_t d_v,
                            int32_t k, float sm_scale, int32_t dtype, void* d_q, float* d_kv,
                            float* d_v_out, void* ws, size_t ws_bytes, dsa_stream_t stream);

/*
 * dsa_select_prefill -- stages 1 and 2 for one sequence of L tokens (query t at position
 * t).  FP8 path: the L x L score matrix is never stored.  Each row's scores are compared
 * on chip with a threshold set from that row's scores at every 32nd key, and only the keys
 * above it (about 1.7 k per row) are written, to a candidate list whose top-k is the
 * row's selection.  A row whose list cannot decide it (fewer than k keys above the
 * threshold, or more than the list holds: heavy ties, adversarial keys) is selected again
 * by a streaming top-k fused with the indexer.  The result is the full-sort definition in
 * every case.  The workspace holds the per-row sample scores and candidate lists of one
 * chunk of up to 16384 rows at a time (about 1 GiB at L = 131072); for L > 262144 the
 * streaming kernel selects every row and no workspace is needed.  The fp32 path ranks a
 * materialised score matrix held in the workspace.
 *
 *   q_idx [L, H_I, d_I], q_scale [L, H_I], k_idx [L, d_I], k_scale [L], w [L, H_I]
 *   idx   [L, k] int32 output, ascending, -1 padded
 * idx_dtype: DSA_FP8_E4M3 (k <= 2048) or DSA_F32.  Workspace:
 * dsa_workspace_size(DSA_OP_SELECT, 1, L, L, 0, 0, k, idx_dtype).
 */
int dsa_select_prefill(const void* q_idx, const float* q_scale, const void* k_idx,
                       const float* k_scale, const float* w, int64_t L, int32_t H_I, int32_t d_I,
                       int32_t k, int32_t idx_dtype, int32_t* idx, void* ws, size_t ws_bytes,
                       dsa_stream_t stream);

/*
 * dsa_forward_prefill -- the whole layer for one sequence of L tokens, query t at
 * position t: the lightning indexer scores every preceding token, the top-k of those
 * scores are kept, and the attention runs over the kept keys only (53ai.com V3.2-Exp
 * summary, section 创新架构 and Figure 1; juhe.plus explainer, sections 第一步：Lightning
 * Indexer and 第二步：Fine-grained Token Selection).  The selection is
 * dsa_select_prefill's (the L x L score matrix is never stored); the attention is
 * dsa_sparse_mla's.
 *
 *   q_idx [L, H_I, d_I], q_scale [L, H_I], k_idx [L, d_I], k_scale [L], w [L, H_I] (dense)
 *   q [L, H] rows of d_qk values ld_q apart; kv [L] rows of d_qk values ld_kv apart;
 *   v [L] rows of d_v values ld_v apart, or NULL (V = kv[:, 0:d_v], ld_v ignored)
 *   idx [L, k] int32 (output: the selection), out [L, H, d_v], lse [L, H] or NULL
 * idx_dtype: DSA_FP8_E4M3 or DSA_F32; attn_dtype: DSA_BF16 or DSA_F32.
 * Workspace: dsa_workspace_size(DSA_OP_PREFILL, 1, L, L, H, d_v, k, attn_dtype).
 * Streams: with the FP8 selection in more than one chunk of rows (L > 16384), the attention
 * of each finished chunk runs on a second stream of the library (default priority, one per
 * host thread and device, created on the first such call and never released),
 * fenced by events; `stream` waits for it before the call's work ends, so every output is
 * complete when the work enqueued on `stream` is.  Results are bit-identical to selecting
 * first and attending after.
 */
int dsa_forward_prefill(const void* q_idx, const float* q_scale, const void* k_idx,
                        const float* k_scale, const float* w, const void* q, int64_t ld_q,
                        const void* kv, int64_t ld_kv, const void* v, int64_t ld_v, int64_t L,
                        int32_t H_I, int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v, int32_t k,
                        float sm_scale, int32_t idx_dtype, int32_t attn_dtype, int32_t* idx,
                        void* out, float* lse, void* ws, size_t ws_bytes, dsa_stream_t stream);

/*
 * dsa_forward_decode -- the whole layer for B sequences with one new token each.  In the
 * decode stage too the indexer scans every previous token and the attention runs over the
 * top-k only, which is what lowers the per-token decode cost (yunpan.plus article, section
 * 1.1 DSA; 53ai.com V3.2-Exp summary, section 创新架构).
 * Sequence b holds ctx_len[b] cached rows (1 <= ctx_len[b] <= n_k_max, device int32);
 * its query sits at position ctx_len[b] - 1 (its own row is already in the caches)
 * and sees every cached row.
 *
 *   q_idx [B, H_I, d_I], q_scale [B, H_I], w [B, H_I] (dense)
 *   k_cache        codes of sequence b, row s: k_cache + (b * kc_seq_stride + s) * d_I
 *                  (rows of d_I bytes; kc_seq_stride >= n_k_max rows)
 *   k_cache_scale  fp32, sequence b row s at k_cache_scale[b * kc_seq_stride + s]
 *   q              [B, H] rows of d_qk values, ld_q elements apart
 *   kv_cache       sequence b row s at kv_cache + b * kv_seq_stride + s * ld_kv (elements;
 *                  kv_seq_stride >= n_k_max * ld_kv)
 *   v_cache        likewise with ld_v / v_seq_stride, or NULL (V = kv[.., 0:d_v]; ld_v and
 *                  v_seq_stride ignored)
 *   idx [B, k] int32 (output), out [B, H, d_v] (dense), lse [B, H] or NULL
 * Workspace: dsa_workspace_size(DSA_OP_DECODE, B, 1, n_k_max, H, d_v, k, attn_dtype).
 */
int dsa_forward_decode(int64_t B, const int32_t* ctx_len, int64_t n_k_max, const void* q_idx,
                       const float* q_scale, const float* w, const void* k_cache,
                       const float* k_cache_scale, int64_t kc_seq_stride, const void* q,
                       int64_t ld_q, const void* kv_cache, int64_t ld_kv, int64_t kv_seq_stride,
                       const void* v_cache, int64_t ld_v, int64_t v_seq_stride, int32_t H_I,
                       int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v, int32_t k,
                       float sm_scale, int32_t idx_dtype, int32_t attn_dtype, int32_t* idx,
                       void* out, float* lse, void* ws, size_t ws_bytes, dsa_stream_t stream);

/*
 * dsa_forward_decode_paged -- dsa_forward_decode over paged caches: the same selection and
 * attention (and bit-identical results) with the rows of every cache stored in fixed pages
 * of a shared pool instead of one contiguous range per sequence, the layout of serving
 * systems that grow sequences page by page (the serving form of the decode stage: yunpan.plus
 * article, section 1.1 DSA).
 * A page holds DSA_PAGE_ROWS consecutive tokens of one sequence.  Token s of sequence b lives
 * in pool page p = block_table[b * bt_stride + s / DSA_PAGE_ROWS], row
 * p * DSA_PAGE_ROWS + s % DSA_PAGE_ROWS of each pool:
 *   k_pool         [n_pages * DSA_PAGE_ROWS, d_I] FP8 codes (16-byte aligned)
 *   k_pool_scale   [n_pages * DSA_PAGE_ROWS] fp32
 *   kv_pool        [n_pages * DSA_PAGE_ROWS] rows of d_qk bf16 values, ld_kv apart; V = the
 *                  first d_v values of each row
 *   block_table    device int32, bt_stride >= ceil(n_k_max / DSA_PAGE_ROWS) entries per
 *                  sequence.  Entries of pages past a sequence's ctx_len[b] tokens may be read
 *                  (by the tails of key tiles) but their rows are never used, and entries
 *                  outside [0, n_pages) are clamped into the pool, so no table makes a kernel
 *                  read outside the pools (a wrong one gives wrong results).
 * q_idx, q_scale, w, q, ctx_len, idx, out, lse as dsa_forward_decode.  FP8 indexer and bf16
 * attention only (DSA_ERR_UNSUPPORTED otherwise).
 * Workspace: dsa_workspace_size(DSA_OP_DECODE, B, 1, n_k_max, H, d_v, k, attn_dtype).
 */
int dsa_forward_decode_paged(int64_t B, const int32_t* ctx_len, int64_t n_k_max, const void* q_idx,
                             const float* q_scale, const float* w, const void* k_pool,
                             const float* k_pool_scale, const void* q, int64_t ld_q,
                             const void* kv_pool, int64_t ld_kv, const int32_t* block_table,
                             int64_t bt_stride, int64_t n_pages, int32_t H_I, int32_t d_I, int32_t H,
                             int32_t d_qk, int32_t d_v, int32_t k, float sm_scale, int32_t idx_dtype,
                             int32_t attn_dtype, int32_t* idx, void* out, float* lse, void* ws,
                             size_t ws_bytes, dsa_stream_t stream);

/*
 * dsa_forward_chunk -- the whole layer for a chunk of n_q new tokens in each of B
 * sequences (chunked prefill; multi-token decode): the chunk's queries attend to the
 * sequence's cached rows, which already hold the chunk's own rows (dsa_kcache_append
 * writes the indexer keys).  The decode path is the n_q = 1 case; dsa_forward_prefill
 * is B = 1, q_pos = 0, n_q = n_k_max.  DSA lowers the per-token cost of both the
 * prefill and the decode stage (yunpan.plus article, section 1.1 DSA, and its
 * inference-cost figure); each query keeps its own top-k of the keys before it (juhe.plus
 * explainer, section 第二步：Fine-grained Token Selection).
 *
 * Row i of sequence b is the query at position p = q_pos[b] + i (q_pos: [B] int32,
 * device).  It sees cached rows 0 .. min(p, n_k_max - 1); a row with p < 0 sees none
 * (idx all -1, out 0, lse -inf).  Rows whose position leaves at most k visible keys keep
 * all of them.
 *
 *   q_idx [B, n_q, H_I, d_I], q_scale [B, n_q, H_I], w [B, n_q, H_I] (dense)
 *   k_cache, k_cache_scale, kc_seq_stride; kv_cache, ld_kv, kv_seq_stride; v_cache, ld_v,
 *   v_seq_stride: the per-sequence caches, laid out as for dsa_forward_decode
 *   q [B, n_q, H] rows of d_qk values, ld_q elements apart
 *   idx [B, n_q, k] int32 (output: S_t ascending, -1 padded), out [B, n_q, H, d_v] (dense),
 *   lse [B, n_q, H] or NULL
 * idx_dtype / attn_dtype: DSA_FP8_E4M3 with DSA_BF16 (dsa_select_prefill's threshold
 * filter per sequence: no score matrix, k <= 2048, n_k_max < 2^25; the workspace holds
 * key-sample scores and candidate lists for up to 16384 rows at a time), or DSA_F32 with
 * DSA_F32 (materialised scores in the workspace, n_q <= 65535).  Selection and
 * attention of a row do not depend on the other rows of the call: a prefill cut into
 * chunks returns what the one-shot prefill returns, bit for bit.
 * Workspace: dsa_workspace_size(DSA_OP_CHUNK, B, n_q, n_k_max, H, d_v, k, attn_dtype).
 * Buffers are device memory owned by the caller.
 */
int dsa_forward_chunk(int64_t B, int64_t n_q, const int32_t* q_pos, int64_t n_k_max,
                      const void* q_idx, const float* q_scale, const float* w,
                      const void* k_cache, const float* k_cache_scale, int64_t kc_seq_stride,
                      const void* q, int64_t ld_q, const void* kv_cache, int64_t ld_kv,
                      int64_t kv_seq_stride, const void* v_cache, int64_t ld_v,
                      int64_t v_seq_stride, int32_t H_I, int32_t d_I, int32_t H, int32_t d_qk,
                      int32_t d_v, int32_t k, float sm_scale, int32_t idx_dtype,
                      int32_t attn_dtype, int32_t* idx, void* out, float* lse, void* ws,
                      size_t ws_bytes, dsa_stream_t stream);

/*
 * dsa_forward_chunk_paged -- dsa_forward_chunk over paged caches (chunked prefill into a
 * paged cache): the same selection and attention, bit-identical results, with every cache
 * row found through the block table as in dsa_forward_decode_paged (pools of n_pages pages
 * of DSA_PAGE_ROWS tokens: k_pool codes, k_pool_scale, kv_pool rows ld_kv apart with V = the
 * first d_v values; block_table with bt_stride >= ceil(n_k_max / DSA_PAGE_ROWS) entries per
 * sequence, entries outside [0, n_pages) clamped into the pools).  The chunk's own rows must
 * already be in the pools.  q_pos, q_idx, q_scale, w, q, idx, out, lse as dsa_forward_chunk.
 * FP8 indexer and bf16 attention only.
 * Workspace: dsa_workspace_size(DSA_OP_CHUNK, B, n_q, n_k_max, H, d_v, k, attn_dtype).
 */
int dsa_forward_chunk_paged(int64_t B, int64_t n_q, const int32_t* q_pos, int64_t n_k_max,
                            const void* q_idx, const float* q_scale, const float* w,
                            const void* k_pool, const float* k_pool_scale, const void* q,
                            int64_t ld_q, const void* kv_pool, int64_t ld_kv,
                            const int32_t* block_table, int64_t bt_stride, int64_t n_pages,
                            int32_t H_I, int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v, int32_t k,
                            float sm_scale, int32_t idx_dtype, int32_t attn_dtype, int32_t* idx,
                            void* out, float* lse, void* ws, size_t ws_bytes, dsa_stream_t stream);

/*
 * dsa_indexer_scores_at -- lightning-indexer scores of the listed keys only (the scores the
 * selection ranked, for the indexer loss below).
 *
 *   q_idx, q_scale, k_idx, k_scale, w: as for dsa_indexer (B sequences, n_q rows, n_k keys)
 *   idx     [B, n_q, k] int32 device: key ids per row; ids outside [0, n_k) score -inf
 *   scores  [B, n_q, k] fp32 output: scores[b][i][j] = I[i, idx[b][i][j]]
 * No causal mask is applied: the ids say which keys to score.  The value of every score
 * is bit-identical to the one dsa_indexer writes for the same (row, key).  FP8 or fp32
 * (dtype); no workspace.
 */
int dsa_indexer_scores_at(const void* q_idx, const float* q_scale, const void* k_idx,
                          const float* k_scale, const float* w, const int32_t* idx, int64_t B,
                          int64_t n_q, int64_t n_k, int32_t H_I, int32_t d_I, int32_t k,
                          int32_t dtype, float* scores, dsa_stream_t stream);

/*
 * dsa_indexer_kl -- forward of the indexer's KL-alignment loss over each query's selected
 * keys (the sparse training stage: juhe.plus explainer, section 阶段二：Sparse Training;
 * 53ai.com V3.2-Exp summary, section 持续预训练).  For query row t with key set S_t (its
 * valid ids):
 *     p_t(s)  = (1/H) sum_h exp(sm_scale q_h . kv_s - lse_h)     (the heads' attention
 *               probabilities over S_t, summed and L1-normalised)
 *     KL_t    = sum_{s in S_t} p_t(s) (ln p_t(s) - ln softmax_{S_t}(idx_scores)(s))
 *
 *   q [B, n_q, H, d_qk], kv [B, n_k, d_qk]   attention operands (dtype DSA_BF16 or DSA_F32)
 *   idx        [B, n_q, k] int32: S_t (ids outside [0, n_k) are ignored)
 *   lse        [B, n_q, H] fp32: log-sum-exp of the scaled logits over S_t, as
 *              dsa_sparse_mla / dsa_forward_* return it
 *   idx_scores [B, n_q, k] fp32: index scores of the slots (dsa_indexer_scores_at)
 *   kl         [B, n_q] fp32 output (0 for a row with no valid id); the loss of a batch
 *              is their sum (or mean)
 *   p_out      [B, n_q, k] fp32 or NULL: p_t of each slot (0 for ignored slots)
 * bf16 path: H = 128, d_qk = 576, k a multiple of 32 up to 2048; fp32 path: H <= 64,
 * d_qk <= 256.  No workspace.
 */
int dsa_indexer_kl(const void* q, const void* kv, const int32_t* idx, const float* lse,
                   const float* idx_scores, int64_t B, int64_t n_q, int64_t n_k, int32_t H,
                   int32_t d_qk, int32_t k, float sm_scale, int32_t dtype, float* kl,
                   float* p_out, dsa_stream_t stream);

/*
 * dsa_indexer_kl_dense -- forward of the indexer's KL-alignment loss in the dense warm-up
 * stage, where the indexer learns to match the main attention's distribution over every
 * preceding token while the rest of the model is frozen (juhe.plus explainer, section
 * 阶段一：Dense Warm-up; 53ai.com V3.2-Exp summary, section 持续预训练).  For query row t of
 * sequence b at position pos = (q_pos ? q_pos[b] : 0) + t, over its keys s = 0 .. n-1,
 * n = min(pos + 1, n_k):
 *     lse_h   = ln sum_s exp(sm_scale q_h . kv_s)                 (dense attention, head h)
 *     p_t(s)  = (1/H) sum_h exp(sm_scale q_h . kv_s - lse_h)      (heads summed, L1-normalised)
 *     KL_t    = sum_s p_t(s) (ln p_t(s) - ln softmax_s(I[t, :n])(s))
 * with I the lightning-indexer scores (the same scores dsa_indexer writes, bit for bit).
 * Nothing of size L x L is stored: the workspace holds the score rows of a chunk of query
 * rows at a time.
 *
 *   q_idx, q_scale, k_idx, k_scale, w: indexer operands as for dsa_indexer (B sequences,
 *                n_q query rows, n_k keys; idx_dtype DSA_FP8_E4M3 or DSA_F32)
 *   q [B, n_q, H, d_qk], kv [B, n_k, d_qk]: attention operands (attn_dtype DSA_BF16 with
 *                H = 128, d_qk = 576; or DSA_F32 with H <= 64, d_qk <= 256, n_k <= 4096), dense
 *   q_pos [B] int32 or NULL (device)
 *   kl  [B, n_q] fp32 output (0 for a row that sees no key)
 *   lse [B, n_q, H] fp32 output or NULL: the dense attention's lse (-inf for such a row)
 * Workspace: dsa_workspace_size(DSA_OP_KL_DENSE, B, n_q, n_k, H, 0, 1, attn_dtype) (the score
 * rows of up to 2^28 / (B n_k) query rows per pass, at least one).
 */
int dsa_indexer_kl_dense(const void* q_idx, const float* q_scale, const void* k_idx,
                         const float* k_scale, const float* w, const void* q, const void* kv,
                         int64_t B, int64_t n_q, int64_t n_k, const int32_t* q_pos, int32_t H_I,
                         int32_t d_I, int32_t H, int32_t d_qk, float sm_scale, int32_t idx_dtype,
                         int32_t attn_dtype, float* kl, float* lse, void* ws, size_t ws_bytes,
                         dsa_stream_t stream);

/*
 * dsa_forward_decode_noalloc -- dsa_forward_decode without a workspace argument, for
 * callers that cannot allocate device memory: code under stream capture, tight serving
 * loops, harnesses that forbid allocation.  The arguments and results are those of
 * dsa_forward_decode (minus ws / ws_bytes), computed by the same kernels.
 *
 * Its scratch is a fixed 128 MiB array of the library in device memory, held on every GPU
 * the library runs on until the process ends (the 64 x 131072-token decode workload needs
 * about 110 MB).  A shape whose dsa_workspace_size(DSA_OP_DECODE, ...) exceeds 128 MiB
 * returns DSA_ERR_UNSUPPORTED before anything is enqueued.  Nothing is allocated, by the
 * library or by any routine it calls.  All calls on one GPU share that GPU's array: calls
 * that overlap on one GPU (concurrent streams, several threads) race and must be ordered
 * by the caller.  The array keeps the previous call's contents; the call needs nothing
 * zeroed.
 */
int dsa_forward_decode_noalloc(int64_t B, const int32_t* ctx_len, int64_t n_k_max,
                               const void* q_idx, const float* q_scale, const float* w,
                               const void* k_cache, const float* k_cache_scale,
                               int64_t kc_seq_stride, const void* q, int64_t ld_q,
                               const void* kv_cache, int64_t ld_kv, int64_t kv_seq_stride,
                               const void* v_cache, int64_t ld_v, int64_t v_seq_stride,
                               int32_t H_I, int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v,
                               int32_t k, float sm_scale, int32_t idx_dtype, int32_t attn_dtype,
                               int32_t* idx, void* out, float* lse, dsa_stream_t stream);

/*
 * dsa_fp8_quantize_rows -- FP8 E4M3FN quantisation of the indexer operands, the step
 * before the lightning indexer (the indexer runs in FP8: 53ai.com V3.2-Exp summary,
 * section 创新架构; juhe.plus explainer, section 第一步：Lightning Indexer).  Per row of
 * `width` values (a key: d_I values; a query token: its H_I x d_I values):
 *     scale = amax / 448 in fp32, correctly rounded (1 when the row is all zero);
 *     code  = the E4M3FN value nearest to x / scale (that quotient in fp32, correctly
 *             rounded), ties to the even mantissa, saturating at +-448.
 *
 *   x      [n_rows, ld_x] input (x_dtype DSA_BF16 or DSA_F32); row r = x + r * ld_x
 *   codes  [n_rows, ld_codes] uint8 output (the first `width` bytes of each row)
 *   scale  output: row r's scale is written `repeat` times, at scale[r * scale_stride + j],
 *          j < repeat (a query token: repeat = H_I, scale_stride = H_I, which fills the
 *          indexer's q_scale [L, H_I]; a key: repeat = scale_stride = 1)
 * Buffers are device memory owned by the caller; nothing is allocated.  Invalid shapes
 * or null pointers return DSA_ERR_INVALID_ARG before anything is enqueued.
 */
int dsa_fp8_quantize_rows(const void* x, int32_t x_dtype, int64_t n_rows, int64_t width,
                          int64_t ld_x, uint8_t* codes, int64_t ld_codes, float* scale,
                          int64_t scale_stride, int32_t repeat, dsa_stream_t stream);

/*
 * dsa_kcache_append -- indexer key-cache append for decode and chunked prefill: the
 * n_new new key rows of each of the B sequences are quantised as by
 * dsa_fp8_quantize_rows (one scale per key) and written into the FP8 key cache at rows
 * pos[b] .. pos[b] + n_new - 1 of sequence b.
 *
 *   k_new        [B, n_new, d_I] (dtype DSA_BF16 or DSA_F32)
 *   pos          [B] int32, device: first cache row of each sequence's new keys; rows at
 *                or past n_k_max (or below 0) are skipped on the device
 *   k_cache      uint8 codes, sequence b row s at k_cache + (b * kc_seq_stride + s) * d_I;
 *   k_cache_scale fp32, sequence b row s at k_cache_scale[b * kc_seq_stride + s]
 *                (kc_seq_stride >= n_k_max rows; updated in place)
 * Buffers are device memory owned by the caller; nothing is allocated.
 */
int dsa_kcache_append(const void* k_new, int32_t dtype, int64_t B, int64_t n_new, int32_t d_I,
                      const int32_t* pos, int64_t n_k_max, int64_t kc_seq_stride,
                      uint8_t* k_cache, float* k_cache_scale, dsa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H_ */
