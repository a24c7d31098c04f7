// Indexer KL-alignment loss, forward, over each query's selected keys; and the index scores
// of given keys.
//
// The indexer is trained to match the main attention's distribution with a KL-divergence
// loss, first densely with the main model frozen, then on the sparse pattern together with
// the model (juhe.plus explainer, sections 阶段一：Dense Warm-up and 阶段二：Sparse Training;
// 53ai.com V3.2-Exp summary, section 持续预训练; wiki-for-amaranth report, section DeepSeek
// Sparse Attention (DSA)).  The pages give no formula; the plain reading, for query t over
// its key set S_t:
//     p_t(s) = (1/H) sum_h softmax_{s in S_t}(sm_scale q_h . kv_s)   (heads summed, then
//                                                                     L1-normalised)
//     q_t(s) = softmax_{s in S_t}(I[t, s])
//     KL_t   = sum_{s in S_t} p_t(s) (ln p_t(s) - ln q_t(s))
// Here S_t is the selection (the sparse stage).  The attention's per-head log-sum-exp over
// S_t comes from the forward (dsa_sparse_mla's lse), so p needs one pass over the keys.
//
// bf16 kernel (H = 128, d_qk = 576), one block of 4 waves per query, two blocks per CU:
//   * rows are gathered into LDS exactly as the sparse attention gathers them (the same
//     layout and loads), two chunk buffers: chunk c+1 is in flight while chunk c is used;
//   * wave w forms S = Q K^T for heads 32w .. 32w+31 (36 MFMAs of 32x32x16 per chunk), so
//     each lane holds 16 heads of one key: exp2(S - lse) summed over them and with lane
//     l^32 gives the wave's 32-head sum for key l%32;
//   * wave 0 adds the four waves' sums of the previous chunk and accumulates the row's KL.
#include "dsa_kernels.h"
#include "indexer_tile.h"
#include "mla_gather.h"

namespace dsa {

// ---------------------------------------------------------------------------------------
// index scores at given keys
// ---------------------------------------------------------------------------------------

// FP8: one wave per query row (4 rows per block), the row's k slots 64 at a time.  The key
// rows are read straight from global memory in the B-operand layout, and the arithmetic is
// the indexer's (indexer_tile.h), so every score equals the one dsa_indexer writes for
// that key, bit for bit.
__global__ __launch_bounds__(256) void idx_scores_at_fp8(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, const float* __restrict__ w, const int32_t* __restrict__ idx, int64_t n_q,
    int64_t n_k, int k, float* __restrict__ out) {
  const int b = blockIdx.y;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + wv;
  if (i >= n_q) return;  // whole waves leave; the block never synchronises
  const int64_t qrow = (int64_t)b * n_q + i;
  IdxRow Q;
  load_idx_row(Q, q8 + qrow * IDX_HEADS * IDX_DIM, qs + qrow * IDX_HEADS, w + qrow * IDX_HEADS);
  const uint8_t* kb = k8 + (int64_t)b * n_k * IDX_DIM;
  const float* ksb = ks + (int64_t)b * n_k;
  const int32_t* irow = idx + qrow * k;
  float* orow = out + qrow * k;
  for (int j0 = 0; j0 < k; j0 += KEY_TILE) {
    const int j = j0 + lane;
    const int32_t id = j < k ? irow[j] : -1;
    const bool valid = id >= 0 && (int64_t)id < n_k;
    const int32_t sid = valid ? id : 0;
    v8i bf[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      // fragment f holds slots j0 + 16f .. +15: lane l supplies bytes 32(l/16) .. +31 of
      // slot 16f + l%16's key row
      const int32_t kid = __shfl(sid, 16 * f + (lane & 15), WAVE);
      const v4i* p = reinterpret_cast<const v4i*>(kb + (int64_t)kid * IDX_DIM + 32 * (lane >> 4));
      const v4i lo = p[0], hi = p[1];
      bf[f] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    const float s = score_tile64(Q, bf, ksb[sid]);
    if (j < k) orow[j] = valid ? s : -INFINITY;
  }
}

// fp32: one thread per (row, slot), the fp32 indexer's arithmetic in the same order.
__global__ __launch_bounds__(256) void idx_scores_at_f32(
    const float* __restrict__ q, const float* __restrict__ qs, const float* __restrict__ kk,
    const float* __restrict__ ks, const float* __restrict__ w, const int32_t* __restrict__ idx, int64_t n_q,
    int64_t n_k, int H_I, int d_I, int k, float* __restrict__ out) {
  const int b = blockIdx.z;
  const int64_t i = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= k) return;
  const int64_t qrow = (int64_t)b * n_q + i;
  const int32_t id = idx[qrow * k + j];
  float* o = out + qrow * k + j;
  if (id < 0 || (int64_t)id >= n_k) {
    *o = -INFINITY;
    return;
  }
  const float* qr = q + qrow * H_I * d_I;
  const float* kr = kk + ((int64_t)b * n_k + id) * d_I;
  float acc = 0.f;
  for (int h = 0; h < H_I; ++h) {
    float dot = 0.f;
    for (int d = 0; d < d_I; ++d) dot = __fmaf_rn(qr[h * d_I + d], kr[d], dot);
    const float c = __fmul_rn(w[qrow * H_I + h], qs[qrow * H_I + h]);
    acc = __fmaf_rn(c, fmaxf(dot, 0.f), acc);
  }
  *o = __fmul_rn(acc, ks[(int64_t)b * n_k + id]);
}

hipError_t launch_indexer_scores_at(const ScoresAtArgs& a, hipStream_t st) {
  if (a.dtype == DSA_F32) {
    dim3 grid((unsigned)((a.k + 255) / 256), (unsigned)a.n_q, (unsigned)a.B);
    hipLaunchKernelGGL(idx_scores_at_f32, grid, dim3(256), 0, st, (const float*)a.q_idx, a.q_scale,
                       (const float*)a.k_idx, a.k_scale, a.w, a.idx, a.n_q, a.n_k, a.H_I, a.d_I, a.k, a.scores);
  } else {
    dim3 grid((unsigned)((a.n_q + 3) / 4), (unsigned)a.B);
    hipLaunchKernelGGL(idx_scores_at_fp8, grid, dim3(256), 0, st, (const uint8_t*)a.q_idx, a.q_scale,
                       (const uint8_t*)a.k_idx, a.k_scale, a.w, a.idx, a.n_q, a.n_k, a.k, a.scores);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// KL loss, bf16 attention operands
// ---------------------------------------------------------------------------------------
constexpr int KL_WAVES = 4;

// The ids one wave needs to gather its part of a chunk (see gather_load): lane l reads the
// id of chunk row 8w + l%8 (latent loads take lanes 0..7 as scalars) and of row 8w + l/8
// (its rope load).
struct KlIds {
  int32_t lat, rope;
};
__device__ __forceinline__ KlIds kl_ids(const int32_t* __restrict__ irow, int c, int wv, int lane) {
  const int32_t* cid = irow + c * KC + 8 * wv;
  return KlIds{cid[lane & 7], cid[lane >> 3]};
}
__device__ __forceinline__ void kl_gather(uint32_t buf, const uint16_t* __restrict__ kvb, const KlIds& id,
                                          uint32_t n_k, int wv, int lane) {
  ChunkIds ci;
  ci.a = int4{__builtin_amdgcn_readlane(id.lat, 0), __builtin_amdgcn_readlane(id.lat, 1),
              __builtin_amdgcn_readlane(id.lat, 2), __builtin_amdgcn_readlane(id.lat, 3)};
  ci.b = int4{__builtin_amdgcn_readlane(id.lat, 4), __builtin_amdgcn_readlane(id.lat, 5),
              __builtin_amdgcn_readlane(id.lat, 6), __builtin_amdgcn_readlane(id.lat, 7)};
  ci.rope = id.rope;
#pragma unroll
  for (int j = 0; j < LOADS_PER_CHUNK; ++j) gather_load(j, ci, buf, kvb, n_k, wv, lane);
}

// grid.x = n_q, grid.y = B.  Chunk loop (c = 0 .. n-1, n = chunks up to the last valid id):
//   top: this wave's loads of chunk c (and everything issued before them) complete, then a
//   barrier: every wave's part of chunk c is in LDS, every wave is done with chunk c-1
//   (its buffer is free) and has published its head sums of chunk c-1;
//   then chunk c+1's loads go out, the ids of chunk c+2 and (wave 0) the ids and index
//   scores of chunk c are fetched into registers (used one step later, after the next
//   top wait), the logits and head sums of chunk c are formed, and wave 0 accumulates
//   chunk c-1.
__global__ __launch_bounds__(KL_WAVES * 64, 2) void indexer_kl_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const float* __restrict__ lse, const float* __restrict__ isc, int64_t n_q, int64_t n_k, int k,
    float scale_log2, float* __restrict__ kl, float* __restrict__ p_out) {
  __shared__ __align__(16) uint8_t buf0[CHUNK_BYTES];
  __shared__ __align__(16) uint8_t buf1[CHUNK_BYTES];
  __shared__ float xs[2][KL_WAVES][KC];  // per-wave head sums of a chunk's 32 keys

  const int tid = threadIdx.x, l = tid & 63, g = l >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.y;
  const int64_t qrow = (int64_t)b * n_q + blockIdx.x;
  const int32_t* irow = idx + qrow * k;
  const float* srow = isc + qrow * k;
  const uint16_t* kvb = kv + (int64_t)b * n_k * MDQK;
  const uint32_t nk = (uint32_t)min(n_k, (int64_t)INT32_MAX);

  // The row's ids (and, in wave 0, its index scores), 4 slots per lane per step, all loads
  // issued before any is used (k is a multiple of 32, at most MAX_K): the last valid slot
  // bounds the chunk loop, and wave 0 forms the log2-sum-exp of the valid slots' scores.
  constexpr int SCAN = MAX_K / (4 * WAVE);
  int4 iv[SCAN];
  float4 sv[SCAN];
#pragma unroll
  for (int it = 0; it < SCAN; ++it) {  // unconditional loads (clamped in bounds), then masked
    const int j = min(4 * l + 4 * WAVE * it, k - 4);
    iv[it] = *reinterpret_cast<const int4*>(irow + j);
    sv[it] = *reinterpret_cast<const float4*>(srow + j);
  }
#pragma unroll
  for (int it = 0; it < SCAN; ++it)
    if (4 * l + 4 * WAVE * it >= k) iv[it] = int4{-1, -1, -1, -1};
  auto ok = [&](int32_t id) { return id >= 0 && (int64_t)id < n_k; };
  int last = -1;
  float m = -INFINITY;
#pragma unroll
  for (int it = 0; it < SCAN; ++it) {
    const int j = 4 * l + 4 * WAVE * it;
    if (ok(iv[it].x)) last = j;
    if (ok(iv[it].y)) last = j + 1;
    if (ok(iv[it].z)) last = j + 2;
    if (ok(iv[it].w)) last = j + 3;
    if (wv == 0) {
      if (ok(iv[it].x)) m = fmaxf(m, sv[it].x * LOG2E);
      if (ok(iv[it].y)) m = fmaxf(m, sv[it].y * LOG2E);
      if (ok(iv[it].z)) m = fmaxf(m, sv[it].z * LOG2E);
      if (ok(iv[it].w)) m = fmaxf(m, sv[it].w * LOG2E);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) last = max(last, __shfl_xor(last, off, WAVE));
  last = __builtin_amdgcn_readfirstlane(last);
  const int n = (last + KC) / KC;  // 0 when no slot is valid
  float lsei2 = -INFINITY;
  if (wv == 0) {
    m = wave_max(m);
    if (m > -INFINITY) {
      float sum = 0.f;
#pragma unroll
      for (int it = 0; it < SCAN; ++it) {
        if (ok(iv[it].x)) sum += exp2f(sv[it].x * LOG2E - m);
        if (ok(iv[it].y)) sum += exp2f(sv[it].y * LOG2E - m);
        if (ok(iv[it].z)) sum += exp2f(sv[it].z * LOG2E - m);
        if (ok(iv[it].w)) sum += exp2f(sv[it].w * LOG2E - m);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, WAVE);
      lsei2 = m + log2f(sum);
    }
  }
  if (n == 0) {
    if (wv == 0) {
      if (l == 0) kl[qrow] = 0.f;
      if (p_out)
        for (int j = l; j < k; j += WAVE) p_out[qrow * k + j] = 0.f;
    }
    return;  // uniform over the block
  }

  // A operands of S = Q K^T: head 32w + l%32, values 16ds + 8g .. +7
  v8bf Qa[D_STEPS];
  {
    const uint16_t* qh = q + (qrow * MH + 32 * wv + (l & 31)) * MDQK + 8 * g;
#pragma unroll
    for (int ds = 0; ds < D_STEPS; ++ds) Qa[ds] = *reinterpret_cast<const v8bf*>(qh + 16 * ds);
#pragma unroll
    for (int ds = 0; ds < D_STEPS; ++ds) asm volatile("" : "+v"(Qa[ds]));
  }
  // lse (log2 units) of the heads of this lane's 16 logits: row 8(r/4) + 4g + r%4
  float L2[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) L2[r] = lse[qrow * MH + 32 * wv + 8 * (r >> 2) + 4 * g + (r & 3)] * LOG2E;

  kl_gather(lds_addr(buf0), kvb, kl_ids(irow, 0, wv, l), nk, wv, l);
  KlIds nxt = kl_ids(irow, n > 1 ? 1 : 0, wv, l);
  float acc = 0.f;          // wave 0: this lane's share of the row's KL
  int32_t a_id = -1;        // wave 0: id and index score of slot 32(c-1) + l%32
  float a_s = 0.f;

  for (int c = 0; c < n; ++c) {
    VMCNT(0);
    block_barrier();
    if (c + 1 < n) kl_gather(lds_addr((c & 1) ? buf0 : buf1), kvb, nxt, nk, wv, l);
    if (c + 2 < n) nxt = kl_ids(irow, c + 2, wv, l);
    int32_t c_id = -1;
    float c_s = 0.f;
    if (wv == 0) {
      c_id = irow[c * KC + (l & 31)];
      c_s = srow[c * KC + (l & 31)];
    }
    // logits and head sums of chunk c
    const KOff ko = k_offsets();
    v16f S = {};
    const uint8_t* cur = (c & 1) ? buf1 : buf0;
#pragma unroll
    for (int ds = 0; ds < D_STEPS; ++ds) S = mfma_bf16_32x32x16(Qa[ds], k_frag(cur, k_off(ko, ds)), S);
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ps += __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], scale_log2, -L2[r]));
    ps += xor32(ps);
    if (l < KC) xs[c & 1][wv][l] = ps;
    // wave 0: chunk c-1, whose sums every wave published before this step's barrier
    if (wv == 0 && c > 0) {
      const float* x = xs[(c - 1) & 1][0];
      const float p = (x[l & 31] + x[KC + (l & 31)] + x[2 * KC + (l & 31)] + x[3 * KC + (l & 31)]) * (1.f / MH);
      const bool valid = a_id >= 0 && (int64_t)a_id < n_k;
      const float pv = valid ? p : 0.f;
      if (l < KC && pv > 0.f) acc += pv * ((log2f(pv) - (a_s * LOG2E - lsei2)) * LN2);
      if (p_out && l < KC) p_out[qrow * k + (c - 1) * KC + l] = pv;
    }
    a_id = c_id;
    a_s = c_s;
  }
  VMCNT(0);
  block_barrier();
  if (wv == 0) {
    const float* x = xs[(n - 1) & 1][0];
    const float p = (x[l & 31] + x[KC + (l & 31)] + x[2 * KC + (l & 31)] + x[3 * KC + (l & 31)]) * (1.f / MH);
    const bool valid = a_id >= 0 && (int64_t)a_id < n_k;
    const float pv = valid ? p : 0.f;
    if (l < KC && pv > 0.f) acc += pv * ((log2f(pv) - (a_s * LOG2E - lsei2)) * LN2);
    if (p_out) {
      if (l < KC) p_out[qrow * k + (n - 1) * KC + l] = pv;
      for (int j = n * KC + l; j < k; j += WAVE) p_out[qrow * k + j] = 0.f;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, WAVE);
    if (l == 0) kl[qrow] = acc;
  }
}

// ---------------------------------------------------------------------------------------
// KL loss, fp32 operands (small shapes): one block per query, one thread per slot
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o = __shfl_xor(v, off, WAVE);
    v = is_max ? fmaxf(v, o) : v + o;
  }
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < 4; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

__global__ __launch_bounds__(256) void indexer_kl_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kv, const int32_t* __restrict__ idx,
    const float* __restrict__ lse, const float* __restrict__ isc, int64_t n_q, int64_t n_k, int H, int d_qk,
    int k, float sm_scale, float* __restrict__ kl, float* __restrict__ p_out) {
  __shared__ float red[4];
  const int b = blockIdx.y;
  const int64_t qrow = (int64_t)b * n_q + blockIdx.x;
  const int32_t* irow = idx + qrow * k;
  const float* srow = isc + qrow * k;
  const float* kvb = kv + (int64_t)b * n_k * d_qk;
  float m = -INFINITY;
  for (int j = threadIdx.x; j < k; j += 256) {
    const int32_t id = irow[j];
    if (id >= 0 && (int64_t)id < n_k) m = fmaxf(m, srow[j]);
  }
  m = block_reduce(m, red, true);
  float s = 0.f;
  if (m > -INFINITY)
    for (int j = threadIdx.x; j < k; j += 256) {
      const int32_t id = irow[j];
      if (id >= 0 && (int64_t)id < n_k) s += expf(srow[j] - m);
    }
  s = block_reduce(s, red, false);
  const float lsei = m > -INFINITY ? m + logf(s) : -INFINITY;
  float acc = 0.f;
  for (int j = threadIdx.x; j < k; j += 256) {
    const int32_t id = irow[j];
    float p = 0.f;
    if (id >= 0 && (int64_t)id < n_k) {
      const float* kr = kvb + (int64_t)id * d_qk;
      for (int h = 0; h < H; ++h) {
        const float* qh = q + (qrow * H + h) * d_qk;
        float dot = 0.f;
        for (int d = 0; d < d_qk; ++d) dot = __fmaf_rn(qh[d], kr[d], dot);
        p += expf(dot * sm_scale - lse[qrow * H + h]);
      }
      p /= (float)H;
      if (p > 0.f) acc += p * (logf(p) - (srow[j] - lsei));
    }
    if (p_out) p_out[qrow * k + j] = p;
  }
  acc = block_reduce(acc, red, false);
  if (threadIdx.x == 0) kl[qrow] = acc;
}

// ---------------------------------------------------------------------------------------
// KL loss of the dense warm-up: every key s <= pos(t), the attention's own dense lse
// ---------------------------------------------------------------------------------------
// Per query row t (position pos, keys 0 .. n-1 with n = min(pos + 1, n_k)):
//     LSE_I   = ln sum_{s<n} exp(I[t,s])                (the index scores of the whole row)
//     lse_h   = ln sum_{s<n} exp(sm_scale q_h . kv_s)     (dense attention, every head)
//     p(s)    = (1/H) sum_h exp(sm_scale q_h . kv_s - lse_h)
//     KL_t    = sum_{s<n} p(s) (ln p(s) - I[t,s] + LSE_I)
// The score row comes from the caller's workspace (written by the indexer just before);
// the rows of kv are contiguous, so chunk c of a row is keys 32c .. 32c+31.

// The ids of a dense chunk (see kl_ids): keys are their own ids.
__device__ __forceinline__ KlIds dense_ids(int c, int wv, int lane) {
  return KlIds{c * KC + 8 * wv + (lane & 7), c * KC + 8 * wv + (lane >> 3)};
}

// log2-domain log-sum-exp of a block's values (NT threads): combines per-thread (m, s)
__device__ __forceinline__ void merge_lse2(float& m, float& s, float om, float os) {
  const float M = fmaxf(m, om);
  s = (M == -INFINITY) ? 0.f : s * exp2f(m - M) + os * exp2f(om - M);
  m = M;
}

// grid.x = rows of the launch, grid.y = B.  Row i of sequence b is query row row_begin + i
// at position (q_pos ? q_pos[b] : 0) + row_begin + i; its index scores are at
// isc + (b * n_rows + i) * ld_s.  Two sweeps over the keys, two chunk buffers each: the
// first forms every head's lse (online, per lane, merged across lanes at the end), the
// second the KL terms exactly as indexer_kl_bf16_kernel does for a selection.
__global__ __launch_bounds__(KL_WAVES * 64, 2) void indexer_kl_dense_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const float* __restrict__ isc, int64_t ld_s,
    const int32_t* __restrict__ q_pos, int64_t row_begin, int64_t n_rows, int64_t n_q, int64_t n_k,
    float scale_log2, float* __restrict__ kl, float* __restrict__ lse_out) {
  __shared__ __align__(16) uint8_t buf0[CHUNK_BYTES];
  __shared__ __align__(16) uint8_t buf1[CHUNK_BYTES];
  __shared__ float xs[2][KL_WAVES][KC];
  __shared__ float red[2][KL_WAVES];

  const int tid = threadIdx.x, l = tid & 63, g = l >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.y;
  const int64_t row = row_begin + blockIdx.x;
  const int64_t qrow = (int64_t)b * n_q + row;
  const int64_t pos = (q_pos ? (int64_t)q_pos[b] : 0) + row;
  const int64_t n64 = pos + 1 < n_k ? pos + 1 : n_k;
  const int n = (int)(n64 > 0 ? n64 : 0);
  const float* srow = isc + ((int64_t)b * n_rows + blockIdx.x) * ld_s;
  const uint16_t* kvb = kv + (int64_t)b * n_k * MDQK;

  if (n == 0) {  // no key before the query: no distribution (uniform over the block)
    if (tid == 0) kl[qrow] = 0.f;
    if (lse_out && tid < MH) lse_out[qrow * MH + tid] = -INFINITY;
    return;
  }

  // ---- LSE_I over the whole score row (log2 units), every thread then the block
  float mi = -INFINITY, si = 0.f;
  for (int s = tid; s < n; s += KL_WAVES * 64) {
    const float x = srow[s] * LOG2E;
    if (x > mi) {
      si = si * exp2f(mi - x) + 1.f;
      mi = x;
    } else {
      si += exp2f(x - mi);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) merge_lse2(mi, si, __shfl_xor(mi, off, WAVE), __shfl_xor(si, off, WAVE));
  if (l == 0) {
    red[0][wv] = mi;
    red[1][wv] = si;
  }
  __syncthreads();
  float lsei2 = -INFINITY;
  {
    float m = red[0][0], sm = red[1][0];
#pragma unroll
    for (int w2 = 1; w2 < KL_WAVES; ++w2) merge_lse2(m, sm, red[0][w2], red[1][w2]);
    lsei2 = m + log2f(sm);
  }

  // A operands of S = Q K^T: head 32w + l%32, values 16ds + 8g .. +7
  v8bf Qa[D_STEPS];
  {
    const uint16_t* qh = q + (qrow * MH + 32 * wv + (l & 31)) * MDQK + 8 * g;
#pragma unroll
    for (int ds = 0; ds < D_STEPS; ++ds) Qa[ds] = *reinterpret_cast<const v8bf*>(qh + 16 * ds);
#pragma unroll
    for (int ds = 0; ds < D_STEPS; ++ds) asm volatile("" : "+v"(Qa[ds]));
  }
  const int nch = (n + KC - 1) / KC;
  const uint32_t nk = (uint32_t)n;  // keys past the row's position read row 0 and are masked
  const KOff ko = k_offsets();

  // ---- sweep 1: every head's log2-sum-exp.  Lane l holds key 32c + l%32 and the 16 heads
  // 32w + 8(r/4) + 4g + r%4; per lane and head a running reference m (moved only when a
  // logit passes it by 8) and a sum of exp2(x - m).
  float L2[16], sr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    L2[r] = -1e30f;  // finite: exp2(-inf - m) is 0, and no -inf - -inf arises
    sr[r] = 0.f;
  }
  kl_gather(lds_addr(buf0), kvb, dense_ids(0, wv, l), nk, wv, l);
  for (int c = 0; c < nch; ++c) {
    VMCNT(0);
    block_barrier();
    if (c + 1 < nch) kl_gather(lds_addr((c & 1) ? buf0 : buf1), kvb, dense_ids(c + 1, wv, l), nk, wv, l);
    v16f S = {};
    const uint8_t* cur = (c & 1) ? buf1 : buf0;
#pragma unroll
    for (int ds = 0; ds < D_STEPS; ++ds) S = mfma_bf16_32x32x16(Qa[ds], k_frag(cur, k_off(ko, ds)), S);
    const bool valid = c * KC + (l & 31) < n;
    float x[16];
    bool up = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = valid ? S[r] * scale_log2 : -INFINITY;
      up |= x[r] > L2[r] + 8.f;
    }
    if (ballot(up)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float nm = fmaxf(L2[r], x[r]);
        sr[r] *= exp2f(L2[r] - nm);
        L2[r] = nm;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sr[r] += __builtin_amdgcn_exp2f(x[r] - L2[r]);
  }
  // merge over the 32 lanes of each half (they hold the same heads)
#pragma unroll
  for (int r = 0; r < 16; ++r) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1)
      merge_lse2(L2[r], sr[r], __shfl_xor(L2[r], off, WAVE), __shfl_xor(sr[r], off, WAVE));
    L2[r] += log2f(sr[r]);
  }
  if (lse_out && (l & 31) == 0)
#pragma unroll
    for (int r = 0; r < 16; ++r) lse_out[qrow * MH + 32 * wv + 8 * (r >> 2) + 4 * g + (r & 3)] = L2[r] * LN2;

  // ---- sweep 2: p(s) and the KL terms (wave 0 adds the four waves' head sums one chunk later)
  VMCNT(0);
  block_barrier();  // every wave is done with both buffers
  kl_gather(lds_addr(buf0), kvb, dense_ids(0, wv, l), nk, wv, l);
  float acc = 0.f;
  float a_s = 0.f;
  bool a_ok = false;
  for (int c = 0; c < nch; ++c) {
    VMCNT(0);
    block_barrier();
    if (c + 1 < nch) kl_gather(lds_addr((c & 1) ? buf0 : buf1), kvb, dense_ids(c + 1, wv, l), nk, wv, l);
    const int key = c * KC + (l & 31);
    const bool c_ok = key < n;
    const float c_s = (wv == 0 && c_ok) ? srow[key] : 0.f;
    v16f S = {};
    const uint8_t* cur = (c & 1) ? buf1 : buf0;
#pragma unroll
    for (int ds = 0; ds < D_STEPS; ++ds) S = mfma_bf16_32x32x16(Qa[ds], k_frag(cur, k_off(ko, ds)), S);
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ps += __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], scale_log2, -L2[r]));
    ps += xor32(ps);
    if (l < KC) xs[c & 1][wv][l] = ps;
    if (wv == 0 && c > 0) {
      const float* xx = xs[(c - 1) & 1][0];
      const float p = (xx[l & 31] + xx[KC + (l & 31)] + xx[2 * KC + (l & 31)] + xx[3 * KC + (l & 31)]) * (1.f / MH);
      if (l < KC && a_ok && p > 0.f) acc += p * ((log2f(p) - (a_s * LOG2E - lsei2)) * LN2);
    }
    a_ok = c_ok;
    a_s = c_s;
  }
  VMCNT(0);
  block_barrier();
  if (wv == 0) {
    const float* xx = xs[(nch - 1) & 1][0];
    const float p = (xx[l & 31] + xx[KC + (l & 31)] + xx[2 * KC + (l & 31)] + xx[3 * KC + (l & 31)]) * (1.f / MH);
    if (l < KC && a_ok && p > 0.f) acc += p * ((log2f(p) - (a_s * LOG2E - lsei2)) * LN2);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, WAVE);
    if (l == 0) kl[qrow] = acc;
  }
}

// fp32 operands (small shapes: H <= 64, d_qk <= 256, n_k <= KLD_F32_MAX_N): one block per
// query row; each head's logits go through LDS, p accumulates there.
constexpr int KLD_F32_MAX_N = 4096;
__global__ __launch_bounds__(256) void indexer_kl_dense_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kv, const float* __restrict__ isc, int64_t ld_s,
    const int32_t* __restrict__ q_pos, int64_t row_begin, int64_t n_rows, int64_t n_q, int64_t n_k, int H,
    int d_qk, float sm_scale, float* __restrict__ kl, float* __restrict__ lse_out) {
  __shared__ float red[4];
  __shared__ float z[KLD_F32_MAX_N];
  __shared__ float pp[KLD_F32_MAX_N];
  const int b = blockIdx.y;
  const int64_t row = row_begin + blockIdx.x;
  const int64_t qrow = (int64_t)b * n_q + row;
  const int64_t pos = (q_pos ? (int64_t)q_pos[b] : 0) + row;
  const int64_t n64 = pos + 1 < n_k ? pos + 1 : n_k;
  const int n = (int)(n64 > 0 ? n64 : 0);
  const float* srow = isc + ((int64_t)b * n_rows + blockIdx.x) * ld_s;
  const float* kvb = kv + (int64_t)b * n_k * d_qk;
  if (n == 0) {
    if (threadIdx.x == 0) kl[qrow] = 0.f;
    if (lse_out)
      for (int h = threadIdx.x; h < H; h += 256) lse_out[qrow * H + h] = -INFINITY;
    return;
  }
  float m = -INFINITY;
  for (int s = threadIdx.x; s < n; s += 256) m = fmaxf(m, srow[s]);
  m = block_reduce(m, red, true);
  float sum = 0.f;
  for (int s = threadIdx.x; s < n; s += 256) sum += expf(srow[s] - m);
  sum = block_reduce(sum, red, false);
  const float lsei = m + logf(sum);
  for (int s = threadIdx.x; s < n; s += 256) pp[s] = 0.f;
  for (int h = 0; h < H; ++h) {
    const float* qh = q + (qrow * H + h) * d_qk;
    float mh = -INFINITY;
    for (int s = threadIdx.x; s < n; s += 256) {
      const float* kr = kvb + (int64_t)s * d_qk;
      float dot = 0.f;
      for (int d = 0; d < d_qk; ++d) dot = __fmaf_rn(qh[d], kr[d], dot);
      z[s] = dot * sm_scale;
      mh = fmaxf(mh, z[s]);
    }
    mh = block_reduce(mh, red, true);
    float sh = 0.f;
    for (int s = threadIdx.x; s < n; s += 256) sh += expf(z[s] - mh);
    sh = block_reduce(sh, red, false);
    const float lh = mh + logf(sh);
    if (lse_out && threadIdx.x == 0) lse_out[qrow * H + h] = lh;
    for (int s = threadIdx.x; s < n; s += 256) pp[s] += expf(z[s] - lh);
  }
  float acc = 0.f;
  for (int s = threadIdx.x; s < n; s += 256) {
    const float p = pp[s] / (float)H;
    if (p > 0.f) acc += p * (logf(p) - (srow[s] - lsei));
  }
  acc = block_reduce(acc, red, false);
  if (threadIdx.x == 0) kl[qrow] = acc;
}

hipError_t launch_indexer_kl_dense(const KlDenseArgs& a, hipStream_t st) {
  dim3 grid((unsigned)a.n_rows, (unsigned)a.B);
  if (a.dtype == DSA_F32) {
    hipLaunchKernelGGL(indexer_kl_dense_f32_kernel, grid, dim3(256), 0, st, (const float*)a.q, (const float*)a.kv,
                       a.scores, a.ld_s, a.q_pos, a.row_begin, a.n_rows, a.n_q, a.n_k, a.H, a.d_qk, a.sm_scale,
                       a.kl, a.lse);
  } else {
    hipLaunchKernelGGL(indexer_kl_dense_bf16_kernel, grid, dim3(KL_WAVES * 64), 0, st, (const uint16_t*)a.q,
                       (const uint16_t*)a.kv, a.scores, a.ld_s, a.q_pos, a.row_begin, a.n_rows, a.n_q, a.n_k,
                       a.sm_scale * LOG2E, a.kl, a.lse);
  }
  return hipGetLastError();
}

hipError_t launch_indexer_kl(const KlArgs& a, hipStream_t st) {
  dim3 grid((unsigned)a.n_q, (unsigned)a.B);
  if (a.dtype == DSA_F32) {
    hipLaunchKernelGGL(indexer_kl_f32_kernel, grid, dim3(256), 0, st, (const float*)a.q, (const float*)a.kv,
                       a.idx, a.lse, a.scores, a.n_q, a.n_k, a.H, a.d_qk, a.k, a.sm_scale, a.kl, a.p_out);
  } else {
    hipLaunchKernelGGL(indexer_kl_bf16_kernel, grid, dim3(KL_WAVES * 64), 0, st, (const uint16_t*)a.q,
                       (const uint16_t*)a.kv, a.idx, a.lse, a.scores, a.n_q, a.n_k, a.k, a.sm_scale * LOG2E,
                       a.kl, a.p_out);
  }
  return hipGetLastError();
}

}  // namespace dsa
