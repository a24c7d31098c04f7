// Attention over the selected keys, MLA in MQA mode (dsa_sparse_mla, prefill, decode).
//
// Every query head attends over the same selected latent rows: one key-value row of
// 576 values serves all 128 heads, and V is its first 512 values (MQA mode of MLA:
// 53ai.com V3.2-Exp summary, section 创新架构 and Figure 1; paperbridge.wiki summary,
// section DeepSeek Sparse Attention).  Attention is computed only over the k kept keys,
// so its cost per query is O(k) (same sections).
//
// bf16 kernel (H = 128, d_qk = 576, d_v = 512), one block of 4 waves per query:
//   * wave w owns heads 32w .. 32w+31 (two 16-head MFMA column blocks); its Q^T operands
//     (144 registers) and O^T accumulators (256 fp32 registers) stay in registers;
//   * keys are processed in chunks of 32 gathered rows.  The rows go straight from HBM to
//     LDS with 16-byte direct loads (no staging registers; the latent half of a row is one
//     wave-wide 1 KB load from a scalar address) into a ring of four buffers, so three
//     chunks are in flight while one is computed;
//   * logits are formed as S^T = K Q^T (keys = MFMA rows, heads = columns), so after the
//     softmax each lane already holds P^T in the B-operand layout of the PV product
//     O^T = V^T P^T; V^T is read from the same row-major rows with the gfx950 transposing
//     LDS read, so no transposed copy is stored;
//   * fp32 online softmax in base 2 whose reference max moves only when a logit exceeds
//     it by 8 (P then stays <= 256, exact enough in bf16), which keeps the 256-register
//     rescale off the common path.
// Keys may be split over several blocks (decode): each writes a normalised partial O and
// its lse, and a combine kernel merges them.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int MH = 128, MDQK = 576, MDV = 512, KC = 32;
// LDS image of one chunk of 32 gathered rows, in two regions whose row pitches sit 4 banks
// past a multiple of the bank count (so 8 consecutive rows read at one column hit distinct
// banks, and every LDS read is a per-lane base plus an immediate offset):
//   latent: values 0..511 of each row, 1040 B apart (1024 B + one unused 16-byte unit);
//   rope:   values 512..575 of each row, 144 B apart (128 B + one unused unit).
constexpr int LAT_PITCH = 1040, ROPE_PITCH = 144;
constexpr int LAT_BYTES = KC * LAT_PITCH;                      // 33280
constexpr int ROPE_UNITS = KC * ROPE_PITCH / 16;               // 288
constexpr int ROPE_INSTR = (ROPE_UNITS + 63) / 64;             // 5
constexpr int CHUNK_BYTES = LAT_BYTES + ROPE_INSTR * 64 * 16;  // 33280 + 5120 = 38400
constexpr int MAX_K = 2048;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_SLACK = 8.f;              // log2 units the running max may lag

#define VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

__device__ __forceinline__ int64_t safe_row(int32_t s, int64_t n_k) {
  return (s >= 0 && s < n_k) ? (int64_t)s : 0;
}

// Issue this wave's direct global->LDS loads for chunk c (rows ids[32c .. 32c+31]):
// the latent halves of rows 8w .. 8w+7 (one wave-wide 1 KB load each, scalar row
// address) and rope instruction w (wave 0 also instruction 4).  Wave 0 issues 10 loads,
// the others 9.
__device__ __forceinline__ void gather_chunk(uint8_t* buf, const uint16_t* __restrict__ kvb,
                                             const int32_t* ids, int c, int64_t n_k, int wv, int lane) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * wv + j;
    const int64_t row = safe_row(__builtin_amdgcn_readfirstlane(ids[c * KC + r]), n_k);
    __builtin_amdgcn_global_load_lds(kvb + row * MDQK + 8 * lane, buf + r * LAT_PITCH, 16, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ins = wv + 4 * i;
    if (ins < ROPE_INSTR) {
      const int u = ins * 64 + lane;               // rope unit: row u / 9, unit u % 9 (8 = pad)
      const int r = min(u / 9, KC - 1);
      const int cu = u - (u / 9) * 9;
      const int64_t row = safe_row(ids[c * KC + r], n_k);
      __builtin_amdgcn_global_load_lds(kvb + row * MDQK + 512 + 8 * (cu & 7), buf + LAT_BYTES + ins * 1024, 16, 0, 0);
    }
  }
}

// A operand of S^T for key block kb and d-step ds (values 32ds .. 32ds+31): MFMA row p is
// key 16kb + p, so the output rows a lane group g sees are keys 16kb+4g .. 16kb+4g+3.
__device__ __forceinline__ v8bf krow_frag(const uint8_t* buf, int kb, int ds) {
  const int l = lane_id();
  const int r = 16 * kb + (l & 15);
  const uint8_t* p = ds < 16 ? buf + r * LAT_PITCH + 64 * ds + 16 * (l >> 4)
                             : buf + LAT_BYTES + r * ROPE_PITCH + 64 * (ds - 16) + 16 * (l >> 4);
  return *reinterpret_cast<const v8bf*>(p);
}

// A operand of O^T = V^T P^T for latent values 16*db .. +15 (rows); the contraction slots
// of lane group g are keys 4g..4g+3 (first read) and 16+4g..16+4g+3 (second read), the
// same keys in the same order as that lane's P^T slots.  The gfx950 transposing LDS read
// does the transpose: in a 16-lane group, lanes 4rr..4rr+3 supply 16 values of one key
// and lane p receives value 16db + p of the four keys.
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v8bf vt_frag(const uint8_t* buf, int db) {
  const int l = lane_id();
  const int p = l & 15, g = l >> 4;
  const int rr = p >> 2, qq = p & 3;
  typedef __attribute__((address_space(3))) v4s* lds_v4s;
  const uint8_t* a0 = buf + (4 * g + rr) * LAT_PITCH + 32 * db + 8 * qq;
  const uint8_t* a1 = a0 + 16 * LAT_PITCH;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(__attribute__((address_space(3))) uint8_t*)a0);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(__attribute__((address_space(3))) uint8_t*)a1);
  const v8s v = v8s{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(v8bf, v);
}

struct MlaState {
  v8bf Qt[2][18];
  v4f O[32][2];
  float m_ref[2], l_run[2];
};

// One chunk: S^T = K Q^T, online softmax (base 2, lazily rescaled), O^T += V^T P^T.
__device__ __forceinline__ void mla_chunk(MlaState& st, const uint8_t* buf, uint32_t vmask, float scale_log2) {
  const int l = lane_id(), g = l >> 4;
  v4f S[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) S[kb][0] = S[kb][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < 18; ++ds)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const v8bf a = krow_frag(buf, kb, ds);
      S[kb][0] = mfma_bf16_16x16x32(a, st.Qt[0][ds], S[kb][0]);
      S[kb][1] = mfma_bf16_16x16x32(a, st.Qt[1][ds], S[kb][1]);
    }
  v8bf P[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    float z[8];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = (vmask >> (16 * (j >> 2) + 4 * g + (j & 3))) & 1u;
      z[j] = ok ? S[j >> 2][hb][j & 3] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, z[j]);
    }
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx));
    // move the reference max only when a logit exceeds it by more than the slack
    if (ballot(mx > st.m_ref[hb] + RESCALE_SLACK)) {
      const float m_new = fmaxf(st.m_ref[hb], mx);
      const float alpha = st.m_ref[hb] == -INFINITY ? 0.f : exp2f(st.m_ref[hb] - m_new);
      st.l_run[hb] *= alpha;
#pragma unroll
      for (int db = 0; db < 32; ++db) st.O[db][hb] *= alpha;
      st.m_ref[hb] = m_new;
    }
    const float m = st.m_ref[hb];
    float ps = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float p0 = z[j] == -INFINITY ? 0.f : exp2f(z[j] - m);
      const float p1 = z[j + 1] == -INFINITY ? 0.f : exp2f(z[j + 1] - m);
      ps += p0 + p1;
      pk[j >> 1] = pack_bf16x2(p0, p1);
    }
    ps += xor16(ps);
    ps += xor32(ps);
    st.l_run[hb] += ps;
    const v4i pv = v4i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
    P[hb] = __builtin_bit_cast(v8bf, pv);
  }
#pragma unroll
  for (int db = 0; db < 32; ++db) {
    const v8bf a = vt_frag(buf, db);
    st.O[db][0] = mfma_bf16_16x16x32(a, P[0], st.O[db][0]);
    st.O[db][1] = mfma_bf16_16x16x32(a, P[1], st.O[db][1]);
  }
}

__device__ __forceinline__ uint32_t chunk_mask(const int32_t* ids, int c, int64_t n_k) {
  const int32_t s = ids[c * KC + (lane_id() & 31)];
  return (uint32_t)ballot(s >= 0 && s < n_k);
}

// grid.x = n_q * n_split, grid.y = B.  Pipeline: chunk c+3 is in flight while chunk c is
// computed (4 LDS buffers, loop unrolled by 4 so each buffer is a distinct static array).
__global__ __launch_bounds__(256, 1) void sparse_mla_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    int64_t n_q, int64_t n_k, int k, float scale_log2, int n_split, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __align__(16) uint8_t buf0[CHUNK_BYTES];
  __shared__ __align__(16) uint8_t buf1[CHUNK_BYTES];
  __shared__ __align__(16) uint8_t buf2[CHUNK_BYTES];
  __shared__ __align__(16) uint8_t buf3[CHUNK_BYTES];
  __shared__ int32_t ids[MAX_K];
  __shared__ int32_t s_last[4];

  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, g = l >> 4;
  const int b = blockIdx.y;
  const int64_t qi = blockIdx.x / n_split;
  const int split = blockIdx.x % n_split;
  const int64_t qrow = (int64_t)b * n_q + qi;
  const int32_t* irow = idx + qrow * k;
  const uint16_t* kvb = kv + (int64_t)b * n_k * MDQK;

  MlaState st;
  const uint16_t* qb = q + qrow * MH * MDQK;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int ds = 0; ds < 18; ++ds)
      st.Qt[hb][ds] = *reinterpret_cast<const v8bf*>(qb + (32 * wv + 16 * hb + (l & 15)) * MDQK + 32 * ds + 8 * g);

  // the row's selected ids -> LDS; chunks up to the last valid id
  int last = -1;
  for (int j = tid; j < k; j += 256) {
    const int32_t s = irow[j];
    ids[j] = s;
    if (s >= 0 && s < n_k) last = j;
  }
  last = (int)wave_max((float)last);
  if (l == 0) s_last[wv] = last;
  __syncthreads();
  last = max(max(s_last[0], s_last[1]), max(s_last[2], s_last[3]));
  const int nchunks = (last + KC) / KC;
  const int c_lo = (int)((int64_t)nchunks * split / n_split);
  const int c_hi = (int)((int64_t)nchunks * (split + 1) / n_split);

#pragma unroll
  for (int db = 0; db < 32; ++db) st.O[db][0] = st.O[db][1] = v4f{0.f, 0.f, 0.f, 0.f};
  st.m_ref[0] = st.m_ref[1] = -INFINITY;
  st.l_run[0] = st.l_run[1] = 0.f;

  uint8_t* bufs[4] = {buf0, buf1, buf2, buf3};
  const int n = c_hi - c_lo;
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (j < n) gather_chunk(bufs[j], kvb, ids, c_lo + j, n_k, wv, l);

  for (int base = 0; base < n; base += 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + j;  // chunk ordinal within this split
      if (i < n) {
        // chunk i must have landed (chunks i+1, i+2 may still be in flight), in every wave
        if (wv == 0) {
          if (i + 2 < n) VMCNT(20);
          else if (i + 1 < n) VMCNT(10);
          else VMCNT(0);
        } else {
          if (i + 2 < n) VMCNT(18);
          else if (i + 1 < n) VMCNT(9);
          else VMCNT(0);
        }
        __builtin_amdgcn_s_barrier();
        if (i + 3 < n) gather_chunk(bufs[(j + 3) & 3], kvb, ids, c_lo + i + 3, n_k, wv, l);
        mla_chunk(st, bufs[j], chunk_mask(ids, c_lo + i, n_k), scale_log2);
      }
    }
  }

  // ---- epilogue: lane holds head 32w+16hb+l%16, values 16db + 4g + i
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = 32 * wv + 16 * hb + (l & 15);
    const bool nonempty = st.l_run[hb] > 0.f;
    const float inv = nonempty ? 1.f / st.l_run[hb] : 0.f;
    const float lse_v = nonempty ? (st.m_ref[hb] + log2f(st.l_run[hb])) * LN2 : -INFINITY;
    if (n_split == 1) {
      uint16_t* orow = out + (qrow * MH + head) * MDV;
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        const v4f o = st.O[db][hb] * inv;
        uint2 pkd;
        pkd.x = pack_bf16x2(o[0], o[1]);
        pkd.y = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<uint2*>(orow + 16 * db + 4 * g) = pkd;
      }
      if (lse && g == 0) lse[qrow * MH + head] = lse_v;
    } else {
      float* prow = part_o + ((qrow * n_split + split) * MH + head) * MDV;
#pragma unroll
      for (int db = 0; db < 32; ++db) *reinterpret_cast<v4f*>(prow + 16 * db + 4 * g) = st.O[db][hb] * inv;
      if (g == 0) part_lse[(qrow * n_split + split) * MH + head] = lse_v;
    }
  }
}

// merge the splits of one (query, head): O = sum_s e^{lse_s - lse} O_s
__global__ __launch_bounds__(128) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse, int n_split,
                                                          int H, int d_v, uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int64_t qh = blockIdx.x;  // qrow * H + head
  const int64_t qrow = qh / H;
  const int head = (int)(qh % H);
  float mx = -INFINITY;
  for (int s = 0; s < n_split; ++s) mx = fmaxf(mx, part_lse[(qrow * n_split + s) * H + head]);
  float den = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float ls = part_lse[(qrow * n_split + s) * H + head];
    den += mx == -INFINITY ? 0.f : exp2f((ls - mx) * LOG2E);
  }
  for (int d = threadIdx.x; d < d_v; d += 128) {
    float acc = 0.f;
    for (int s = 0; s < n_split; ++s) {
      const float ls = part_lse[(qrow * n_split + s) * H + head];
      const float wgt = mx == -INFINITY ? 0.f : exp2f((ls - mx) * LOG2E);
      acc += wgt * part_o[((qrow * n_split + s) * H + head) * d_v + d];
    }
    out[qh * d_v + d] = f32_to_bf16_bits(den > 0.f ? acc / den : 0.f);
  }
  if (lse && threadIdx.x == 0) lse[qh] = den > 0.f ? mx + logf(den) : -INFINITY;
}

// fp32 attention (any H, d_qk, d_v <= 256, k <= 4096): one wave per (query, head),
// exact two-pass softmax over the selected keys.
constexpr int F32_MAX_K = 4096;
__global__ __launch_bounds__(64) void sparse_mla_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kv, const float* __restrict__ v,
    const int32_t* __restrict__ idx, int64_t n_q, int64_t n_k, int H, int d_qk, int d_v, int k,
    float sm_scale, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float z[F32_MAX_K];
  const int lane = threadIdx.x;
  const int64_t qh = blockIdx.x;  // (b * n_q + t) * H + head
  const int b = blockIdx.y;
  const int64_t qrow = (int64_t)b * n_q + qh / H;
  const int head = (int)(qh % H);
  const float* qv = q + (qrow * H + head) * d_qk;
  const int32_t* irow = idx + qrow * k;
  const float* kvb = kv + (int64_t)b * n_k * d_qk;
  const float* vb = v ? v + (int64_t)b * n_k * d_v : kvb;
  const int64_t vstride = v ? d_v : d_qk;
  float mx = -INFINITY;
  for (int j = 0; j < k; ++j) {
    const int32_t s = irow[j];
    float zz = -INFINITY;
    if (s >= 0 && s < n_k) {
      float part = 0.f;
      for (int d = lane; d < d_qk; d += 64) part = __fmaf_rn(qv[d], kvb[(int64_t)s * d_qk + d], part);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
      zz = sm_scale * part;
    }
    if (lane == 0) z[j] = zz;
    mx = fmaxf(mx, zz);
  }
  __syncthreads();
  float den = 0.f;
  for (int j = 0; j < k; ++j) den += mx == -INFINITY ? 0.f : expf(z[j] - mx);
  float* orow = out + (qrow * H + head) * d_v;
  for (int d = lane; d < d_v; d += 64) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int32_t s = irow[j];
      if (s >= 0 && s < n_k) acc = __fmaf_rn(expf(z[j] - mx), vb[(int64_t)s * vstride + d], acc);
    }
    orow[d] = den > 0.f ? acc / den : 0.f;
  }
  if (lse && lane == 0) lse[qrow * H + head] = den > 0.f ? mx + logf(den) : -INFINITY;
}

int sparse_mla_splits(int64_t B, int64_t n_q, int32_t k, int32_t dtype) {
  if (dtype != DSA_BF16) return 1;
  const int64_t blocks = B * n_q;
  if (blocks >= 1024) return 1;
  const int64_t chunks = (k + KC - 1) / KC;
  int64_t s = (1024 + blocks - 1) / blocks;
  if (s > chunks / 4) s = chunks / 4;  // at least 4 chunks per split
  if (s > 16) s = 16;
  return s < 1 ? 1 : (int)s;
}

size_t sparse_mla_ws_bytes(int64_t B, int64_t n_q, int32_t H, int32_t d_v, int32_t k, int32_t dtype) {
  const int s = sparse_mla_splits(B, n_q, k, dtype);
  if (s <= 1) return 0;
  return (size_t)B * n_q * s * H * ((size_t)d_v + 1) * sizeof(float);
}

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t st) {
  if (a.dtype == DSA_F32) {
    dim3 grid((unsigned)(a.n_q * a.H), (unsigned)a.B);
    hipLaunchKernelGGL(sparse_mla_f32_kernel, grid, dim3(64), 0, st, (const float*)a.q, (const float*)a.kv,
                       (const float*)a.v, a.idx, a.n_q, a.n_k, a.H, a.d_qk, a.d_v, a.k, a.sm_scale,
                       (float*)a.out, a.lse);
    return hipGetLastError();
  }
  const int s = sparse_mla_splits(a.B, a.n_q, a.k, a.dtype);
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (s > 1) {
    part_o = (float*)a.ws;
    part_lse = part_o + (size_t)a.B * a.n_q * s * a.H * a.d_v;
  }
  dim3 grid((unsigned)(a.n_q * s), (unsigned)a.B);
  hipLaunchKernelGGL(sparse_mla_bf16_kernel, grid, dim3(256), 0, st, (const uint16_t*)a.q,
                     (const uint16_t*)a.kv, a.idx, a.n_q, a.n_k, a.k, a.sm_scale * LOG2E, s,
                     (uint16_t*)a.out, a.lse, part_o, part_lse);
  if (s > 1)
    hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)(a.B * a.n_q * a.H)), dim3(128), 0, st, part_o,
                       part_lse, s, a.H, a.d_v, (uint16_t*)a.out, a.lse);
  return hipGetLastError();
}

}  // namespace dsa
