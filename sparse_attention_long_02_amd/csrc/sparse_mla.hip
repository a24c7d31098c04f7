// Attention over the selected keys, MLA in MQA mode (dsa_sparse_mla, prefill, decode).
//
// Every query head attends over the same selected latent rows: one key-value row of
// 576 values serves all 128 heads, and V is its first 512 values (MQA mode of MLA:
// 53ai.com V3.2-Exp summary, section 创新架构 and Figure 1; paperbridge.wiki summary,
// section DeepSeek Sparse Attention).  Attention is computed only over the k kept keys,
// so its cost per query is O(k) (same sections).
//
// bf16 kernel (H = 128, d_qk = 576, d_v = 512), one block of 4 waves per query:
//   * wave w owns heads 32w .. 32w+31 (two 16-head MFMA column blocks);
//   * keys are processed in chunks of 32 gathered rows, double-buffered in LDS in two
//     layouts: row-major K (1152 B/row + pad) and a transposed copy of the 512 latent
//     values (V^T, 32 keys contiguous per value);
//   * logits are formed as S^T = K Q^T (keys = MFMA rows, heads = columns), so after the
//     softmax each lane already holds P^T in the B-operand layout of the PV product
//     O^T = V^T P^T: no register transpose of P is needed;
//   * fp32 online softmax in base 2; O^T stays in 256 fp32 registers per lane.
// Keys may be split over several blocks (decode): each writes a normalised partial O and
// its lse, and a combine kernel merges them.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int MH = 128, MDQK = 576, MDV = 512, KC = 32;
constexpr int KROW_STRIDE = MDQK * 2 + 16;        // bytes per key row in LDS
constexpr int VT_STRIDE = KC * 2 + 16;            // bytes per latent value row of V^T
constexpr int KROW_BYTES = KC * KROW_STRIDE;      // 37376
constexpr int VT_BYTES = MDV * VT_STRIDE;         // 40960
constexpr int BUF_BYTES = KROW_BYTES + VT_BYTES;  // 78336
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// one chunk's worth of gathered 16-byte units held by a thread between load and store
struct ChunkRegs {
  v4i lat[8];  // keys 8*o .. 8*o+7, latent values 8*u .. 8*u+7
  v4i rope;    // key t/8, rope values 512 + 8*(t%8) ..
};

__device__ __forceinline__ int64_t clamp_key(int32_t s, int64_t n_k) {
  return (s >= 0 && s < n_k) ? (int64_t)s : 0;
}

__device__ __forceinline__ void load_chunk(ChunkRegs& R, const uint16_t* __restrict__ kvb,
                                           const int32_t* __restrict__ keys, int tid, int64_t n_k) {
  const int o = tid >> 6, u = tid & 63;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t s = clamp_key(keys[8 * o + j], n_k);
    R.lat[j] = *reinterpret_cast<const v4i*>(kvb + s * MDQK + 8 * u);
  }
  const int64_t s = clamp_key(keys[tid >> 3], n_k);
  R.rope = *reinterpret_cast<const v4i*>(kvb + s * MDQK + 512 + 8 * (tid & 7));
}

__device__ __forceinline__ void store_chunk(const ChunkRegs& R, uint8_t* buf, int tid) {
  const int o = tid >> 6, u = tid & 63;
  uint8_t* krow = buf;
  uint8_t* vt = buf + KROW_BYTES;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<v4i*>(krow + (8 * o + j) * KROW_STRIDE + 16 * u) = R.lat[j];
  *reinterpret_cast<v4i*>(krow + (tid >> 3) * KROW_STRIDE + 1024 + 16 * (tid & 7)) = R.rope;
  // 8x8 transpose of 16-bit values: row i of the output = value 8u+i of keys 8o..8o+7
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
    v4i t;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      t[m] = (int)__builtin_amdgcn_perm((uint32_t)R.lat[2 * m + 1][i >> 1], (uint32_t)R.lat[2 * m][i >> 1], sel);
    *reinterpret_cast<v4i*>(vt + (8 * u + i) * VT_STRIDE + 16 * o) = t;
  }
}

// A operand of S^T: key block kb holds keys sigma(r) = 8*(r/4) + 4*kb + r%4 for MFMA row r,
// so the four rows a lane group sees in the output are keys 8g+4kb .. 8g+4kb+3.
__device__ __forceinline__ v8bf krow_frag(const uint8_t* buf, int kb, int ds) {
  const int l = lane_id();
  const int r = l & 15, g = l >> 4;
  const int key = 8 * (r >> 2) + 4 * kb + (r & 3);
  return *reinterpret_cast<const v8bf*>(buf + key * KROW_STRIDE + 64 * ds + 16 * g);
}

// A operand of O^T = V^T P^T for latent values 16*db .. +15: row = value, 8 keys 8g..8g+7
__device__ __forceinline__ v8bf vt_frag(const uint8_t* buf, int db) {
  const int l = lane_id();
  return *reinterpret_cast<const v8bf*>(buf + KROW_BYTES + (16 * db + (l & 15)) * VT_STRIDE + 16 * (l >> 4));
}

// grid.x = n_q * n_split, grid.y = B
__global__ __launch_bounds__(256, 1) void sparse_mla_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    int64_t n_q, int64_t n_k, int k, float scale_log2, int n_split, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __align__(16) uint8_t smem[2 * BUF_BYTES];
  __shared__ int32_t s_last[4];

  const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, g = l >> 4;
  const int b = blockIdx.y;
  const int64_t qi = blockIdx.x / n_split;
  const int split = blockIdx.x % n_split;
  const int64_t qrow = (int64_t)b * n_q + qi;
  const int32_t* irow = idx + qrow * k;
  const uint16_t* kvb = kv + (int64_t)b * n_k * MDQK;

  // number of chunks up to the last valid index of the row
  int last = -1;
  for (int j = tid; j < k; j += 256)
    if (irow[j] >= 0 && irow[j] < n_k) last = j;
  last = (int)wave_max((float)last);
  if (l == 0) s_last[wv] = last;
  __syncthreads();
  last = max(max(s_last[0], s_last[1]), max(s_last[2], s_last[3]));
  const int nchunks = (last + KC) / KC;  // 0 if no valid key
  const int c_lo = (int)((int64_t)nchunks * split / n_split);
  const int c_hi = (int)((int64_t)nchunks * (split + 1) / n_split);

  // Q^T B operands: head 32w + 16hb + l%16, values 32ds + 8g .. +7
  v8bf Qt[2][18];
  const uint16_t* qb = q + qrow * MH * MDQK;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int ds = 0; ds < 18; ++ds)
      Qt[hb][ds] = *reinterpret_cast<const v8bf*>(qb + (32 * wv + 16 * hb + (l & 15)) * MDQK + 32 * ds + 8 * g);

  v4f O[32][2];
#pragma unroll
  for (int db = 0; db < 32; ++db) O[db][0] = O[db][1] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  ChunkRegs CR;
  if (c_lo < c_hi) {
    load_chunk(CR, kvb, irow + c_lo * KC, tid, n_k);
    store_chunk(CR, smem, tid);
  }
  __syncthreads();
  for (int c = c_lo; c < c_hi; ++c) {
    uint8_t* buf = smem + ((c - c_lo) & 1) * BUF_BYTES;
    const bool more = c + 1 < c_hi;
    // validity of the chunk's 32 keys (bit j = key j), wave-uniform
    const int32_t my = irow[c * KC + (l & 31)];
    const uint32_t vmask = (uint32_t)ballot(c * KC + (l & 31) < k && my >= 0 && my < n_k);

    // ---- S^T = K Q^T
    v4f S[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) S[kb][0] = S[kb][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < 18; ++ds)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const v8bf a = krow_frag(buf, kb, ds);
        S[kb][0] = mfma_bf16_16x16x32(a, Qt[0][ds], S[kb][0]);
        S[kb][1] = mfma_bf16_16x16x32(a, Qt[1][ds], S[kb][1]);
      }

    // ---- online softmax per head (lane: head l%16 of block hb, keys 8g .. 8g+7)
    v8bf P[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float z[8];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = (vmask >> (8 * g + j)) & 1u;
        z[j] = ok ? S[j >> 2][hb][j & 3] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, z[j]);
      }
      mx = fmaxf(mx, xor16(mx));
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run[hb], mx);
      const bool any = m_new != -INFINITY;
      const float alpha = any ? exp2f(m_run[hb] - m_new) : 1.f;
      float ps = 0.f;
      uint32_t pk[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float p0 = any ? exp2f(z[j] - m_new) : 0.f;
        const float p1 = any ? exp2f(z[j + 1] - m_new) : 0.f;
        ps += p0 + p1;
        pk[j >> 1] = pack_bf16x2(p0, p1);
      }
      ps += xor16(ps);
      ps += xor32(ps);
      l_run[hb] = l_run[hb] * alpha + ps;
      m_run[hb] = m_new;
      if (ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < 32; ++db) O[db][hb] *= alpha;
      }
      v4i pv = v4i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
      P[hb] = __builtin_bit_cast(v8bf, pv);
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      const v8bf a = vt_frag(buf, db);
      O[db][0] = mfma_bf16_16x16x32(a, P[0], O[db][0]);
      O[db][1] = mfma_bf16_16x16x32(a, P[1], O[db][1]);
    }
    if (more) {
      load_chunk(CR, kvb, irow + (c + 1) * KC, tid, n_k);
      store_chunk(CR, smem + ((c + 1 - c_lo) & 1) * BUF_BYTES, tid);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds head 32w+16hb+l%16, values 16db + 4g + i
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = 32 * wv + 16 * hb + (l & 15);
    const bool nonempty = l_run[hb] > 0.f;
    const float inv = nonempty ? 1.f / l_run[hb] : 0.f;
    const float lse_v = nonempty ? (m_run[hb] + log2f(l_run[hb])) * LN2 : -INFINITY;
    if (n_split == 1) {
      uint16_t* orow = out + (qrow * MH + head) * MDV;
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        const v4f o = O[db][hb] * inv;
        uint2 pkd;
        pkd.x = pack_bf16x2(o[0], o[1]);
        pkd.y = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<uint2*>(orow + 16 * db + 4 * g) = pkd;
      }
      if (lse && g == 0) lse[qrow * MH + head] = lse_v;
    } else {
      float* prow = part_o + ((qrow * n_split + split) * MH + head) * MDV;
#pragma unroll
      for (int db = 0; db < 32; ++db) *reinterpret_cast<v4f*>(prow + 16 * db + 4 * g) = O[db][hb] * inv;
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
