// Backward of the attention over the selected keys (MLA in MQA mode), for the sparse
// training stage, where the main model is trained with the language-modelling loss on the
// sparse pattern (juhe.plus explainer, section 阶段二：Sparse Training; 53ai.com V3.2-Exp
// summary, section 持续预训练; wiki-for-amaranth report, section DeepSeek Sparse Attention).
//
// For query t, head h, selected keys s (valid ids of idx[t]), with the forward's
// P[h,s] = exp(sm_scale q_h . kv_s - lse_h) and O_h = sum_s P[h,s] kv_s[:d_v]:
//     dP[h,s] = dO_h . kv_s[:d_v]
//     D_h     = dO_h . O_h                         (= sum_s P[h,s] dP[h,s])
//     dZ[h,s] = P[h,s] (dP[h,s] - D_h)
//     dq_h    = sm_scale sum_s dZ[h,s] kv_s
//     dkv_s  += sm_scale sum_h dZ[h,s] q_h  +  [sum_h P[h,s] dO_h, 0]   (V = kv[:, :d_v])
//
// bf16 path (H = 128, d_qk = 576, d_v = 512), rows in passes of at most BWD_ROWS queries:
//   1. mla_bwd_transpose: q and dO of the pass, head-minor ([dim][head]), so the dkv
//      product can take head-contiguous operands;
//   2. mla_bwd_dq_kernel: one block of 4 waves per (query, half of the heads), 16 heads
//      per wave.  Selected rows are gathered into LDS as in the forward; per 32-key chunk
//      the wave forms S^T and dP^T with 16x16x32 MFMAs (the two products share their K
//      operand), then P and dZ on the VALU, and accumulates dq^T += K^T dZ^T (K^T by
//      transposing LDS reads; each lane's dZ values are already the B operand).  P and dZ
//      go to the workspace in bf16 ([query][slot][head]);
//   3. dkv, in sub-passes of at most DKV_ROWS queries, without atomics on the rows:
//      a. the (query, slot) pairs of the sub-pass are grouped by key id on the GPU (a CSR:
//         per-key counts, an exclusive scan, then each pair's position in its key's list);
//      b. mla_bwd_dkv_kernel: one block of 4 waves per query; wave w owns the 32-column
//         output tiles w, w+4, .. of the 576; per chunk it contracts over all 128 heads
//         (dZ^T q and P^T dO, 32x32x16 MFMAs) and stores each selected key's fp32 row of
//         contributions (576 values) to the workspace, at the pair's (query, slot) place;
//      c. mla_bwd_dkv_reduce: one wave per key sums the rows its list names and adds the
//         sum to dkv (the only writer of that row in the sub-pass).
//      The contributions are exactly the fp32 values per-pair atomic adds into dkv would
//      carry; only the order of the additions differs (and atomics fix no order either).
#include "dsa_kernels.h"
#include "mla_gather.h"

namespace dsa {

constexpr int BWD_ROWS = 4096;  // queries per pass (bounds the workspace)
constexpr int DKV_ROWS = 2048;  // queries per dkv sub-pass (bounds the contribution rows)

// bf16 workspace elements per query of a pass: q^T and dO^T, then P and dZ per slot
__host__ __device__ constexpr int64_t bwd_ws_elems_per_row(int k) {
  return (int64_t)MDQK * MH + (int64_t)MDV * MH + 2 * (int64_t)k * MH;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the bf16 path, in order: the pass's q^T, dO^T, P and dZ (bf16); the dkv
// sub-pass's fp32 contribution rows [rows][k][576], its pair lists [rows * k] (int32) and
// the per-key list offsets [keys + 1] (uint32) over the sequences a sub-pass can span.
struct BwdWs {
  size_t contrib, perm, off, total;
};
static BwdWs bwd_ws_layout(int64_t B, int64_t n_q, int64_t n_k, int32_t k) {
  const int64_t rows = B * n_q < BWD_ROWS ? B * n_q : BWD_ROWS;
  const int64_t rs = rows < DKV_ROWS ? rows : DKV_ROWS;
  int64_t seqs = (rs + n_q - 1) / n_q + 1;
  seqs = seqs < B ? seqs : B;
  BwdWs w;
  w.contrib = align256((size_t)rows * bwd_ws_elems_per_row(k) * sizeof(uint16_t));
  w.perm = w.contrib + align256((size_t)rs * k * MDQK * sizeof(float));
  w.off = w.perm + align256((size_t)rs * k * sizeof(int32_t));
  w.total = w.off + align256((size_t)(seqs * n_k + 1) * sizeof(uint32_t));
  return w;
}

size_t sparse_mla_bwd_ws_bytes(int64_t B, int64_t n_q, int64_t n_k, int32_t k, int32_t dtype) {
  if (dtype != DSA_BF16) return 0;
  return bwd_ws_layout(B, n_q, n_k, k).total;
}

// ---------------------------------------------------------------------------------------
// 1. per-row transpose [rows][A][C] -> [rows][C][A] of bf16, 32 x 32 tiles through LDS
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_bwd_transpose(const uint16_t* __restrict__ in, int64_t in_row_stride,
                                                         uint16_t* __restrict__ out, int A, int C) {
  __shared__ uint16_t t[32][33];
  const int64_t r = blockIdx.z;
  const int a0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const uint16_t* src = in + r * in_row_stride;
  uint16_t* dst = out + r * (int64_t)A * C;
  for (int i = ty; i < 32; i += 8) {
    const int a = a0 + i, c = c0 + tx;
    if (a < A && c < C) t[i][tx] = src[(int64_t)a * C + c];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, a = a0 + tx;
    if (a < A && c < C) dst[(int64_t)c * A + a] = t[tx][i];
  }
}

// ---------------------------------------------------------------------------------------
// shared pieces
// ---------------------------------------------------------------------------------------
typedef short v4s __attribute__((ext_vector_type(4)));

// instruction classes of the scheduler's group directives
constexpr int SG_MFMA = 0x008, SG_DS_READ = 0x100;

// The row's last valid slot (every lane of every wave gets it), from all its ids loaded at
// once (k a multiple of 32, at most MAX_K); returns the number of 32-key chunks to run.
__device__ __forceinline__ int bwd_chunks(const int32_t* __restrict__ irow, int k, int64_t n_k, int l) {
  constexpr int SCAN = MAX_K / (4 * WAVE);
  int4 iv[SCAN];
#pragma unroll
  for (int it = 0; it < SCAN; ++it) iv[it] = *reinterpret_cast<const int4*>(irow + min(4 * l + 4 * WAVE * it, k - 4));
  int last = -1;
#pragma unroll
  for (int it = 0; it < SCAN; ++it) {
    const int j = 4 * l + 4 * WAVE * it;
    if (j < k) {
      if (iv[it].x >= 0 && (int64_t)iv[it].x < n_k) last = j;
      if (iv[it].y >= 0 && (int64_t)iv[it].y < n_k) last = j + 1;
      if (iv[it].z >= 0 && (int64_t)iv[it].z < n_k) last = j + 2;
      if (iv[it].w >= 0 && (int64_t)iv[it].w < n_k) last = j + 3;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) last = max(last, __shfl_xor(last, off, WAVE));
  return (__builtin_amdgcn_readfirstlane(last) + KC) / KC;
}

// The ids a wave needs to gather its part of a chunk (lane l: chunk rows 8w + l%8 and
// 8w + l/8; see gather_load), and the gather itself.
struct BwdIds {
  int32_t lat, rope;
};
__device__ __forceinline__ BwdIds bwd_ids(const int32_t* __restrict__ irow, int c, int wv, int lane) {
  const int32_t* cid = irow + c * KC + 8 * wv;
  return BwdIds{cid[lane & 7], cid[lane >> 3]};
}
__device__ __forceinline__ void bwd_gather(uint32_t buf, const uint16_t* __restrict__ kvb, const BwdIds& id,
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

__device__ __forceinline__ v8bf lds_v8bf(const uint8_t* buf, int off) {
  typedef __attribute__((address_space(3))) const v8bf lds_t;
  typedef __attribute__((address_space(3))) const uint8_t lds_u8;
  return *(lds_t*)((lds_u8*)buf + off);
}
// Transposing read (ds_read_b64_tr_b16): in a 16-lane group, lanes 4rr .. 4rr+3 supply the
// addresses of values 4qq .. 4qq+3 (qq = lane % 4) of row rr, and lane p receives value p
// of the group's 16 values for its four rows (element rr = row rr).
__device__ __forceinline__ v4s lds_tr4(const uint8_t* buf, int off) {
  typedef __attribute__((address_space(3))) v4s lds_t;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_t*)((buf + off)));
}

// Byte offset (in a chunk buffer) of the 16 values 32s + 8g .. +7 of chunk row r
// (s < 16: latent, s = 16, 17: rope).
__device__ __forceinline__ int row_unit_off(int r, int s, int g) {
  if (s < 16) return r * LAT_PITCH + 16 * ((4 * s + g) ^ lat_swz(r));
  const int u = 4 * (s - 16) + g;
  return LAT_BYTES + r * ROPE_PITCH + 16 * (u ^ rope_swz(r));
}
// Byte offset of the 4 values 16j + 4qq .. +3 of chunk row r (j < 32 latent, 32..35 rope).
__device__ __forceinline__ int row_quad_off(int r, int j, int qq) {
  if (j < 32) return r * LAT_PITCH + 16 * ((2 * j + (qq >> 1)) ^ lat_swz(r)) + 8 * (qq & 1);
  const int u = 2 * (j - 32) + (qq >> 1);
  return LAT_BYTES + r * ROPE_PITCH + 16 * (u ^ rope_swz(r)) + 8 * (qq & 1);
}

// Blocks are dispatched to the 8 XCDs round robin (block i on XCD i % 8).  This maps block
// i to a logical index so that each XCD takes one contiguous eighth of [0, n): neighbouring
// queries, which select many of the same keys, then share that XCD's L2 (for the gathered
// rows, and the q^T / dO^T rows of neighbouring queries).  Identity when n is not a
// multiple of 8.
__device__ __forceinline__ int64_t xcd_contiguous(int64_t i, int64_t n) {
  return (n & 7) ? i : (i & 7) * (n >> 3) + (i >> 3);
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// ---------------------------------------------------------------------------------------
// 2. dq, P and dZ
// ---------------------------------------------------------------------------------------
constexpr int BWD_WAVES = 4;
constexpr int DQ_TILES = MDQK / 16;  // 36 tiles of 16 dims

// grid.x = 2 * rows of the pass (query g0 + x/2, head half x%2), 256 threads.
__global__ __launch_bounds__(BWD_WAVES * 64, 1) void mla_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ o, const float* __restrict__ lse, const uint16_t* __restrict__ dout,
    int64_t n_q, int64_t n_k, int k, float scale_log2, float sm_scale, int64_t g0,
    uint16_t* __restrict__ dq, uint16_t* __restrict__ wsp, uint16_t* __restrict__ wsz) {
  __shared__ __align__(16) uint8_t buf0[CHUNK_BYTES];
  __shared__ __align__(16) uint8_t buf1[CHUNK_BYTES];

  const int tid = threadIdx.x, l = tid & 63, G = l >> 4, p = l & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t lb = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t gl = lb >> 1;           // query within the pass
  const int64_t g = g0 + gl;            // query over all sequences
  const int64_t b = g / n_q;
  const int head = 64 * (int)(lb & 1) + 16 * wv + p;
  const int32_t* irow = idx + g * k;
  const uint16_t* kvb = kv + b * n_k * MDQK;
  const uint32_t nk = (uint32_t)min(n_k, (int64_t)INT32_MAX);
  const int n = bwd_chunks(irow, k, n_k, l);

  // B operands: q (18 steps of 32 values) and dO (16 steps) of this lane's head, values
  // 32s + 8G .. +7; D_h from the same dO values and O, summed over the four lane groups
  const int64_t hrow = g * MH + head;
  v8bf Qb[18], Db[16];
  float dsum = 0.f;
#pragma unroll
  for (int s = 0; s < 18; ++s) Qb[s] = *reinterpret_cast<const v8bf*>(q + hrow * MDQK + 32 * s + 8 * G);
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    Db[s] = *reinterpret_cast<const v8bf*>(dout + hrow * MDV + 32 * s + 8 * G);
    const v8bf ob = *reinterpret_cast<const v8bf*>(o + hrow * MDV + 32 * s + 8 * G);
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf((float)Db[s][e], (float)ob[e], dsum);
  }
  dsum += __shfl_xor(dsum, 16, WAVE);
  dsum += __shfl_xor(dsum, 32, WAVE);
  const float lse2 = lse[hrow] * LOG2E;

  v4f dQt[DQ_TILES];
#pragma unroll
  for (int j = 0; j < DQ_TILES; ++j) dQt[j] = v4f{0.f, 0.f, 0.f, 0.f};

  if (n > 0) bwd_gather(lds_addr(buf0), kvb, bwd_ids(irow, 0, wv, l), nk, wv, l);
  BwdIds nxt = bwd_ids(irow, n > 1 ? 1 : 0, wv, l);
  // ids of this lane's eight keys of chunk c (rows 4G + r and 16 + 4G + r), one step ahead
  int4 kid0 = *reinterpret_cast<const int4*>(irow + 4 * G);
  int4 kid1 = *reinterpret_cast<const int4*>(irow + 16 + 4 * G);
  uint16_t* prow = wsp + gl * (int64_t)k * MH;
  uint16_t* zrow = wsz + gl * (int64_t)k * MH;

  for (int c = 0; c < n; ++c) {
    VMCNT(0);
    block_barrier();
    if (c + 1 < n) bwd_gather(lds_addr((c & 1) ? buf0 : buf1), kvb, nxt, nk, wv, l);
    if (c + 2 < n) nxt = bwd_ids(irow, c + 2, wv, l);
    const int4 cid0 = kid0, cid1 = kid1;
    if (c + 1 < n) {
      kid0 = *reinterpret_cast<const int4*>(irow + (c + 1) * KC + 4 * G);
      kid1 = *reinterpret_cast<const int4*>(irow + (c + 1) * KC + 16 + 4 * G);
    }
    const uint8_t* cur = (c & 1) ? buf1 : buf0;

    // S^T and dP^T for key tiles 0 (rows 0..15) and 1 (rows 16..31): A = the rows, read
    // KPRE steps ahead of the MFMAs (step i: tile i/18, values 32(i%18) + 8G .. +7)
    v4f S[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
    v4f dP[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
    {
      constexpr int KPRE = 8, NSTEP = 36;
      v8bf kr[KPRE];
#pragma unroll
      for (int i = 0; i < KPRE; ++i) kr[i] = lds_v8bf(cur, row_unit_off(16 * (i / 18) + p, i % 18, G));
#pragma unroll
      for (int i = 0; i < NSTEP; ++i) {
        const int kt = i / 18, s = i % 18;
        const v8bf kf = kr[i % KPRE];
        if (i + KPRE < NSTEP)
          kr[i % KPRE] = lds_v8bf(cur, row_unit_off(16 * ((i + KPRE) / 18) + p, (i + KPRE) % 18, G));
        S[kt] = mfma_bf16_16x16x32(kf, Qb[s], S[kt]);
        if (s < 16) dP[kt] = mfma_bf16_16x16x32(kf, Db[s], dP[kt]);
      }
      // keep the reads ahead: the scheduler would otherwise sink each next to its MFMAs
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, KPRE, 0);
#pragma unroll
      for (int i = 0; i < NSTEP; ++i) {
        if (i % 18 < 16) __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
        else __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        if (i + KPRE < NSTEP) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      }
    }
    // P, dZ (this lane: head `head`, keys 4G + r and 16 + 4G + r of the chunk)
    const int32_t ids8[8] = {cid0.x, cid0.y, cid0.z, cid0.w, cid1.x, cid1.y, cid1.z, cid1.w};
    float Pv[8], Zv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int kt = e >> 2, r = e & 3;
      const bool valid = ids8[e] >= 0 && (int64_t)ids8[e] < n_k;
      const float pe = valid ? __builtin_amdgcn_exp2f(__builtin_fmaf(S[kt][r], scale_log2, -lse2)) : 0.f;
      Pv[e] = pe;
      Zv[e] = pe * (dP[kt][r] - dsum);
    }
    // to the workspace ([query][slot][head], bf16; dZ scaled by sm_scale for the dkv product)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int slot = c * KC + 16 * (e >> 2) + 4 * G + (e & 3);
      prow[(int64_t)slot * MH + head] = bf16_bits(Pv[e]);
      zrow[(int64_t)slot * MH + head] = bf16_bits(Zv[e] * sm_scale);
    }
    // dq^T += K^T dZ^T: contraction slot e of lane group G is key 4G + e (e < 4) or
    // 16 + 4G + e - 4, which is where this lane's dZ values sit; the K^T operand comes from
    // two transposing reads (lanes 4rr + qq of a 16-lane group supply values 4qq .. +3 of
    // row 4G + rr, resp. 16 + 4G + rr)
    v8bf Zb;
#pragma unroll
    for (int e = 0; e < 8; ++e) Zb[e] = (__bf16)Zv[e];
    const int rr = p >> 2, qq = p & 3;
    const int r0 = 4 * G + rr, r1 = 16 + 4 * G + rr;
    {
      constexpr int TPRE = 8;  // tiles whose K^T reads run ahead of the MFMAs
      v4s tlo[TPRE], thi[TPRE];
#pragma unroll
      for (int j = 0; j < TPRE; ++j) {
        tlo[j] = lds_tr4(cur, row_quad_off(r0, j, qq));
        thi[j] = lds_tr4(cur, row_quad_off(r1, j, qq));
      }
#pragma unroll
      for (int j = 0; j < DQ_TILES; ++j) {
        const v8bf kt8 =
            __builtin_bit_cast(v8bf, __builtin_shufflevector(tlo[j % TPRE], thi[j % TPRE], 0, 1, 2, 3, 4, 5, 6, 7));
        if (j + TPRE < DQ_TILES) {
          tlo[j % TPRE] = lds_tr4(cur, row_quad_off(r0, j + TPRE, qq));
          thi[j % TPRE] = lds_tr4(cur, row_quad_off(r1, j + TPRE, qq));
        }
        dQt[j] = mfma_bf16_16x16x32(kt8, Zb, dQt[j]);
      }
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2 * TPRE, 0);
#pragma unroll
      for (int j = 0; j < DQ_TILES; ++j) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        if (j + TPRE < DQ_TILES) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 0);
      }
    }
  }
  // dq[g][head][16j + 4G + r] = sm_scale * dQt[j][r]
  uint16_t* dqh = dq + hrow * MDQK;
#pragma unroll
  for (int j = 0; j < DQ_TILES; ++j) {
    const uint32_t lo = (uint32_t)bf16_bits(dQt[j][0] * sm_scale) | ((uint32_t)bf16_bits(dQt[j][1] * sm_scale) << 16);
    const uint32_t hi = (uint32_t)bf16_bits(dQt[j][2] * sm_scale) | ((uint32_t)bf16_bits(dQt[j][3] * sm_scale) << 16);
    *reinterpret_cast<uint2*>(dqh + 16 * j + 4 * G) = uint2{lo, hi};
  }
}

// ---------------------------------------------------------------------------------------
// 3. dkv: pair lists by key, contribution rows, per-key sums
// ---------------------------------------------------------------------------------------
constexpr int DKV_WAVES = 4;
constexpr int DKV_TILES = MDQK / 32;  // 18 column tiles; tiles < 16 also take the V part
constexpr int DKV_MAXT = (DKV_TILES + DKV_WAVES - 1) / DKV_WAVES;  // 5

// 3a. Pair lists.  Row r of the sub-pass is query g0 + r (sequence b = (g0 + r) / n_q); its
// valid slot j names key b * n_k + idx - kbase of the sub-pass's key range.  Count: one
// atomic increment of that key's counter per pair.  Fill (after the scan turned the counters
// into list starts): each pair takes the next place of its key's list, which leaves off[key]
// at the start of the next key's list, i.e. at the end of its own.
template <bool FILL>
__global__ __launch_bounds__(256) void mla_bwd_pairs(const int32_t* __restrict__ idx, int64_t n_q, int64_t n_k,
                                                     int k, int64_t g0, int64_t kbase, uint32_t* __restrict__ off,
                                                     int32_t* __restrict__ perm) {
  const int64_t r = blockIdx.x;
  const int64_t g = g0 + r;
  const int64_t kb = (g / n_q) * n_k - kbase;
  const int32_t* irow = idx + g * k;
  for (int j = threadIdx.x; j < k; j += 256) {
    const int32_t id = irow[j];
    if (id < 0 || (int64_t)id >= n_k) continue;
    if constexpr (FILL) perm[atomicAdd(&off[kb + id], 1u)] = (int32_t)(r * k + j);
    else atomicAdd(&off[kb + id], 1u);
  }
}

// 3a. Exclusive prefix sum of off[0 .. n) in place, one block of 1024 threads, 4096 entries
// per step (4 consecutive per thread), the running total carried between steps.
__global__ __launch_bounds__(1024) void mla_bwd_scan(uint32_t* __restrict__ off, int64_t n) {
  __shared__ uint32_t wtot[16];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  uint32_t carry = 0;
  for (int64_t base = 0; base < n; base += 4096) {
    const int64_t i0 = base + 4 * tid;
    uint32_t v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = i0 + e < n ? off[i0 + e] : 0u;
    const uint32_t own = v[0] + v[1] + v[2] + v[3];
    const uint32_t incl = wave_incl_scan(own);
    if (lane == WAVE - 1) wtot[wv] = incl;
    __syncthreads();
    uint32_t before = carry, step = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t t = wtot[i];
      before += i < wv ? t : 0u;
      step += t;
    }
    __syncthreads();
    uint32_t run = before + incl - own;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i0 + e < n) off[i0 + e] = run;
      run += v[e];
    }
    carry += step;
  }
}

// 3b. grid.x = rows of the sub-pass, 256 threads; wave w owns column tiles w, w+4, .., < 18
// (one wave per SIMD: its q^T and dO^T operands take up to 288 registers).  The fp32
// contributions of row gl's slot j go to contrib[(gl * k + j) * 576 ..] (valid slots only).
__global__ __launch_bounds__(DKV_WAVES * 64, 1) void mla_bwd_dkv_kernel(
    const uint16_t* __restrict__ qT, const uint16_t* __restrict__ doT, const int32_t* __restrict__ idx,
    const uint16_t* __restrict__ wsp, const uint16_t* __restrict__ wsz, int64_t n_q, int64_t n_k, int k,
    int64_t g0, float* __restrict__ contrib) {
  __shared__ __align__(16) uint16_t pz[2][2][KC][MH];  // [buffer][P, dZ][slot][head]
  __shared__ int32_t sid[2][KC];

  const int tid = threadIdx.x, l = tid & 63, G = l >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t gl = xcd_contiguous(blockIdx.x, gridDim.x);
  const int64_t g = g0 + gl;
  const int32_t* irow = idx + g * k;
  const int n = bwd_chunks(irow, k, n_k, l);
  if (n == 0) return;  // uniform over the block

  // B operands (head-contiguous): q^T and dO^T columns 32j + l%32, heads 16s + 8G .. +7
  v8bf Qt[DKV_MAXT][8], Dt[DKV_MAXT - 1][8];
  const uint16_t* qTr = qT + gl * (int64_t)MDQK * MH;
  const uint16_t* dTr = doT + gl * (int64_t)MDV * MH;
#pragma unroll
  for (int t = 0; t < DKV_MAXT; ++t) {
    const int j = wv + DKV_WAVES * t;
    const int col = 32 * j + (l & 31);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      Qt[t][s] = j < DKV_TILES ? *reinterpret_cast<const v8bf*>(qTr + (int64_t)col * MH + 16 * s + 8 * G) : v8bf{};
      if (t < DKV_MAXT - 1) Dt[t][s] = *reinterpret_cast<const v8bf*>(dTr + (int64_t)col * MH + 16 * s + 8 * G);
    }
  }

  const uint16_t* prow = wsp + gl * (int64_t)k * MH;
  const uint16_t* zrow = wsz + gl * (int64_t)k * MH;
  float* crow = contrib + gl * (int64_t)k * MDQK;
  // chunk staging: thread t moves 64 bytes (32 heads) of P (t < 128) or dZ: slot (t%128)/4,
  // heads 32 (t%4) .. +31; the next chunk is loaded into registers while this one is used
  const int which = tid >> 7, u = tid & 127, srow = u >> 2, hcol = 32 * (u & 3);
  v8bf x[4];
  int32_t idv = 0;
  auto stage_load = [&](int c) {
    const uint16_t* src = (which ? zrow : prow) + (int64_t)(c * KC + srow) * MH + hcol;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = *reinterpret_cast<const v8bf*>(src + 8 * i);
    if (tid < KC) idv = irow[c * KC + tid];
  };
  auto stage_store = [&](int bi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<v8bf*>(&pz[bi][which][srow][hcol + 8 * i]) = x[i];
    if (tid < KC) sid[bi][tid] = idv;
  };
  stage_load(0);
  stage_store(0);
  for (int c = 0; c < n; ++c) {
    const int bi = c & 1;
    if (c + 1 < n) stage_load(c + 1);
    __syncthreads();  // chunk c staged; chunk c-1's buffer free
    const int32_t sid_l = sid[bi][l & 31];
    const bool sok = sid_l >= 0 && (int64_t)sid_l < n_k;  // this lane's slot holds a valid key
#pragma unroll
    for (int t = 0; t < DKV_MAXT; ++t) {
      const int j = wv + DKV_WAVES * t;
      if (j >= DKV_TILES) break;
      v16f acc = {};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const v8bf az = *reinterpret_cast<const v8bf*>(&pz[bi][1][l & 31][16 * s + 8 * G]);
        acc = mfma_bf16_32x32x16(Qt[t][s], az, acc);
      }
      if (t < DKV_MAXT - 1) {  // j < 16: the V part
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const v8bf ap = *reinterpret_cast<const v8bf*>(&pz[bi][0][l & 31][16 * s + 8 * G]);
          acc = mfma_bf16_32x32x16(Dt[t][s], ap, acc);
        }
      }
      // The columns are the product's rows and the slots its columns (q^T / dO^T as the A
      // operand, dZ / P as B; both operands have the same per-lane layout): lane l holds
      // slot l%32 of chunk c at columns 32j + 8(r/4) + 4G + r%4, so each register quad is
      // four consecutive columns, written with one 16-byte store.
      if (sok) {
        float* dst = crow + (int64_t)(c * KC + (l & 31)) * MDQK + 32 * j + 4 * G;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<v4f*>(dst + 8 * q) = v4f{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
      }
    }
    if (c + 1 < n) stage_store(bi ^ 1);
  }
}

// 3c. One wave per key of the sub-pass's range (4 per block): the sum of the contribution
// rows its list names, added to dkv[kbase + key].  Lane l holds values 4l .. 4l+3,
// 256 + 4l .. +3 and, for l < 16, 512 + 4l .. +3 of the 576; four rows are loaded at once.
__global__ __launch_bounds__(256) void mla_bwd_dkv_reduce(const float* __restrict__ contrib,
                                                          const int32_t* __restrict__ perm,
                                                          const uint32_t* __restrict__ off, int64_t n_keys,
                                                          int64_t kbase, float* __restrict__ dkv) {
  const int lane = threadIdx.x & 63;
  const int64_t key = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (key >= n_keys) return;
  const uint32_t lo = key ? off[key - 1] : 0u, hi = off[key];
  if (lo == hi) return;
  const bool third = lane < 16;
  v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0;
  for (uint32_t e0 = lo; e0 < hi; e0 += WAVE) {
    const uint32_t m = hi - e0 < (uint32_t)WAVE ? hi - e0 : (uint32_t)WAVE;
    const int32_t pl = (uint32_t)lane < m ? perm[e0 + lane] : 0;
    uint32_t j = 0;
    for (; j + 4 <= m; j += 4) {
      v4f x0[4], x1[4], x2[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t p = __builtin_amdgcn_readlane(pl, (int)(j + u));
        const v4f* row = reinterpret_cast<const v4f*>(contrib + p * MDQK);
        x0[u] = row[lane];
        x1[u] = row[64 + lane];
        x2[u] = third ? row[128 + lane] : v4f{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a0 += x0[u];
        a1 += x1[u];
        a2 += x2[u];
      }
    }
    for (; j < m; ++j) {
      const int64_t p = __builtin_amdgcn_readlane(pl, (int)j);
      const v4f* row = reinterpret_cast<const v4f*>(contrib + p * MDQK);
      a0 += row[lane];
      a1 += row[64 + lane];
      if (third) a2 += row[128 + lane];
    }
  }
  v4f* d = reinterpret_cast<v4f*>(dkv + (kbase + key) * MDQK);
  d[lane] += a0;
  d[64 + lane] += a1;
  if (third) d[128 + lane] += a2;
}

__global__ __launch_bounds__(256) void fill_zero_f32(float* __restrict__ x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = 0.f;
}

// ---------------------------------------------------------------------------------------
// fp32 path (small shapes): one block per query, one thread per head; dkv by atomics
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void mla_bwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kv, const float* __restrict__ v,
    const int32_t* __restrict__ idx, const float* __restrict__ lse, const float* __restrict__ dout, int64_t n_q,
    int64_t n_k, int H, int d_qk, int d_v, int k, float sm_scale, float* __restrict__ dq, float* __restrict__ dkv,
    float* __restrict__ dv) {
  const int b = blockIdx.y;
  const int64_t row = (int64_t)b * n_q + blockIdx.x;
  const int h = threadIdx.x;
  if (h >= H) return;
  const float* qh = q + (row * H + h) * d_qk;
  const float* doh = dout + (row * H + h) * d_v;
  const float* kvb = kv + (int64_t)b * n_k * d_qk;
  const float* vb = v ? v + (int64_t)b * n_k * d_v : kvb;
  const int64_t vstride = v ? d_v : d_qk;
  const int32_t* irow = idx + row * k;
  const float L = lse[row * H + h];
  // D_h = sum_s P dP over the valid slots
  float D = 0.f;
  for (int j = 0; j < k; ++j) {
    const int32_t s = irow[j];
    if (s < 0 || (int64_t)s >= n_k) continue;
    float z = 0.f, dp = 0.f;
    for (int d = 0; d < d_qk; ++d) z = __fmaf_rn(qh[d], kvb[(int64_t)s * d_qk + d], z);
    for (int d = 0; d < d_v; ++d) dp = __fmaf_rn(doh[d], vb[(int64_t)s * vstride + d], dp);
    D = __fmaf_rn(expf(z * sm_scale - L), dp, D);
  }
  float* dqh = dq + (row * H + h) * d_qk;
  for (int d = 0; d < d_qk; ++d) dqh[d] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int32_t s = irow[j];
    if (s < 0 || (int64_t)s >= n_k) continue;
    float z = 0.f, dp = 0.f;
    for (int d = 0; d < d_qk; ++d) z = __fmaf_rn(qh[d], kvb[(int64_t)s * d_qk + d], z);
    for (int d = 0; d < d_v; ++d) dp = __fmaf_rn(doh[d], vb[(int64_t)s * vstride + d], dp);
    const float P = expf(z * sm_scale - L);
    const float dz = P * (dp - D) * sm_scale;
    float* dks = dkv + ((int64_t)b * n_k + s) * d_qk;
    for (int d = 0; d < d_qk; ++d) {
      dqh[d] = __fmaf_rn(dz, kvb[(int64_t)s * d_qk + d], dqh[d]);
      unsafeAtomicAdd(dks + d, dz * qh[d]);
    }
    float* dvs = v ? dv + ((int64_t)b * n_k + s) * d_v : dks;
    for (int d = 0; d < d_v; ++d) unsafeAtomicAdd(dvs + d, P * doh[d]);
  }
}

hipError_t launch_sparse_mla_bwd(const MlaBwdArgs& a, hipStream_t st) {
  const int64_t rows = a.B * a.n_q;
  const int64_t n_kv = a.B * a.n_k * a.d_qk;
  const unsigned zb = (unsigned)((n_kv + 255) / 256 < 65536 ? (n_kv + 255) / 256 : 65536);
  hipLaunchKernelGGL(fill_zero_f32, dim3(zb), dim3(256), 0, st, a.dkv, n_kv);
  if (a.dtype == DSA_F32) {
    if (a.v) {
      const int64_t n_v = a.B * a.n_k * a.d_v;
      const unsigned vb = (unsigned)((n_v + 255) / 256 < 65536 ? (n_v + 255) / 256 : 65536);
      hipLaunchKernelGGL(fill_zero_f32, dim3(vb), dim3(256), 0, st, a.dv, n_v);
    }
    hipLaunchKernelGGL(mla_bwd_f32_kernel, dim3((unsigned)a.n_q, (unsigned)a.B), dim3(64), 0, st,
                       (const float*)a.q, (const float*)a.kv, (const float*)a.v, a.idx, a.lse,
                       (const float*)a.dout, a.n_q, a.n_k, a.H, a.d_qk, a.d_v, a.k, a.sm_scale, (float*)a.dq,
                       a.dkv, a.dv);
    return hipGetLastError();
  }
  uint16_t* ws = (uint16_t*)a.ws;
  const BwdWs wl = bwd_ws_layout(a.B, a.n_q, a.n_k, a.k);
  float* contrib = (float*)((char*)a.ws + wl.contrib);
  int32_t* perm = (int32_t*)((char*)a.ws + wl.perm);
  uint32_t* off = (uint32_t*)((char*)a.ws + wl.off);
  for (int64_t g0 = 0; g0 < rows; g0 += BWD_ROWS) {
    const int64_t R = rows - g0 < BWD_ROWS ? rows - g0 : BWD_ROWS;
    uint16_t* qT = ws;
    uint16_t* dT = qT + R * (int64_t)MDQK * MH;
    uint16_t* wp = dT + R * (int64_t)MDV * MH;
    uint16_t* wz = wp + R * (int64_t)a.k * MH;
    hipLaunchKernelGGL(mla_bwd_transpose, dim3(MDQK / 32, MH / 32, (unsigned)R), dim3(256), 0, st,
                       (const uint16_t*)a.q + g0 * MH * MDQK, (int64_t)MH * MDQK, qT, MH, MDQK);
    hipLaunchKernelGGL(mla_bwd_transpose, dim3(MDV / 32, MH / 32, (unsigned)R), dim3(256), 0, st,
                       (const uint16_t*)a.dout + g0 * MH * MDV, (int64_t)MH * MDV, dT, MH, MDV);
    hipLaunchKernelGGL(mla_bwd_dq_kernel, dim3((unsigned)(2 * R)), dim3(BWD_WAVES * 64), 0, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.kv, a.idx, (const uint16_t*)a.out, a.lse,
                       (const uint16_t*)a.dout, a.n_q, a.n_k, a.k, a.sm_scale * LOG2E, a.sm_scale, g0,
                       (uint16_t*)a.dq, wp, wz);
    for (int64_t s0 = 0; s0 < R; s0 += DKV_ROWS) {
      const int64_t Rs = R - s0 < DKV_ROWS ? R - s0 : DKV_ROWS;
      const int64_t gs = g0 + s0;
      // keys of the sequences rows gs .. gs + Rs - 1 belong to
      const int64_t b_lo = gs / a.n_q, b_hi = (gs + Rs - 1) / a.n_q;
      const int64_t kbase = b_lo * a.n_k, n_keys = (b_hi - b_lo + 1) * a.n_k;
      hipLaunchKernelGGL(fill_zero_f32, dim3((unsigned)((n_keys + 1 + 255) / 256 < 65536 ? (n_keys + 1 + 255) / 256
                                                                                           : 65536)),
                         dim3(256), 0, st, (float*)off, n_keys + 1);
      hipLaunchKernelGGL(mla_bwd_pairs<false>, dim3((unsigned)Rs), dim3(256), 0, st, a.idx, a.n_q, a.n_k, a.k, gs,
                         kbase, off, perm);
      hipLaunchKernelGGL(mla_bwd_scan, dim3(1), dim3(1024), 0, st, off, n_keys + 1);
      hipLaunchKernelGGL(mla_bwd_pairs<true>, dim3((unsigned)Rs), dim3(256), 0, st, a.idx, a.n_q, a.n_k, a.k, gs,
                         kbase, off, perm);
      hipLaunchKernelGGL(mla_bwd_dkv_kernel, dim3((unsigned)Rs), dim3(DKV_WAVES * 64), 0, st,
                         qT + s0 * (int64_t)MDQK * MH, dT + s0 * (int64_t)MDV * MH, a.idx, wp + s0 * (int64_t)a.k * MH,
                         wz + s0 * (int64_t)a.k * MH, a.n_q, a.n_k, a.k, gs, contrib);
      hipLaunchKernelGGL(mla_bwd_dkv_reduce, dim3((unsigned)((n_keys + 3) / 4)), dim3(256), 0, st, contrib, perm, off,
                         n_keys, kbase, a.dkv);
    }
  }
  return hipGetLastError();
}

}  // namespace dsa
