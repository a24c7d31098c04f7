// Attention over the selected keys, MLA in MQA mode (dsa_sparse_mla, prefill, decode).
//
// Every query head attends over the same selected latent rows: one key-value row of
// 576 values serves all 128 heads, and V is its first 512 values (MQA mode of MLA:
// 53ai.com V3.2-Exp summary, section 创新架构 and Figure 1; paperbridge.wiki summary,
// section DeepSeek Sparse Attention).  Attention is computed only over the k kept keys,
// so its cost per query is O(k) (same sections).
//
// bf16 kernel (H = 128, d_qk = 576, d_v = 512), one block of 8 waves per query:
//   * waves 2h and 2h+1 share heads 32h .. +31.  The even wave forms the partial logits
//     S^T = K Q^T over values 0..287 of each row, the odd one over values 288..575; the
//     two exchange partials through LDS and add them in the same order, so both hold the
//     same S.  Each then keeps the softmax state of its 32 heads and accumulates
//     O^T = V^T P^T for its half of the 512 output values.  Per wave: Q^T operands 72
//     registers, O^T accumulators 128, so two waves share a SIMD, and those two (w, w+4)
//     run half a chunk apart;
//   * 32x32x16 bf16 MFMAs: S^T is one 32 keys x 32 heads tile; O^T is 8 tiles of 32
//     values x 32 heads;
//   * keys are processed in chunks of 32 gathered rows.  The rows go straight from HBM to
//     LDS with 16-byte direct loads (no staging registers; the latent half of a row is one
//     wave-wide 1 KB load from a scalar address) into a ring of three buffers, so two
//     chunks are in flight while one is computed;
//   * after the softmax each lane already holds P^T in the B-operand layout of the PV
//     product; V^T is read from the same row-major rows with the gfx950 transposing LDS
//     read, so no transposed copy is stored;
//   * fp32 online softmax in base 2 whose reference max moves only when a logit exceeds
//     it by 8 (P then stays <= 256, exact enough in bf16), which keeps the rescale of the
//     accumulators off the common path.
// Keys may be split over several blocks (decode): each writes a normalised partial O and
// its lse, and a combine kernel merges them.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int MH = 128, MDQK = 576, MDV = 512, KC = 32;
// LDS image of one chunk of 32 gathered rows, in two regions (every LDS read is a per-lane
// base plus an immediate offset):
//   latent: values 0..511 of each row, rows 1088 B apart (16 banks past a multiple of 64
//     banks), and within row r the 16-byte unit u is stored at unit u ^ ((r >> 2) & 3).
//     Both read patterns are then free of bank conflicts: the K operand (one unit of 16
//     rows per pass) and the transposed V operand (4 consecutive rows x 4 units per pass);
//   rope:   values 512..575 of each row, 144 B apart (128 B + one unused unit).
constexpr int LAT_PITCH = 1088, ROPE_PITCH = 144;
constexpr int LAT_BYTES = KC * LAT_PITCH;                      // 34816
constexpr int ROPE_UNITS = KC * ROPE_PITCH / 16;               // 288
constexpr int ROPE_INSTR = (ROPE_UNITS + 63) / 64;             // 5
constexpr int CHUNK_BYTES = LAT_BYTES + ROPE_INSTR * 64 * 16;  // 34816 + 5120 = 39936
__device__ __forceinline__ int lat_swz(int r) { return (r >> 2) & 3; }
constexpr int MLA_WAVES = 8;
constexpr int HALF_STEPS = MDQK / 2 / 16;                      // 18 d-steps of 16 per half
constexpr int MAX_K = 2048;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_SLACK = 8.f;              // log2 units the running max may lag

typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));

#define VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
#define LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

// D = A(32x16 bf16) * B(16x32 bf16) + C, fp32.  Lane l: row (A) / column (B) l%32,
// contraction elements 8*(l/32) .. +7; C/D: column l%32, register r holds row
// 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ v16f mfma_bf16_32x32x16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// instruction classes for the scheduler's interleave directives
constexpr int SG_MFMA = 0x008, SG_DS_READ = 0x100;

// two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// The value itself, opaque to the optimiser: keeps lane offsets from being computed once
// and held across the chunk loop (they would not fit in registers beside the Q^T operands
// and the accumulators); recomputing them costs a few VALU ops per chunk.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ int64_t safe_row(int32_t s, int64_t n_k) {
  return (s >= 0 && s < n_k) ? (int64_t)s : 0;
}

// Issue this wave's direct global->LDS loads for chunk c (rows ids[32c .. 32c+31]): the
// latent halves of rows 4w .. 4w+3 (one wave-wide 1 KB load each, scalar row address)
// and, for w < 5, rope instruction w, whose lane loads unit u = 64w + lane: row u / 9,
// 16-byte unit u % 9 of the row's rope part (unit 8 is the pitch padding and loads a
// harmless copy).  Waves 0-4 issue 5 loads, waves 5-7 issue 4.
__device__ __forceinline__ void gather_chunk(uint8_t* buf, const uint16_t* __restrict__ kvb,
                                             const int32_t* ids, int c, int64_t n_k, int wv, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * wv + j;
    const int64_t row = safe_row(__builtin_amdgcn_readfirstlane(ids[c * KC + r]), n_k);
    // LDS unit `lane` of the row holds the row's unit lane ^ swz
    __builtin_amdgcn_global_load_lds(kvb + row * MDQK + 8 * (lane ^ lat_swz(r)), buf + r * LAT_PITCH, 16, 0, 0);
  }
  if (wv < ROPE_INSTR) {
    const int u = opaque(wv * 64 + lane);
    const int rope_r = min(u / 9, KC - 1);
    const int rope_e = 512 + 8 * ((u % 9) & 7);
    const int64_t row = safe_row(ids[c * KC + rope_r], n_k);
    __builtin_amdgcn_global_load_lds(kvb + row * MDQK + rope_e, buf + LAT_BYTES + wv * 1024, 16, 0, 0);
  }
}

// A operand of S^T for d-step ds (values 16ds .. 16ds+15): row = key r = l%32, elements
// 16ds + 8(l/32) .. +7, i.e. logical unit 2ds + g of the row (g = l/32), stored at unit
// (2ds + g) ^ swz(r).  As the swizzle only flips the two low unit bits, that is
// 2ds + ((g ^ swz) & 1) + (swz & 2) for even ds and 2ds + ((g ^ swz) & 1) - (swz & 2) for
// odd ds: `lat_e` / `lat_o` are this lane's byte offsets of those two cases at ds = 0, so
// the step offsets 32ds are compile-time constants that fold into the LDS read's
// immediate.  `rope` = this lane's offset of step 32 in the rope region.
__device__ __forceinline__ v8bf krow_frag(const uint8_t* buf, int lat_e, int lat_o, int rope, int ds) {
  const uint8_t* p = ds < 32 ? buf + ((ds & 1) ? lat_o : lat_e) + 32 * ds : buf + rope + 32 * (ds - 32);
  return *reinterpret_cast<const v8bf*>(p);
}

// A operand of O^T = V^T P^T for latent values d0 .. d0+31 (rows) and key step s: the
// contraction slots j of lane group g = l/32 are keys 16s + 4g + 8(j/4) + j%4, the keys
// whose probabilities that lane holds in P^T slot j.  The gfx950 transposing LDS read does
// the transpose: in a 16-lane group, lanes 4rr..4rr+3 supply 16 values of one key and lane
// p receives value p of the group's 16 values for four keys.
// Lane (G = l/16, p = l%16, rr = p/4, qq = p%4) reads row 16s + 4(G/2) + rr (first read;
// second read: 8 rows further), values d0 + 16(G%2) + 4qq .. +3 = logical unit
// 32 half + 4t + 2(G%2) + qq/2, bytes 8(qq%2) within it.  The row's swizzle is G/2 (first
// read) or G/2 + 2 (second read) for every s, and it only flips the unit's two low bits,
// so `vt0` / `vt1` (byte offsets at s = 0, t = 0) plus the constants 16 s LAT_PITCH + 64 t
// address every fragment.
__device__ __forceinline__ int vt_lane_offset(int half, int second) {
  const int l = lane_id();
  const int p = l & 15, G = l >> 4;
  const int rr = p >> 2, qq = p & 3;
  const int row = 4 * (G >> 1) + rr + 8 * second;
  const int unit = 32 * half + ((2 * (G & 1) + (qq >> 1)) ^ lat_swz(row));
  return row * LAT_PITCH + 16 * unit + 8 * (qq & 1);
}
__device__ __forceinline__ v8bf vt_frag(const uint8_t* buf, int vt0, int vt1, int t, int s) {
  typedef __attribute__((address_space(3))) v4s* lds_v4s;
  const uint8_t* a0 = buf + vt0 + 16 * s * LAT_PITCH + 64 * t;
  const uint8_t* a1 = buf + vt1 + 16 * s * LAT_PITCH + 64 * t;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(__attribute__((address_space(3))) uint8_t*)a0);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(__attribute__((address_space(3))) uint8_t*)a1);
  const v8s v = v8s{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(v8bf, v);
}

struct MlaState {
  v8bf Qt[HALF_STEPS];  // B operands of S^T for this wave's 288 values
  v16f O[8];            // O^T tiles: values 256*half + 32t + row, head l%32
  float m_ref, l_run;   // softmax state of head l%32 (the same in both lane halves)
};

// Partial-logit exchange between the two waves of a head group: [wave][4][64 lanes][4].
__shared__ __align__(16) float s_xch[MLA_WAVES][4][64][4];

// Phase 1 of a chunk: this wave's partial logits S^T over its 288 values, left in its
// exchange slot.
__device__ __forceinline__ void mla_logits(const MlaState& st, const uint8_t* buf, int wv, int half) {
  // lane offsets recomputed per chunk (a few VALU ops) rather than held across the loop
  const int l = opaque(lane_id());
  const int r = l & 31, g = l >> 5;
  const int swz = lat_swz(r);
  const int lat_e = r * LAT_PITCH + 16 * (((g ^ swz) & 1) + (swz & 2));
  const int lat_o = r * LAT_PITCH + 16 * (((g ^ swz) & 1) - (swz & 2));
  const int rope = LAT_BYTES + r * ROPE_PITCH + 16 * g;
  v16f S = {};
  // each K fragment read is issued one step ahead of the MFMA that uses it
  if (half == 0) {
#pragma unroll
    for (int j = 0; j < HALF_STEPS; ++j) S = mfma_bf16_32x32x16(krow_frag(buf, lat_e, lat_o, rope, j), st.Qt[j], S);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
#pragma unroll
    for (int j = 0; j < HALF_STEPS - 1; ++j) {
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
  } else {
#pragma unroll
    for (int j = 0; j < HALF_STEPS; ++j)
      S = mfma_bf16_32x32x16(krow_frag(buf, lat_e, lat_o, rope, HALF_STEPS + j), st.Qt[j], S);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
#pragma unroll
    for (int j = 0; j < HALF_STEPS - 1; ++j) {
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<float4*>(&s_xch[wv][q][l][0]) = make_float4(S[4 * q], S[4 * q + 1], S[4 * q + 2], S[4 * q + 3]);
}

// Phase 2 of a chunk (after a barrier): S = S(values 0..287) + S(values 288..575) read
// from the two exchange slots in that order (so both waves hold the same bits), online
// softmax (base 2, lazily rescaled), O^T += V^T P^T.
__device__ __forceinline__ void mla_update(MlaState& st, const uint8_t* buf, uint32_t vmask, float scale_log2,
                                           int wv, int half) {
  const int l = lane_id(), g = l >> 5;
  const int vt0 = opaque(vt_lane_offset(half, 0)), vt1 = opaque(vt_lane_offset(half, 1));
  v16f S;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 a = *reinterpret_cast<const float4*>(&s_xch[wv & ~1][q][l][0]);
    const float4 o = *reinterpret_cast<const float4*>(&s_xch[wv | 1][q][l][0]);
    S[4 * q] = a.x + o.x;
    S[4 * q + 1] = a.y + o.y;
    S[4 * q + 2] = a.z + o.z;
    S[4 * q + 3] = a.w + o.w;
  }
  // lane holds head l%32 and keys 8(r/4) + 4g + r%4; S becomes the base-2 logits
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const bool ok = (vmask >> (8 * (r >> 2) + 4 * g + (r & 3))) & 1u;
    S[r] = ok ? S[r] * scale_log2 : -INFINITY;
    mx = fmaxf(mx, S[r]);
  }
  mx = fmaxf(mx, xor32(mx));
  // move the reference max only when a logit exceeds it by more than the slack
  if (ballot(mx > st.m_ref + RESCALE_SLACK)) {
    const float m_new = fmaxf(st.m_ref, mx);
    const float alpha = st.m_ref == -INFINITY ? 0.f : exp2f(st.m_ref - m_new);
    st.l_run *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.O[t] *= alpha;
    st.m_ref = m_new;
  }
  // m is finite once any key of the row was valid; before that every logit is -inf and
  // m = -inf, so use 0 as the offset (exp2(-inf) = 0 either way)
  const float m = st.m_ref == -INFINITY ? 0.f : st.m_ref;
  float ps = 0.f;
  uint32_t pk[8];
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float p0 = __builtin_amdgcn_exp2f(S[r] - m);
    const float p1 = __builtin_amdgcn_exp2f(S[r + 1] - m);
    ps += p0 + p1;
    pk[r >> 1] = cvt_pk_bf16(p0, p1);
  }
  ps += xor32(ps);
  st.l_run += ps;
  // P^T for key step s = slots 8s .. 8s+7 (keys 16s + 4g + 8(j/4) + j%4)
  const v8bf P0 = __builtin_bit_cast(v8bf, v4i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]});
  const v8bf P1 = __builtin_bit_cast(v8bf, v4i{(int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]});
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    st.O[t] = mfma_bf16_32x32x16(vt_frag(buf, vt0, vt1, t, 0), P0, st.O[t]);
    st.O[t] = mfma_bf16_32x32x16(vt_frag(buf, vt0, vt1, t, 1), P1, st.O[t]);
  }
  // V fragment reads (two per MFMA) run one MFMA ahead
  __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 1);
#pragma unroll
  for (int j = 0; j < 15; ++j) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 1);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 2, 1);
  }
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 1);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ uint32_t chunk_mask(const int32_t* ids, int c, int64_t n_k) {
  const int32_t s = ids[c * KC + (lane_id() & 31)];
  return (uint32_t)ballot(s >= 0 && s < n_k);
}

// grid.x = n_q * n_split, grid.y = B.  Pipeline: chunk c+1 is in flight while chunk c is
// computed, and chunk c+2's loads are issued right after (3 LDS buffers, loop unrolled by 3
// so each buffer is a distinct static array).
__global__ __launch_bounds__(MLA_WAVES * 64, 1) void sparse_mla_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    int64_t n_q, int64_t n_k, int k, float scale_log2, int n_split, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __align__(16) uint8_t buf0[CHUNK_BYTES];
  __shared__ __align__(16) uint8_t buf1[CHUNK_BYTES];
  __shared__ __align__(16) uint8_t buf2[CHUNK_BYTES];
  __shared__ int32_t ids[MAX_K];
  __shared__ int32_t s_last[MLA_WAVES];

  const int tid = threadIdx.x, l = tid & 63, g = l >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in scalar registers
  const bool grp_x = wv < 4;
  const int hg = wv >> 1, half = wv & 1;  // head group (heads 32hg..), value half of the pair
  const int b = blockIdx.y;
  const int64_t qi = blockIdx.x / n_split;
  const int split = blockIdx.x % n_split;
  const int64_t qrow = (int64_t)b * n_q + qi;
  const int32_t* irow = idx + qrow * k;
  const uint16_t* kvb = kv + (int64_t)b * n_k * MDQK;
  const int head = 32 * hg + (l & 31);

  MlaState st;
  const uint16_t* qh = q + (qrow * MH + head) * MDQK + 288 * half + 8 * g;
#pragma unroll
  for (int j = 0; j < HALF_STEPS; ++j) st.Qt[j] = *reinterpret_cast<const v8bf*>(qh + 16 * j);

  // the row's selected ids -> LDS; chunks up to the last valid id
  int last = -1;
  for (int j = tid; j < k; j += MLA_WAVES * 64) {
    const int32_t s = irow[j];
    ids[j] = s;
    if (s >= 0 && s < n_k) last = j;
  }
  last = (int)wave_max((float)last);
  if (l == 0) s_last[wv] = last;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < MLA_WAVES; ++w) last = max(last, s_last[w]);
  const int nchunks = (last + KC) / KC;
  const int c_lo = (int)((int64_t)nchunks * split / n_split);
  const int c_hi = (int)((int64_t)nchunks * (split + 1) / n_split);

#pragma unroll
  for (int t = 0; t < 8; ++t) st.O[t] = v16f{};
  st.m_ref = -INFINITY;
  st.l_run = 0.f;

  uint8_t* bufs[3] = {buf0, buf1, buf2};
  const int n = c_hi - c_lo;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (j < n) gather_chunk(bufs[j], kvb, ids, c_lo + j, n_k, wv, l);

  // Chunk periods p = 0..n, each split by two barriers.  Waves 0-3 (group X) form chunk
  // p's logits in the first half and finish chunk p in the second; waves 4-7 (group Y)
  // finish chunk p-1 in the first half and form chunk p's logits in the second.  The two
  // waves of a SIMD (w, w+4) are in different groups, so one's softmax and fragment reads
  // run while the other's MFMAs keep the matrix core busy.
  // the two groups run the same barriers in separate loops (one ordering each keeps the
  // register allocation of the two orderings apart)
#define MLA_WAIT_CHUNK(p)                   \
  if (wv < ROPE_INSTR) {                    \
    if ((p) + 1 < n) VMCNT(5);              \
    else VMCNT(0);                          \
  } else {                                  \
    if ((p) + 1 < n) VMCNT(4);              \
    else VMCNT(0);                          \
  }                                         \
  LGKM0();                                  \
  __builtin_amdgcn_s_barrier()
  if (grp_x) {
    for (int base = 0; base <= n; base += 3) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int p = base + j;
        if (p <= n) {
          MLA_WAIT_CHUNK(p);
          if (p < n) mla_logits(st, bufs[j], wv, half);
          LGKM0();
          __builtin_amdgcn_s_barrier();
          if (p + 2 < n) gather_chunk(bufs[(j + 2) % 3], kvb, ids, c_lo + p + 2, n_k, wv, l);
          if (p < n) mla_update(st, bufs[j], chunk_mask(ids, c_lo + p, n_k), scale_log2, wv, half);
        }
      }
    }
  } else {
    for (int base = 0; base <= n; base += 3) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int p = base + j;
        if (p <= n) {
          MLA_WAIT_CHUNK(p);
          if (p >= 1)
            mla_update(st, bufs[(j + 2) % 3], chunk_mask(ids, c_lo + p - 1, n_k), scale_log2, wv, half);
          LGKM0();
          __builtin_amdgcn_s_barrier();
          if (p + 2 < n) gather_chunk(bufs[(j + 2) % 3], kvb, ids, c_lo + p + 2, n_k, wv, l);
          if (p < n) mla_logits(st, bufs[j], wv, half);
        }
      }
    }
  }
#undef MLA_WAIT_CHUNK

  // ---- epilogue: lane holds head 32hg + l%32, values 256 half + 32t + 8(r/4) + 4g + r%4
  // (addresses recomputed here rather than kept from the prologue across the loop)
  const int le = opaque(l);
  const int ge = le >> 5;
  const int64_t row_head = ((int64_t)b * n_q + qi) * MH + 32 * hg + (le & 31);
  const bool nonempty = st.l_run > 0.f;
  const float inv = nonempty ? 1.f / st.l_run : 0.f;
  const float lse_v = nonempty ? (st.m_ref + log2f(st.l_run)) * LN2 : -INFINITY;
  if (n_split == 1) {
    uint16_t* orow = out + row_head * MDV + 256 * half + 4 * ge;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 pkd;
        pkd.x = pack_bf16x2(st.O[t][4 * i] * inv, st.O[t][4 * i + 1] * inv);
        pkd.y = pack_bf16x2(st.O[t][4 * i + 2] * inv, st.O[t][4 * i + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * t + 8 * i) = pkd;
      }
    if (lse && half == 0 && ge == 0) lse[row_head] = lse_v;
  } else {
    const int64_t prh = (((int64_t)b * n_q + qi) * n_split + split) * MH + 32 * hg + (le & 31);
    float* prow = part_o + prh * MDV + 256 * half + 4 * ge;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<v4f*>(prow + 32 * t + 8 * i) =
            v4f{st.O[t][4 * i], st.O[t][4 * i + 1], st.O[t][4 * i + 2], st.O[t][4 * i + 3]} * inv;
    if (half == 0 && ge == 0) part_lse[prh] = lse_v;
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
  if (blocks >= 256) return 1;
  const int64_t chunks = (k + KC - 1) / KC;
  int64_t s = (256 + blocks - 1) / blocks;
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
  hipLaunchKernelGGL(sparse_mla_bf16_kernel, grid, dim3(MLA_WAVES * 64), 0, st, (const uint16_t*)a.q,
                     (const uint16_t*)a.kv, a.idx, a.n_q, a.n_k, a.k, a.sm_scale * LOG2E, s,
                     (uint16_t*)a.out, a.lse, part_o, part_lse);
  if (s > 1)
    hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)(a.B * a.n_q * a.H)), dim3(128), 0, st, part_o,
                       part_lse, s, a.H, a.d_v, (uint16_t*)a.out, a.lse);
  return hipGetLastError();
}

}  // namespace dsa
