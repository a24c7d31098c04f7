// Attention over the selected keys, MLA in MQA mode (dsa_sparse_mla, prefill, decode).
//
// Every query head attends over the same selected latent rows: one key-value row of
// 576 values serves all 128 heads, and V is its first 512 values (MQA mode of MLA:
// 53ai.com V3.2-Exp summary, section 创新架构 and Figure 1; paperbridge.wiki summary,
// section DeepSeek Sparse Attention).  Attention is computed only over the k kept keys,
// so its cost per query is O(k) (same sections).
//
// bf16 kernel (H = 128, d_qk = 576, d_v = 512), one block of 4 waves per query:
//   * wave w owns heads 32w .. 32w+31 over all 576 values of S^T = K Q^T (one 32 keys x 32
//     heads tile, 36 MFMAs of 32x32x16 per chunk) and all 512 values of O^T = V^T P^T
//     (16 tiles, 32 MFMAs per chunk).  Its Q^T operands take 144 vector registers and its
//     O^T accumulators all 256 accumulation registers, so one wave runs per SIMD and no
//     wave exchanges partial results with another;
//   * keys are processed in chunks of 32 gathered rows.  The rows go straight from HBM to
//     LDS with 16-byte direct loads (no staging registers; the latent half of a row is one
//     wave-wide 1 KB load from a scalar address) into a ring of four buffers: while chunk c
//     is finished, chunk c+2 is in flight (a third chunk in flight measured slower);
//   * per chunk, the logits of chunk c+1 are formed while the softmax of chunk c runs on
//     the VALU between those MFMAs, then O^T += V^T P^T for chunk c;
//   * after the softmax each lane already holds P^T in the B-operand layout of the PV
//     product; V^T is read from the same row-major rows with the gfx950 transposing LDS
//     read, so no transposed copy is stored;
//   * fp32 online softmax in base 2 whose reference max moves only when a logit exceeds
//     it by 8 (P then stays <= 256), which keeps the rescale of the accumulators off the
//     common path.  P enters the PV product rounded to bf16; O is divided by the sum of
//     those rounded weights (lse by the fp32 sum), so a dominant key's rounding cancels.
// Keys may be split over several blocks (decode): each writes a normalised partial O and
// its lse, and a combine kernel merges them.
#include "dsa_kernels.h"
#include "mla_gather.h"

namespace dsa {

constexpr int NBUF = 4;       // chunk buffers (4 x 38912 B)
constexpr int MLA_WAVES = 4;
constexpr int KRING = 4;      // K fragments read ahead of the logit MFMAs
constexpr int O_TILES = MDV / 32;   // 16 O^T tiles per wave
constexpr float RESCALE_SLACK = 8.f;  // log2 units the running max may lag

typedef short v4s __attribute__((ext_vector_type(4)));

// O^T += V^T P^T for one chunk: 32 MFMAs (key step s = i/16, value tile t = i%16) with the
// accumulator tiles pinned in the accumulation registers (a[]): the 16 O^T tiles of a
// wave take all 256 of them, leaving the 256 vector registers for the Q^T operands, the
// logits and the fragments.  Written as one block so that the V^T fragments (two
// transposing reads each, into the four staging quads v240..v255) run three MFMAs ahead
// with exact LDS counter waits.  The matrix core forwards an accumulator to the next MFMA
// on the same tile without wait states; P^T and the tiles were last written by the VALU at
// least the 7 instructions of the block's head earlier (2 wait states are required).
// `va` / `vb`: LDS byte addresses of this lane's first / second read of fragment 0.
__device__ __forceinline__ void pv_chunk(v16f* O, v8bf P0, v8bf P1, uint32_t va, uint32_t vb) {
  asm volatile(
      "ds_read_b64_tr_b16 v[240:241], %[va] offset:0\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[vb] offset:0\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[va] offset:64\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[vb] offset:64\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[va] offset:128\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[vb] offset:128\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o0], v[240:243], %[p0], %[o0]\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[va] offset:192\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[vb] offset:192\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o1], v[244:247], %[p0], %[o1]\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[va] offset:256\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[vb] offset:256\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o2], v[248:251], %[p0], %[o2]\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[va] offset:320\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[vb] offset:320\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o3], v[252:255], %[p0], %[o3]\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[va] offset:384\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[vb] offset:384\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o4], v[240:243], %[p0], %[o4]\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[va] offset:448\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[vb] offset:448\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o5], v[244:247], %[p0], %[o5]\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[va] offset:512\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[vb] offset:512\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o6], v[248:251], %[p0], %[o6]\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[va] offset:576\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[vb] offset:576\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o7], v[252:255], %[p0], %[o7]\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[va] offset:640\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[vb] offset:640\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o8], v[240:243], %[p0], %[o8]\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[va] offset:704\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[vb] offset:704\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o9], v[244:247], %[p0], %[o9]\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[va] offset:768\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[vb] offset:768\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o10], v[248:251], %[p0], %[o10]\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[va] offset:832\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[vb] offset:832\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o11], v[252:255], %[p0], %[o11]\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[va] offset:896\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[vb] offset:896\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o12], v[240:243], %[p0], %[o12]\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[va] offset:960\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[vb] offset:960\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o13], v[244:247], %[p0], %[o13]\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[va] offset:17408\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[vb] offset:17408\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o14], v[248:251], %[p0], %[o14]\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[va] offset:17472\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[vb] offset:17472\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o15], v[252:255], %[p0], %[o15]\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[va] offset:17536\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[vb] offset:17536\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o0], v[240:243], %[p1], %[o0]\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[va] offset:17600\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[vb] offset:17600\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o1], v[244:247], %[p1], %[o1]\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[va] offset:17664\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[vb] offset:17664\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o2], v[248:251], %[p1], %[o2]\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[va] offset:17728\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[vb] offset:17728\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o3], v[252:255], %[p1], %[o3]\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[va] offset:17792\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[vb] offset:17792\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o4], v[240:243], %[p1], %[o4]\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[va] offset:17856\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[vb] offset:17856\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o5], v[244:247], %[p1], %[o5]\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[va] offset:17920\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[vb] offset:17920\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o6], v[248:251], %[p1], %[o6]\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[va] offset:17984\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[vb] offset:17984\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o7], v[252:255], %[p1], %[o7]\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[va] offset:18048\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[vb] offset:18048\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o8], v[240:243], %[p1], %[o8]\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[va] offset:18112\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[vb] offset:18112\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o9], v[244:247], %[p1], %[o9]\n\t"
      "ds_read_b64_tr_b16 v[240:241], %[va] offset:18176\n\t"
      "ds_read_b64_tr_b16 v[242:243], %[vb] offset:18176\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o10], v[248:251], %[p1], %[o10]\n\t"
      "ds_read_b64_tr_b16 v[244:245], %[va] offset:18240\n\t"
      "ds_read_b64_tr_b16 v[246:247], %[vb] offset:18240\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o11], v[252:255], %[p1], %[o11]\n\t"
      "ds_read_b64_tr_b16 v[248:249], %[va] offset:18304\n\t"
      "ds_read_b64_tr_b16 v[250:251], %[vb] offset:18304\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o12], v[240:243], %[p1], %[o12]\n\t"
      "ds_read_b64_tr_b16 v[252:253], %[va] offset:18368\n\t"
      "ds_read_b64_tr_b16 v[254:255], %[vb] offset:18368\n\t"
      "s_waitcnt lgkmcnt(4)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o13], v[244:247], %[p1], %[o13]\n\t"
      "s_waitcnt lgkmcnt(2)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o14], v[248:251], %[p1], %[o14]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "v_mfma_f32_32x32x16_bf16 %[o15], v[252:255], %[p1], %[o15]\n\t"
      : [o0] "+a"(O[0]), [o1] "+a"(O[1]), [o2] "+a"(O[2]), [o3] "+a"(O[3]), [o4] "+a"(O[4]),
        [o5] "+a"(O[5]), [o6] "+a"(O[6]), [o7] "+a"(O[7]), [o8] "+a"(O[8]), [o9] "+a"(O[9]),
        [o10] "+a"(O[10]), [o11] "+a"(O[11]), [o12] "+a"(O[12]), [o13] "+a"(O[13]), [o14] "+a"(O[14]),
        [o15] "+a"(O[15])
      : [p0] "v"(P0), [p1] "v"(P1), [va] "v"(va), [vb] "v"(vb)
      : "memory", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250",
        "v251", "v252", "v253", "v254", "v255");
}

// Orders every access to the O^T tiles after the last MFMA issued on them and before the
// next: 20 wait states cover an MFMA result read or overwritten by the VALU (and the
// VALU-write-then-MFMA-read case), whatever the pass count.
__device__ __forceinline__ void o_guard(v16f* O) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
               : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]), "+a"(O[4]), "+a"(O[5]), "+a"(O[6]),
                 "+a"(O[7]), "+a"(O[8]), "+a"(O[9]), "+a"(O[10]), "+a"(O[11]), "+a"(O[12]), "+a"(O[13]),
                 "+a"(O[14]), "+a"(O[15]));
}

// two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
// acc + the two bf16 values of a packed pair, in fp32 (one v_dot2c_f32_bf16 against 1.0, 1.0)
__device__ __forceinline__ float bf16_pair_sum(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                         acc, false);
}

// A operand of O^T = V^T P^T for latent values 32t .. 32t+31 (rows) and key step s: the
// contraction slots j of lane group g = l/32 are keys 16s + 4g + 8(j/4) + j%4, the keys
// whose probabilities that lane holds in P^T slot j.  The gfx950 transposing LDS read does
// the transpose: in a 16-lane group, lanes 4rr..4rr+3 supply 16 values of one key and lane
// p receives value p of the group's 16 values for four keys.
// Lane (G = l/16, p = l%16, rr = p/4, qq = p%4) reads row 16s + 4(G/2) + rr (first read;
// second read: 8 rows further), values 32t + 16(G%2) + 4qq .. +3 = logical unit
// 4t + 2(G%2) + qq/2, bytes 8(qq%2) within it.  The row's swizzle is G/2 (first read) or
// G/2 + 2 (second read) for every s, and it only flips the unit's two low bits, so `vt0` /
// `vt1` (byte offsets at s = 0, t = 0) plus the constants 16 s LAT_PITCH + 64 t address
// every fragment.
__device__ __forceinline__ int vt_lane_offset(int second) {
  const int l = lane_id();
  const int p = l & 15, G = l >> 4;
  const int rr = p >> 2, qq = p & 3;
  const int row = 4 * (G >> 1) + rr + 8 * second;
  const int unit = (2 * (G & 1) + (qq >> 1)) ^ lat_swz(row);
  return row * LAT_PITCH + 16 * unit + 8 * (qq & 1);
}
// S^T (32 keys x this wave's 32 heads) of one chunk, all 36 steps (used for the first chunk).
__device__ __forceinline__ v16f mla_logits(const v8bf* Qt, const uint8_t* buf) {
  const KOff ko = k_offsets();
  v16f S = {};
#pragma unroll
  for (int ds = 0; ds < D_STEPS; ++ds) S = mfma_bf16_32x32x16(k_frag(buf, k_off(ko, ds)), Qt[ds], S);
  return S;
}

// grid.x = n_q * n_split, grid.y = B.  One block of 4 waves per query (and key split);
// wave w owns heads 32w .. 32w+31 over all 576 values (S^T) and all 512 output values
// (O^T).  Pipeline over chunks of 32 selected rows, 4 LDS buffers: in the step of chunk
// c, chunk c+2 is in flight, the logits of chunk c+1 are formed while the
// softmax of chunk c runs, then O^T += V^T P^T for chunk c.
__global__ __launch_bounds__(MLA_WAVES * 64, 1) void sparse_mla_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    int64_t n_q, int64_t n_k, int64_t ld_q, int64_t ld_kv, int64_t bs_kv, int k, float scale_log2, int n_split,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse,
    PageTable pt) {
  __shared__ __align__(16) uint8_t buf0[CHUNK_BYTES];
  __shared__ __align__(16) uint8_t buf1[CHUNK_BYTES];
  __shared__ __align__(16) uint8_t buf2[CHUNK_BYTES];
  __shared__ __align__(16) uint8_t buf3[CHUNK_BYTES];
  __shared__ int32_t ids[MAX_K];

  const int tid = threadIdx.x, l = tid & 63, g = l >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.y;
  const int64_t qi = blockIdx.x / n_split;
  const int split = blockIdx.x % n_split;
  const int64_t qrow = (int64_t)b * n_q + qi;
  const int32_t* irow = idx + qrow * k;
  // paged caches: kv is the pool, and the ids become pool rows as they are staged below
  const uint16_t* kvb = pt.table ? kv : kv + (int64_t)b * bs_kv;

  // B operands of S^T: head 32w + l%32, values 16ds + 8g .. +7
  v8bf Qt[D_STEPS];
  {
    const uint16_t* qh = q + (qrow * MH + 32 * wv + (l & 31)) * ld_q + 8 * g;
#pragma unroll
    for (int ds = 0; ds < D_STEPS; ++ds) Qt[ds] = *reinterpret_cast<const v8bf*>(qh + 16 * ds);
  }

  // the row's selected ids -> LDS (pool rows for paged caches, invalid ids kept invalid),
  // their loads in flight together with the Q loads; the block's last valid id (the
  // chunks run up to the one holding it) comes from the ids each thread staged
  const uint32_t nk_seq = (uint32_t)min(n_k, (int64_t)INT32_MAX);
  const uint32_t nk = pt.table ? (uint32_t)min(pt.n_pages * PAGE_ROWS, (int64_t)INT32_MAX) : nk_seq;
  constexpr int IDS_PER_THREAD = MAX_K / (MLA_WAVES * 64);
  static_assert(MAX_K % (MLA_WAVES * 64) == 0, "the ids split evenly over the threads");
  int32_t id[IDS_PER_THREAD];
#pragma unroll
  for (int i = 0; i < IDS_PER_THREAD; ++i) {
    const int j = tid + i * MLA_WAVES * 64;
    id[i] = j < k ? irow[j] : -1;
  }
  if (pt.table) {  // every table lookup in flight at once (an invalid id looks up token 0)
    int64_t prow[IDS_PER_THREAD];
#pragma unroll
    for (int i = 0; i < IDS_PER_THREAD; ++i) prow[i] = paged_row(pt, b, (uint32_t)id[i] < nk_seq ? id[i] : 0);
#pragma unroll
    for (int i = 0; i < IDS_PER_THREAD; ++i) id[i] = (uint32_t)id[i] < nk_seq ? (int32_t)prow[i] : -1;
  }
  int last = -1;
#pragma unroll
  for (int i = 0; i < IDS_PER_THREAD; ++i) {
    const int j = tid + i * MLA_WAVES * 64;
    if (j < k) {
      ids[j] = id[i];
      if ((uint32_t)id[i] < nk) last = j;
    }
  }
  // Q is held in registers for the whole row (never re-read from memory)
#pragma unroll
  for (int ds = 0; ds < D_STEPS; ++ds) asm volatile("" : "+v"(Qt[ds]));
  // (exchanged through buffer 3, whose first chunk is gathered after the next barrier)
  int32_t* wave_last = reinterpret_cast<int32_t*>(buf3);
  last = (int)wave_max((float)last);
  if (l == 0) wave_last[wv] = last;
  __syncthreads();
  last = wave_last[0];
#pragma unroll
  for (int w = 1; w < MLA_WAVES; ++w) last = max(last, wave_last[w]);
  last = __builtin_amdgcn_readfirstlane(last);
  const int nchunks = (last + KC) / KC;
  const int c_lo = (int)((int64_t)nchunks * split / n_split);
  const int c_hi = (int)((int64_t)nchunks * (split + 1) / n_split);
  const int n = c_hi - c_lo;

  v16f O[O_TILES];
#pragma unroll
  for (int t = 0; t < O_TILES; ++t) O[t] = v16f{};
  // l_run: sum of the fp32 probabilities (for lse); l_bf: sum of the bf16-rounded ones that
  // the PV product actually weighs, which normalises O (see the epilogue)
  float m_ref = -INFINITY, l_run = 0.f, l_bf = 0.f;

  uint8_t* bufs[NBUF] = {buf0, buf1, buf2, buf3};
  VMCNT(0);  // the Q^T operands are in registers before the chunk loads start
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (j < n) gather_chunk(lds_addr(bufs[j]), kvb, ids, c_lo + j, nk, wv, l, ld_kv);

  v16f S_cur = {};
  if (n > 0) {
    if (n >= 2) VMCNT(LOADS_PER_CHUNK);
    else VMCNT(0);
    block_barrier();
    S_cur = mla_logits(Qt, buf0);
  }

  for (int base = 0; base < n; base += NBUF) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      const int c = base + j;
      if (c < n) {
        // chunk c+1 has landed (every wave's loads; they are the only ones in flight), and
        // chunk c-2's buffer is free
        VMCNT(0);
        LGKM0();
        block_barrier();
        // chunk c+2's loads go out one every four logit MFMAs; past the last chunk they load
        // the last chunk's rows again into the buffer chunk c+2 would take, which no later
        // step reads (cheaper than narrowing the exec mask around every load)
        const ChunkIds gi = chunk_ids(ids, c_lo + min(c + 2, n - 1), wv, l);
        const uint32_t gbuf = lds_addr(bufs[(j + 2) % NBUF]);
        // online softmax of chunk c (base 2, lazily rescaled) interleaved with the logits
        // of chunk c+1 (formed from a stale buffer on the last chunk, and then unused):
        // lane holds head l%32 and keys 8(r/4) + 4g + r%4 of S^T
        const uint32_t vmask = (uint32_t)ballot((uint32_t)ids[(c_lo + c) * KC + (l & 31)] < nk);
        if (vmask != 0xFFFFFFFFu) {
          const uint32_t vm = vmask >> (4 * (opaque(lane_id()) >> 5));  // this lane's keys at bit 8(r/4) + r%4
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!((vm >> (8 * (r >> 2) + (r & 3))) & 1u)) S_cur[r] = -INFINITY;
        }
        const uint8_t* bn = bufs[(j + 1) % NBUF];
        const KOff ko = k_offsets();
        v8bf kf[KRING];
#pragma unroll
        for (int i = 0; i < KRING; ++i) kf[i] = k_frag(bn, k_off(ko, i));
        v16f S_next = {};
        // logits, part 1 (with chunk c's row max)
        constexpr int PART1 = LOADS_PER_CHUNK + 1;
#pragma unroll
        for (int ds = 0; ds < PART1; ++ds) {
          S_next = mfma_bf16_32x32x16(kf[ds % KRING], Qt[ds], S_next);
          kf[ds % KRING] = k_frag(bn, k_off(ko, ds + KRING));
          if (ds % 4 == 1) gather_load(ds / 4, gi, gbuf, kvb, nk, wv, l, ld_kv);
        }
        float mx = fmaxf(fmaxf(S_cur[0], S_cur[1]), S_cur[2]);
#pragma unroll
        for (int r = 3; r < 16; r += 2) mx = fmaxf(fmaxf(mx, S_cur[r]), S_cur[r + 1]);
        mx = fmaxf(mx, S_cur[15]);
        mx = fmaxf(mx, xor32(mx)) * scale_log2;
        if (ballot(mx > m_ref + RESCALE_SLACK)) {
          const float m_new = fmaxf(m_ref, mx);
          if (ballot(m_ref != -INFINITY)) {
            const float alpha = m_ref == -INFINITY ? 0.f : exp2f(m_ref - m_new);
            l_run *= alpha;
            l_bf *= alpha;
            o_guard(O);
            // one tile at a time, each back in its accumulation registers before the next
#pragma unroll
            for (int t = 0; t < O_TILES; ++t) {
              O[t] *= alpha;
              asm volatile("" : "+a"(O[t]));
              __builtin_amdgcn_sched_barrier(0);
            }
            o_guard(O);
          }
          m_ref = m_new;
        }
        // chunk c's probabilities (before any valid key, m_ref = -inf and every logit is
        // -inf: offset 0), then the rest of the logits
        const float m = m_ref == -INFINITY ? 0.f : m_ref;
        float ps = 0.f;
        uint32_t pk[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S_cur[r], scale_log2, -m));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S_cur[r + 1], scale_log2, -m));
          ps += p0 + p1;
          pk[r >> 1] = cvt_pk_bf16(p0, p1);
        }
        ps += xor32(ps);
        l_run += ps;
        float pb = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) pb = bf16_pair_sum(pk[i], pb);
        pb += xor32(pb);
        l_bf += pb;
        const v8bf P0 = __builtin_bit_cast(v8bf, v4i{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]});
        const v8bf P1 = __builtin_bit_cast(v8bf, v4i{(int)pk[4], (int)pk[5], (int)pk[6], (int)pk[7]});
#pragma unroll
        for (int ds = PART1; ds < D_STEPS; ++ds) {
          S_next = mfma_bf16_32x32x16(kf[ds % KRING], Qt[ds], S_next);
          if (ds + KRING < D_STEPS) kf[ds % KRING] = k_frag(bn, k_off(ko, ds + KRING));
          if (ds % 4 == 1 && ds / 4 < LOADS_PER_CHUNK) gather_load(ds / 4, gi, gbuf, kvb, nk, wv, l, ld_kv);
        }
        const uint32_t bc = lds_addr(bufs[j]);
        pv_chunk(O, P0, P1, bc + opaque(vt_lane_offset(0)), bc + opaque(vt_lane_offset(1)));
        S_cur = S_next;
      }
    }
  }

  VMCNT(0);  // the loads issued past the last chunk have landed before the block ends
  // ---- epilogue: lane holds head 32w + l%32, values 32t + 8(r/4) + 4g + r%4
  o_guard(O);
  const int le = opaque(l);
  const int ge = le >> 5;
  const int64_t row_head = ((int64_t)b * n_q + qi) * MH + 32 * wv + (le & 31);
  // O is normalised by the sum of the very bf16 weights its PV product used, so O is a
  // convex combination of V rows with weights of exact sum 1: the rounding of a dominant
  // weight cancels.  lse keeps the fp32 sum.  (When l_run > 0 the key that set m_ref has
  // weight 1, so l_bf >= 1.)
  const bool nonempty = l_run > 0.f;
  const float inv = nonempty ? 1.f / l_bf : 0.f;
  const float lse_v = nonempty ? (m_ref + log2f(l_run)) * LN2 : -INFINITY;
  if (n_split == 1) {
    uint16_t* orow = out + row_head * MDV + 4 * ge;
#pragma unroll
    for (int t = 0; t < O_TILES; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 pkd;
        pkd.x = pack_bf16x2(O[t][4 * i] * inv, O[t][4 * i + 1] * inv);
        pkd.y = pack_bf16x2(O[t][4 * i + 2] * inv, O[t][4 * i + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * t + 8 * i) = pkd;
      }
    if (lse && ge == 0) lse[row_head] = lse_v;
  } else {
    const int64_t prh = (((int64_t)b * n_q + qi) * n_split + split) * MH + 32 * wv + (le & 31);
    float* prow = part_o + prh * MDV + 4 * ge;
#pragma unroll
    for (int t = 0; t < O_TILES; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<v4f*>(prow + 32 * t + 8 * i) =
            v4f{O[t][4 * i], O[t][4 * i + 1], O[t][4 * i + 2], O[t][4 * i + 3]} * inv;
    if (ge == 0) part_lse[prh] = lse_v;
  }
}

// merge the NS splits of one (query, head): O = sum_s e^{lse_s - lse} O_s.  NS is a template
// argument so that every load is unconditional (a load on one path only makes the compiler
// copy its result between registers, and the copy waits for the load).
constexpr int MLA_MAX_SPLIT = 16;
template <int NS>
__global__ __launch_bounds__(128) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse, int H, int d_v,
                                                          uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int PER = MDV / 128;  // the bf16 path: d_v = 512
  static_assert(PER == 4, "a thread merges four adjacent values");
  const int64_t qh = blockIdx.x;  // qrow * H + head
  const int64_t qrow = blockIdx.x / (uint32_t)H;
  const int head = (int)(blockIdx.x % (uint32_t)H);
  // every partial value this thread needs (values 4t .. 4t+3 of each split, one 16-byte load
  // per split) and the splits' weights, all loads issued before any is used
  v4f po[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    po[s] = *reinterpret_cast<const v4f*>(part_o + ((qrow * NS + s) * H + head) * d_v + PER * threadIdx.x);
  float ls[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) ls[s] = part_lse[(qrow * NS + s) * H + head];
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s) mx = fmaxf(mx, ls[s]);
  float den = 0.f, acc[PER] = {};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float wgt = mx != -INFINITY ? exp2f((ls[s] - mx) * LOG2E) : 0.f;
    den += wgt;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] += wgt * po[s][j];
  }
  uint16_t o[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) o[j] = f32_to_bf16_bits(den > 0.f ? acc[j] / den : 0.f);
  *reinterpret_cast<uint2*>(out + qh * d_v + PER * threadIdx.x) =
      make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
  if (lse && threadIdx.x == 0) lse[qh] = den > 0.f ? mx + logf(den) : -INFINITY;
}

template <int... NS>
struct CombineTable {
  static constexpr decltype(&mla_combine_kernel<2>) fn[] = {mla_combine_kernel<NS>...};
};
using Combines = CombineTable<2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>;
static_assert(MLA_MAX_SPLIT == 16, "one combine instantiation per split count 2 .. MLA_MAX_SPLIT");

// fp32 attention (any H, d_qk, d_v <= 256, k <= 4096): one wave per (query, head),
// exact two-pass softmax over the selected keys.
constexpr int F32_MAX_K = 4096;
__global__ __launch_bounds__(64) void sparse_mla_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kv, const float* __restrict__ v,
    const int32_t* __restrict__ idx, int64_t n_q, int64_t n_k, int H, int d_qk, int d_v, int k,
    int64_t ld_q, int64_t ld_kv, int64_t ld_v, int64_t bs_kv, int64_t bs_v, float sm_scale,
    float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float z[F32_MAX_K];
  const int lane = threadIdx.x;
  const int64_t qh = blockIdx.x;  // (b * n_q + t) * H + head
  const int b = blockIdx.y;
  const int64_t qrow = (int64_t)b * n_q + qh / H;
  const int head = (int)(qh % H);
  const float* qv = q + (qrow * H + head) * ld_q;
  const int32_t* irow = idx + qrow * k;
  const float* kvb = kv + (int64_t)b * bs_kv;
  const float* vb = v ? v + (int64_t)b * bs_v : kvb;
  const int64_t vstride = v ? ld_v : ld_kv;
  float mx = -INFINITY;
  for (int j = 0; j < k; ++j) {
    const int32_t s = irow[j];
    float zz = -INFINITY;
    if (s >= 0 && s < n_k) {
      float part = 0.f;
      for (int d = lane; d < d_qk; d += 64) part = __fmaf_rn(qv[d], kvb[(int64_t)s * ld_kv + d], part);
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
  if (s > MLA_MAX_SPLIT) s = MLA_MAX_SPLIT;
  return s < 1 ? 1 : (int)s;
}

size_t sparse_mla_ws_bytes(int64_t B, int64_t n_q, int32_t H, int32_t d_v, int32_t k, int32_t dtype) {
  const int s = sparse_mla_splits(B, n_q, k, dtype);
  if (s <= 1) return 0;
  return (size_t)B * n_q * s * H * ((size_t)d_v + 1) * sizeof(float);
}

hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t st) {
  const int64_t ld_q = a.ld_q ? a.ld_q : a.d_qk;
  const int64_t ld_kv = a.ld_kv ? a.ld_kv : a.d_qk;
  const int64_t ld_v = a.ld_v ? a.ld_v : a.d_v;
  const int64_t bs_kv = a.bs_kv ? a.bs_kv : a.n_k * ld_kv;
  const int64_t bs_v = a.bs_v ? a.bs_v : a.n_k * ld_v;
  if (a.dtype == DSA_F32) {
    dim3 grid((unsigned)(a.n_q * a.H), (unsigned)a.B);
    hipLaunchKernelGGL(sparse_mla_f32_kernel, grid, dim3(64), 0, st, (const float*)a.q, (const float*)a.kv,
                       (const float*)a.v, a.idx, a.n_q, a.n_k, a.H, a.d_qk, a.d_v, a.k, ld_q, ld_kv, ld_v, bs_kv,
                       bs_v, a.sm_scale, (float*)a.out, a.lse);
    return hipGetLastError();
  }
  int s = sparse_mla_splits(a.B, a.n_q, a.k, a.dtype);
  if (a.max_split > 0 && s > a.max_split) s = a.max_split;
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (s > 1) {
    part_o = (float*)a.ws;
    part_lse = part_o + (size_t)a.B * a.n_q * s * a.H * a.d_v;
  }
  dim3 grid((unsigned)(a.n_q * s), (unsigned)a.B);
  hipLaunchKernelGGL(sparse_mla_bf16_kernel, grid, dim3(MLA_WAVES * 64), 0, st, (const uint16_t*)a.q,
                     (const uint16_t*)a.kv, a.idx, a.n_q, a.n_k, ld_q, ld_kv, bs_kv, a.k, a.sm_scale * LOG2E, s,
                     (uint16_t*)a.out, a.lse, part_o, part_lse, a.pages);
  if (s > 1)
    hipLaunchKernelGGL(Combines::fn[s - 2], dim3((unsigned)(a.B * a.n_q * a.H)), dim3(128), 0, st, part_o,
                       part_lse, a.H, a.d_v, (uint16_t*)a.out, a.lse);
  return hipGetLastError();
}

}  // namespace dsa
