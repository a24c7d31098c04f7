// Gathering selected MLA latent rows (576 bf16 values: 512 latent + 64 rope) from HBM into
// LDS, and the operands of the 32x32x16 bf16 logit MFMAs read back from there.  Shared by
// the sparse attention kernel and the indexer KL-loss kernel, which both form the logits
// of 128 query heads against the same gathered rows (MQA mode of MLA: 53ai.com V3.2-Exp
// summary, section 创新架构 and Figure 1).
#pragma once

#include "dsa_device.h"
#include "lds_dma.h"

namespace dsa {

constexpr int MH = 128, MDQK = 576, MDV = 512, KC = 32;
// LDS image of one chunk of 32 gathered rows, in two regions (every LDS read is a per-lane
// base plus an immediate offset):
//   latent: values 0..511 of each row, rows 1088 B apart (16 banks past a multiple of 64
//     banks), and within row r the 16-byte unit u is stored at unit u ^ ((r >> 2) & 3).
//     Both read patterns are then free of bank conflicts: the K operand (one unit of 16
//     rows per pass) and the transposed V operand (4 consecutive rows x 4 units per pass);
//   rope:   values 512..575 of each row, 128 B apart, unit u of row r stored at unit
//     u ^ ((r >> 1) & 7): 16 consecutive rows at one unit then fall in 16 distinct
//     16-byte bank groups.
constexpr int LAT_PITCH = 1088, ROPE_PITCH = 128;
constexpr int LAT_BYTES = KC * LAT_PITCH;                 // 34816
constexpr int CHUNK_BYTES = LAT_BYTES + KC * ROPE_PITCH;  // 38912
__device__ __forceinline__ int lat_swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int rope_swz(int r) { return (r >> 1) & 7; }
constexpr int D_STEPS = MDQK / 16;  // 36 contraction steps of S^T
constexpr int MAX_K = 2048;  // most keys a row may select
constexpr int LOADS_PER_CHUNK = 9;  // per wave: 8 latent rows + 1 rope instruction
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef float v16f __attribute__((ext_vector_type(16)));


// D = A(32x16 bf16) * B(16x32 bf16) + C, fp32.  Lane l: row (A) / column (B) l%32,
// contraction elements 8*(l/32) .. +7; C/D: column l%32, register r holds row
// 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ v16f mfma_bf16_32x32x16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The value itself, opaque to the optimiser: keeps lane offsets from being computed once
// and held across the chunk loop, where registers are scarce.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Row read for id s: ids outside [0, n_k) read row 0 (their keys are masked).
__device__ __forceinline__ uint32_t safe_row(int32_t s, uint32_t n_k) {
  return (uint32_t)s < n_k ? (uint32_t)s : 0u;
}

// The ids of this wave's eight rows of one chunk (read ahead of the loads that use them).
struct ChunkIds {
  int4 a, b;       // rows 8w .. 8w+7
  int32_t rope;    // row 8w + lane/8
};
__device__ __forceinline__ ChunkIds chunk_ids(const int32_t* ids, int c, int wv, int lane) {
  const int32_t* cid = ids + c * KC + 8 * wv;
  ChunkIds r;
  r.a = *reinterpret_cast<const int4*>(cid);
  r.b = *reinterpret_cast<const int4*>(cid + 4);
  r.rope = cid[lane >> 3];
  return r;
}
// A wave's direct global->LDS loads for chunk c cover rows 8w .. 8w+7 of the chunk: each
// latent half as one wave-wide 1 KB load from a scalar row address, and their rope parts
// as one instruction whose lane L loads unit (L%8) ^ swz of row 8w + L/8.
// Load number j (0..7: latent half of row 8w + j; 8: the rope parts of rows 8w .. 8w+7)
// of this wave's share of a chunk into the buffer at LDS address `buf`.
// Rows are `ld` elements apart (ld >= 576, a multiple of 8).
__device__ __forceinline__ void gather_load(int j, const ChunkIds& ci, uint32_t buf, const uint16_t* __restrict__ kvb,
                                            uint32_t n_k, int wv, int lane, int64_t ld = MDQK) {
  if (j < 8) {
    const int32_t id = j == 0 ? ci.a.x : j == 1 ? ci.a.y : j == 2 ? ci.a.z : j == 3 ? ci.a.w
                     : j == 4 ? ci.b.x : j == 5 ? ci.b.y : j == 6 ? ci.b.z : ci.b.w;
    const int r = 8 * wv + j;
    const uint32_t row = safe_row(__builtin_amdgcn_readfirstlane(id), n_k);
    dma16_saddr(kvb + (size_t)row * ld, 16 * (lane ^ lat_swz(r)), buf + r * LAT_PITCH);
  } else {
    const int r = 8 * wv + (lane >> 3);
    const uint32_t row = safe_row(ci.rope, n_k);
    dma16_vaddr(kvb + (size_t)row * ld + 512 + 8 * ((lane & 7) ^ rope_swz(r)), buf + LAT_BYTES + wv * 1024);
  }
}
__device__ __forceinline__ void gather_chunk(uint32_t buf, const uint16_t* __restrict__ kvb, const int32_t* ids,
                                             int c, uint32_t n_k, int wv, int lane, int64_t ld = MDQK) {
  const ChunkIds ci = chunk_ids(ids, c, wv, lane);
#pragma unroll
  for (int j = 0; j < LOADS_PER_CHUNK; ++j) gather_load(j, ci, buf, kvb, n_k, wv, lane, ld);
}

// A operand of S^T for d-step ds (values 16ds .. 16ds+15): row = key r = l%32, elements
// 16ds + 8(l/32) .. +7, i.e. logical unit 2ds + g of the row (g = l/32).  Latent steps
// (ds < 32): stored at unit (2ds + g) ^ swz(r); as the swizzle only flips the two low
// unit bits, that is 2ds + ((g ^ swz) & 1) + (swz & 2) for even ds and
// 2ds + ((g ^ swz) & 1) - (swz & 2) for odd ds, so `lat_e` / `lat_o` (this lane's byte
// offsets of those two cases at ds = 0) plus the constant 32ds address every step.  Rope
// steps (ds >= 32) use `rope`, this lane's offset for that step.
__device__ __forceinline__ v8bf k_frag(const uint8_t* buf, int off) {
  typedef __attribute__((address_space(3))) const v8bf lds_v8bf;
  typedef __attribute__((address_space(3))) const uint8_t lds_u8;
  return *(lds_v8bf*)((lds_u8*)buf + off);
}
__device__ __forceinline__ int rope_offset(int r, int g, int ds) {
  return LAT_BYTES + r * ROPE_PITCH + 16 * ((2 * (ds - 32) + g) ^ rope_swz(r));
}

// This lane's K-fragment offsets (see k_frag / rope_offset), from a lane index the
// optimiser cannot hoist out of the chunk loop.
struct KOff {
  int lat_e, lat_o, r, g;
};
__device__ __forceinline__ KOff k_offsets() {
  const int l = opaque(lane_id());
  KOff o;
  o.r = l & 31;
  o.g = l >> 5;
  const int swz = lat_swz(o.r);
  o.lat_e = o.r * LAT_PITCH + 16 * (((o.g ^ swz) & 1) + (swz & 2));
  o.lat_o = o.r * LAT_PITCH + 16 * (((o.g ^ swz) & 1) - (swz & 2));
  return o;
}
__device__ __forceinline__ int k_off(const KOff& o, int ds) {
  return ds < 32 ? ((ds & 1) ? o.lat_o : o.lat_e) + 32 * ds : rope_offset(o.r, o.g, ds);
}

}  // namespace dsa
