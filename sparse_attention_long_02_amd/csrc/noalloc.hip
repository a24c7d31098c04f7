// dsa_forward_decode_noalloc: the decode layer with its scratch memory in a fixed device
// array of the library instead of a caller-supplied workspace, for callers that cannot
// allocate device memory (code under stream capture, tight serving loops, harnesses that
// forbid allocation).
//
// The array lives in device memory of every GPU the library runs on, from the library's
// first use on that GPU until the process ends.  Its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and cached; host code never uses
// the array's own name, which on the host is only a stand-in for the symbol.  Every call on
// one GPU shares that GPU's array: calls that overlap on one GPU (different streams, or
// threads) race on it.  Nothing in the decode path needs the scratch to start zeroed (every
// byte it reads was written earlier in the same call).
#include <mutex>

#include "dsa_kernels.h"

namespace {

constexpr size_t SCRATCH_BYTES = (size_t)128 << 20;
constexpr int MAX_DEVICES = 64;

__device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

std::mutex g_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The current device's address of `scratch` (looked up on the first call on that device).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dsa::set_error(DSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return dsa::set_error(DSA_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return dsa::set_error(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                            hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" int dsa_forward_decode_noalloc(
    int64_t B, const int32_t* ctx_len, int64_t n_k_max, const void* q_idx, const float* q_scale, const float* w,
    const void* k_cache, const float* k_cache_scale, int64_t kc_seq_stride, const void* q, int64_t ld_q,
    const void* kv_cache, int64_t ld_kv, int64_t kv_seq_stride, const void* v_cache, int64_t ld_v,
    int64_t v_seq_stride, int32_t H_I, int32_t d_I, int32_t H, int32_t d_qk, int32_t d_v, int32_t k, float sm_scale,
    int32_t idx_dtype, int32_t attn_dtype, int32_t* idx, void* out, float* lse, dsa_stream_t stream) {
  // the size check comes first and touches no device: a request beyond the array fails
  // with DSA_ERR_UNSUPPORTED whatever else is wrong with it
  const size_t need = dsa_workspace_size(DSA_OP_DECODE, B, 1, n_k_max, H, d_v, k, attn_dtype);
  if (need > SCRATCH_BYTES)
    return dsa::set_error(DSA_ERR_UNSUPPORTED,
                          "dsa_forward_decode_noalloc: this shape needs %zu bytes of scratch; the library's "
                          "fixed scratch holds %zu (use dsa_forward_decode with a workspace)",
                          need, SCRATCH_BYTES);
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st) return st;
  return dsa_forward_decode(B, ctx_len, n_k_max, q_idx, q_scale, w, k_cache, k_cache_scale, kc_seq_stride, q, ld_q,
                            kv_cache, ld_kv, kv_seq_stride, v_cache, ld_v, v_seq_stride, H_I, d_I, H, d_qk, d_v, k,
                            sm_scale, idx_dtype, attn_dtype, idx, out, lse, ws, SCRATCH_BYTES, stream);
}
