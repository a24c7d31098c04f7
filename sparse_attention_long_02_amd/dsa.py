"""Python binding of libdsa (the C ABI in include/dsa.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, passes their device
pointers, sizes and torch's current HIP stream to the library, and returns the output
tensors it allocated.  All arithmetic runs in the library's HIP kernels; there is no
fallback of any kind: if libdsa.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = 0, -1, -2, -3, -4
DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
DSA_PAGE_ROWS = 64  # tokens per page of the paged caches
(DSA_OP_INDEXER, DSA_OP_TOPK, DSA_OP_SPARSE_MLA, DSA_OP_PREFILL, DSA_OP_DECODE, DSA_OP_SELECT, DSA_OP_CHUNK,
 DSA_OP_MLA_BWD, DSA_OP_KL_DENSE) = range(9)

_i64, _i32, _f32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

_SIGNATURES = {
    "dsa_abi_version": (ctypes.c_int, []),
    "dsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dsa_last_error": (ctypes.c_char_p, []),
    "dsa_workspace_size": (_sz, [_i32, _i64, _i64, _i64, _i32, _i32, _i32, _i32]),
    "dsa_indexer": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _i32, _i32,
                                   _i64, _i64, _vp, _i64, _vp]),
    "dsa_topk": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _i32, _vp, _vp, _sz, _vp]),
    "dsa_sparse_mla": (ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i32, _i32,
                                      _i32, _i32, _f32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "dsa_select_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp,
                                          _sz, _vp]),
    "dsa_forward_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _i64,
                                           _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _vp, _vp,
                                           _vp, _vp, _sz, _vp]),
    "dsa_forward_decode": (ctypes.c_int, [_i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp,
                                          _i64, _i64, _vp, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _i32,
                                          _f32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dsa_forward_decode_noalloc": (ctypes.c_int, [_i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64,
                                                  _vp, _i64, _i64, _vp, _i64, _i64, _i32, _i32, _i32, _i32,
                                                  _i32, _i32, _f32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "dsa_forward_decode_paged": (ctypes.c_int, [_i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64,
                                                _vp, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                                _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dsa_forward_chunk_paged": (ctypes.c_int, [_i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp,
                                               _i64, _vp, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                               _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dsa_forward_chunk": (ctypes.c_int, [_i64, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64,
                                         _vp, _i64, _i64, _vp, _i64, _i64, _i32, _i32, _i32, _i32, _i32,
                                         _i32, _f32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dsa_sparse_mla_backward": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32,
                                               _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dsa_indexer_scores_at": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32,
                                             _i32, _vp, _vp]),
    "dsa_indexer_kl": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _f32, _i32,
                                      _vp, _vp, _vp]),
    "dsa_indexer_kl_dense": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _i32,
                                            _i32, _i32, _f32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "dsa_fp8_quantize_rows": (ctypes.c_int, [_vp, _i32, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i32, _vp]),
    "dsa_kcache_append": (ctypes.c_int, [_vp, _i32, _i64, _i64, _i32, _vp, _i64, _i64, _vp, _vp, _vp]),
}

_lib = None


class DSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libdsa.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_attention_long_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != DSA_OK:
        raise DSAError(status, lib().dsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libdsa takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libdsa takes contiguous tensors")
    return t.data_ptr()


def _rows(t: Optional[torch.Tensor], n_row_dims: int = 1):
    """(device pointer, row stride in elements) of a tensor whose innermost dimension is
    contiguous and whose leading dimensions lay its rows out evenly (a padded view such
    as x[..., :d] of a wider buffer).  ``n_row_dims`` leading-to-innermost dimensions
    (before the last) must form one evenly strided run of rows."""
    if t is None:
        return None, 0
    if not t.is_cuda:
        raise ValueError("libdsa takes device tensors")
    if t.stride(-1) != 1:
        raise ValueError("the innermost dimension must be contiguous")
    ld = t.stride(-2) if t.dim() >= 2 else t.shape[-1]
    run = ld
    for d in range(t.dim() - 2, t.dim() - 2 - n_row_dims, -1):
        if d < 0:
            break
        if t.shape[d] > 1 and t.stride(d) != run:
            raise ValueError("rows must be evenly strided")
        run *= t.shape[d]
    return t.data_ptr(), ld


def _cache(t: Optional[torch.Tensor]):
    """(device pointer, row stride, sequence stride) of a per-sequence cache [B, n, width]
    whose rows are evenly strided within each sequence."""
    if t is None:
        return None, 0, 0
    if not t.is_cuda:
        raise ValueError("libdsa takes device tensors")
    if t.dim() != 3 or t.stride(-1) != 1:
        raise ValueError("caches are [B, n, width] with the innermost dimension contiguous")
    ld, bs = t.stride(1), t.stride(0)
    if t.shape[1] == 1:
        ld = max(ld, t.shape[2])
    if t.shape[0] == 1:
        bs = max(bs, t.shape[1] * ld)
    return t.data_ptr(), ld, bs


def _key_cache(k_cache: torch.Tensor, k_cache_scale: torch.Tensor):
    """(codes pointer, sequence stride in key rows) of an indexer key cache [B, n, d_I]
    with dense rows, and its scales [B, n] on the same sequence stride."""
    if not (k_cache.is_cuda and k_cache_scale.is_cuda):
        raise ValueError("libdsa takes device tensors")
    d_I = k_cache.shape[-1]
    if k_cache.stride(-1) != 1 or k_cache.stride(-2) != d_I or k_cache_scale.stride(-1) != 1:
        raise ValueError("indexer key-cache rows must be dense")
    bs = k_cache.stride(0) // d_I
    if k_cache.stride(0) != bs * d_I or (k_cache.shape[0] > 1 and k_cache_scale.stride(0) != bs):
        raise ValueError("the key cache and its scales must share one sequence stride (in rows)")
    if k_cache.shape[0] == 1:
        bs = max(bs, k_cache.shape[1])
    return k_cache.data_ptr(), bs


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _idx_dtype(t: torch.Tensor) -> int:
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DSA_FP8_E4M3
    if t.dtype == torch.float32:
        return DSA_F32
    raise TypeError(f"indexer operands must be FP8 codes (uint8 / float8_e4m3fn) or float32, got {t.dtype}")


def _attn_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float32:
        return DSA_F32
    raise TypeError(f"attention operands must be bfloat16 or float32, got {t.dtype}")


def workspace_size(op: int, B: int, n_q: int, n_k: int, H: int, d_v: int, k: int, dtype: int) -> int:
    return int(lib().dsa_workspace_size(op, B, n_q, n_k, H, d_v, k, dtype))


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def indexer(q_idx, q_scale, k_idx, k_scale, w, q_pos=None, row_begin: int = 0,
            n_rows: Optional[int] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Index scores [B, n_rows, n_k] (fp32).  Shapes: q_idx [B, n_q, H_I, d_I] (or without
    the leading B), q_scale/w [B, n_q, H_I], k_idx [B, n_k, d_I], k_scale [B, n_k]."""
    squeeze = q_idx.dim() == 3
    if squeeze:
        q_idx, q_scale, w, k_idx, k_scale = (x.unsqueeze(0) for x in (q_idx, q_scale, w, k_idx, k_scale))
    B, n_q, H_I, d_I = q_idx.shape
    n_k = k_idx.shape[1]
    n_rows = n_q - row_begin if n_rows is None else n_rows
    if out is None:
        out = torch.empty((B, n_rows, n_k), dtype=torch.float32, device=q_idx.device)
    _check(lib().dsa_indexer(_ptr(q_idx), _ptr(q_scale), _ptr(k_idx), _ptr(k_scale), _ptr(w), B, n_q, n_k,
                             _ptr(q_pos), H_I, d_I, _idx_dtype(q_idx), row_begin, n_rows, _ptr(out),
                             out.shape[-1], _stream()))
    return out[0] if squeeze else out


def topk(scores, k: int, q_pos=None, row_begin: int = 0, n_k: Optional[int] = None) -> torch.Tensor:
    """Top-k selection of scores [B, n_rows, ld] (or [n_rows, ld]) -> idx int32 [.., n_rows, k]."""
    squeeze = scores.dim() == 2
    if squeeze:
        scores = scores.unsqueeze(0)
    B, n_rows, ld = scores.shape
    n_k = ld if n_k is None else n_k
    idx = torch.empty((B, n_rows, k), dtype=torch.int32, device=scores.device)
    _check(lib().dsa_topk(_ptr(scores), ld, B, n_rows, n_k, _ptr(q_pos), row_begin, k, _ptr(idx), None, 0,
                          _stream()))
    return idx[0] if squeeze else idx


def sparse_mla(q, kv, idx, sm_scale: float, d_v: int, v=None):
    """Sparse MQA attention.  q [B, n_q, H, d_qk] (or without B), kv [B, n_k, d_qk],
    idx [B, n_q, k] int32, v [B, n_k, d_v] or None (V = kv[..., :d_v]) -> (out, lse)."""
    squeeze = q.dim() == 3
    if squeeze:
        q, kv, idx = q.unsqueeze(0), kv.unsqueeze(0), idx.unsqueeze(0)
        v = v.unsqueeze(0) if v is not None else None
    B, n_q, H, d_qk = q.shape
    n_k, k = kv.shape[1], idx.shape[-1]
    dt = _attn_dtype(q)
    out = torch.empty((B, n_q, H, d_v), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=q.device)
    ws = _workspace(workspace_size(DSA_OP_SPARSE_MLA, B, n_q, n_k, H, d_v, k, dt), q.device)
    q_p, ld_q = _rows(q, 3)
    kv_p, ld_kv = _rows(kv, 2)
    v_p, ld_v = _rows(v, 2)
    _check(lib().dsa_sparse_mla(q_p, ld_q, kv_p, ld_kv, v_p, ld_v, _ptr(idx), B, n_q, n_k, H, d_qk, d_v, k,
                                float(sm_scale), dt, _ptr(out), _ptr(lse), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream()))
    return (out[0], lse[0]) if squeeze else (out, lse)


def select_prefill(q_idx, q_scale, k_idx, k_scale, w, k: int, idx=None, ws=None) -> torch.Tensor:
    """Stages 1-2 over one sequence: idx [L, k] int32 (scores never stored on the FP8 path)."""
    L, H_I, d_I = q_idx.shape
    it = _idx_dtype(q_idx)
    idx = torch.empty((L, k), dtype=torch.int32, device=q_idx.device) if idx is None else idx
    if ws is None:
        ws = _workspace(workspace_size(DSA_OP_SELECT, 1, L, L, 1, 1, k, it), q_idx.device)
    _check(lib().dsa_select_prefill(_ptr(q_idx), _ptr(q_scale), _ptr(k_idx), _ptr(k_scale), _ptr(w), L, H_I,
                                    d_I, k, it, _ptr(idx), _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    return idx


def forward_prefill(q_idx, q_scale, k_idx, k_scale, w, q, kv, k: int, sm_scale: float, d_v: int, v=None,
                    idx=None, out=None, lse=None, ws=None):
    """Whole DSA layer over one sequence of L tokens -> (idx [L, k], out [L, H, d_v], lse [L, H])."""
    L, H_I, d_I = q_idx.shape
    _, H, d_qk = q.shape
    it, at = _idx_dtype(q_idx), _attn_dtype(q)
    dev = q.device
    idx = torch.empty((L, k), dtype=torch.int32, device=dev) if idx is None else idx
    out = torch.empty((L, H, d_v), dtype=q.dtype, device=dev) if out is None else out
    lse = torch.empty((L, H), dtype=torch.float32, device=dev) if lse is None else lse
    if ws is None:
        ws = _workspace(workspace_size(DSA_OP_PREFILL, 1, L, L, H, d_v, k, at), dev)
    q_p, ld_q = _rows(q, 2)
    kv_p, ld_kv = _rows(kv, 1)
    v_p, ld_v = _rows(v, 1)
    _check(lib().dsa_forward_prefill(_ptr(q_idx), _ptr(q_scale), _ptr(k_idx), _ptr(k_scale), _ptr(w),
                                     q_p, ld_q, kv_p, ld_kv, v_p, ld_v, L, H_I, d_I, H, d_qk, d_v, k,
                                     float(sm_scale), it, at, _ptr(idx), _ptr(out), _ptr(lse), _ptr(ws),
                                     0 if ws is None else ws.numel(), _stream()))
    return idx, out, lse


def forward_decode(ctx_len, q_idx, q_scale, w, k_cache, k_cache_scale, q, kv_cache, k: int, sm_scale: float,
                   d_v: int, v_cache=None, idx=None, out=None, lse=None, ws=None):
    """Whole DSA layer for B sequences with one new token each -> (idx [B, k], out, lse)."""
    B, H_I, d_I = q_idx.shape
    n_k_max = k_cache.shape[1]
    _, H, d_qk = q.shape
    it, at = _idx_dtype(q_idx), _attn_dtype(q)
    dev = q.device
    idx = torch.empty((B, k), dtype=torch.int32, device=dev) if idx is None else idx
    out = torch.empty((B, H, d_v), dtype=q.dtype, device=dev) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=dev) if lse is None else lse
    if ws is None:
        ws = _workspace(workspace_size(DSA_OP_DECODE, B, 1, n_k_max, H, d_v, k, at), dev)
    kc_p, kc_bs = _key_cache(k_cache, k_cache_scale)
    q_p, ld_q = _rows(q, 2)
    kv_p, ld_kv, bs_kv = _cache(kv_cache)
    v_p, ld_v, bs_v = _cache(v_cache)
    _check(lib().dsa_forward_decode(B, _ptr(ctx_len), n_k_max, _ptr(q_idx), _ptr(q_scale), _ptr(w),
                                    kc_p, k_cache_scale.data_ptr(), kc_bs, q_p, ld_q, kv_p, ld_kv, bs_kv,
                                    v_p, ld_v, bs_v, H_I, d_I, H, d_qk, d_v, k, float(sm_scale), it, at,
                                    _ptr(idx), _ptr(out), _ptr(lse), _ptr(ws),
                                    0 if ws is None else ws.numel(), _stream()))
    return idx, out, lse


def _pools(k_pool, k_pool_scale, kv_pool, block_table, d_I):
    """Check the page pools and the block table; returns the number of whole pages."""
    if not (k_pool.is_cuda and k_pool_scale.is_cuda and kv_pool.is_cuda and block_table.is_cuda):
        raise ValueError("libdsa takes device tensors")
    if k_pool.dim() != 2 or k_pool.stride(1) != 1 or k_pool.stride(0) != d_I or k_pool_scale.stride(-1) != 1:
        raise ValueError("the indexer key pool is [rows, d_I] with dense rows")
    if block_table.dim() != 2 or block_table.stride(1) != 1 or block_table.dtype != torch.int32:
        raise ValueError("block_table is [B, pages] int32 with contiguous rows")
    return min(k_pool.shape[0], k_pool_scale.shape[0], kv_pool.shape[0]) // DSA_PAGE_ROWS


def forward_decode_paged(ctx_len, q_idx, q_scale, w, k_pool, k_pool_scale, q, kv_pool, block_table, n_k_max: int,
                         k: int, sm_scale: float, d_v: int, idx=None, out=None, lse=None, ws=None):
    """forward_decode over paged caches -> (idx [B, k], out, lse).  Pools of n_pages pages of
    DSA_PAGE_ROWS tokens: k_pool [n_pages * DSA_PAGE_ROWS, d_I] FP8 codes, k_pool_scale
    [n_pages * DSA_PAGE_ROWS], kv_pool [n_pages * DSA_PAGE_ROWS, d_qk] bf16 (rows may be a
    padded view); block_table [B, >= ceil(n_k_max / DSA_PAGE_ROWS)] int32 page ids."""
    B, H_I, d_I = q_idx.shape
    _, H, d_qk = q.shape
    it, at = _idx_dtype(q_idx), _attn_dtype(q)
    dev = q.device
    n_pages = _pools(k_pool, k_pool_scale, kv_pool, block_table, d_I)
    idx = torch.empty((B, k), dtype=torch.int32, device=dev) if idx is None else idx
    out = torch.empty((B, H, d_v), dtype=q.dtype, device=dev) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=dev) if lse is None else lse
    if ws is None:
        ws = _workspace(workspace_size(DSA_OP_DECODE, B, 1, n_k_max, H, d_v, k, at), dev)
    q_p, ld_q = _rows(q, 2)
    kv_p, ld_kv = _rows(kv_pool, 1)
    _check(lib().dsa_forward_decode_paged(B, _ptr(ctx_len), n_k_max, _ptr(q_idx), _ptr(q_scale), _ptr(w),
                                          k_pool.data_ptr(), k_pool_scale.data_ptr(), q_p, ld_q, kv_p, ld_kv,
                                          block_table.data_ptr(), block_table.stride(0), n_pages, H_I, d_I, H,
                                          d_qk, d_v, k, float(sm_scale), it, at, _ptr(idx), _ptr(out), _ptr(lse),
                                          _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    return idx, out, lse


def forward_decode_noalloc(ctx_len, q_idx, q_scale, w, k_cache, k_cache_scale, q, kv_cache, k: int,
                           sm_scale: float, d_v: int, v_cache=None, idx=None, out=None, lse=None):
    """forward_decode with the library's fixed scratch instead of a workspace (the entry
    point for callers that cannot allocate; the outputs must be passed in to allocate
    nothing here either)."""
    B, H_I, d_I = q_idx.shape
    n_k_max = k_cache.shape[1]
    _, H, d_qk = q.shape
    it, at = _idx_dtype(q_idx), _attn_dtype(q)
    dev = q.device
    idx = torch.empty((B, k), dtype=torch.int32, device=dev) if idx is None else idx
    out = torch.empty((B, H, d_v), dtype=q.dtype, device=dev) if out is None else out
    lse = torch.empty((B, H), dtype=torch.float32, device=dev) if lse is None else lse
    kc_p, kc_bs = _key_cache(k_cache, k_cache_scale)
    q_p, ld_q = _rows(q, 2)
    kv_p, ld_kv, bs_kv = _cache(kv_cache)
    v_p, ld_v, bs_v = _cache(v_cache)
    _check(lib().dsa_forward_decode_noalloc(B, _ptr(ctx_len), n_k_max, _ptr(q_idx), _ptr(q_scale), _ptr(w), kc_p,
                                            k_cache_scale.data_ptr(), kc_bs, q_p, ld_q, kv_p, ld_kv, bs_kv, v_p,
                                            ld_v, bs_v, H_I, d_I, H, d_qk, d_v, k, float(sm_scale), it, at,
                                            _ptr(idx), _ptr(out), _ptr(lse), _stream()))
    return idx, out, lse


def forward_chunk(q_pos, q_idx, q_scale, w, k_cache, k_cache_scale, q, kv_cache, k: int, sm_scale: float,
                  d_v: int, v_cache=None, idx=None, out=None, lse=None, ws=None):
    """Whole DSA layer for a chunk of n_q new tokens in each of B sequences; row i of
    sequence b sits at position q_pos[b] + i and sees cache rows up to it
    -> (idx [B, n_q, k], out [B, n_q, H, d_v], lse [B, n_q, H])."""
    B, n_q, H_I, d_I = q_idx.shape
    n_k_max = k_cache.shape[1]
    _, _, H, d_qk = q.shape
    it, at = _idx_dtype(q_idx), _attn_dtype(q)
    dev = q.device
    idx = torch.empty((B, n_q, k), dtype=torch.int32, device=dev) if idx is None else idx
    out = torch.empty((B, n_q, H, d_v), dtype=q.dtype, device=dev) if out is None else out
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=dev) if lse is None else lse
    if ws is None:
        ws = _workspace(workspace_size(DSA_OP_CHUNK, B, n_q, n_k_max, H, d_v, k, at), dev)
    kc_p, kc_bs = _key_cache(k_cache, k_cache_scale)
    q_p, ld_q = _rows(q, 3)
    kv_p, ld_kv, bs_kv = _cache(kv_cache)
    v_p, ld_v, bs_v = _cache(v_cache)
    _check(lib().dsa_forward_chunk(B, n_q, _ptr(q_pos), n_k_max, _ptr(q_idx), _ptr(q_scale), _ptr(w),
                                   kc_p, k_cache_scale.data_ptr(), kc_bs, q_p, ld_q, kv_p, ld_kv, bs_kv,
                                   v_p, ld_v, bs_v, H_I, d_I, H, d_qk, d_v, k, float(sm_scale), it, at,
                                   _ptr(idx), _ptr(out), _ptr(lse), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream()))
    return idx, out, lse


def forward_chunk_paged(q_pos, q_idx, q_scale, w, k_pool, k_pool_scale, q, kv_pool, block_table, n_k_max: int,
                        k: int, sm_scale: float, d_v: int, idx=None, out=None, lse=None, ws=None):
    """forward_chunk over paged caches (pools and block table as forward_decode_paged)
    -> (idx [B, n_q, k], out [B, n_q, H, d_v], lse [B, n_q, H])."""
    B, n_q, H_I, d_I = q_idx.shape
    _, _, H, d_qk = q.shape
    it, at = _idx_dtype(q_idx), _attn_dtype(q)
    dev = q.device
    n_pages = _pools(k_pool, k_pool_scale, kv_pool, block_table, d_I)
    idx = torch.empty((B, n_q, k), dtype=torch.int32, device=dev) if idx is None else idx
    out = torch.empty((B, n_q, H, d_v), dtype=q.dtype, device=dev) if out is None else out
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=dev) if lse is None else lse
    if ws is None:
        ws = _workspace(workspace_size(DSA_OP_CHUNK, B, n_q, n_k_max, H, d_v, k, at), dev)
    q_p, ld_q = _rows(q, 3)
    kv_p, ld_kv = _rows(kv_pool, 1)
    _check(lib().dsa_forward_chunk_paged(B, n_q, _ptr(q_pos), n_k_max, _ptr(q_idx), _ptr(q_scale), _ptr(w),
                                         k_pool.data_ptr(), k_pool_scale.data_ptr(), q_p, ld_q, kv_p, ld_kv,
                                         block_table.data_ptr(), block_table.stride(0), n_pages, H_I, d_I, H,
                                         d_qk, d_v, k, float(sm_scale), it, at, _ptr(idx), _ptr(out), _ptr(lse),
                                         _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    return idx, out, lse


def sparse_mla_backward(q, kv, idx, out, lse, d_out, sm_scale: float, v=None, ws=None):
    """Gradients of sparse_mla: q [n_q, H, d_qk] or [B, n_q, H, d_qk], kv [.., n_k, d_qk],
    idx [.., n_q, k], the forward's out and lse, and d_out -> (d_q like q, d_kv fp32 like
    kv, d_v fp32 or None)."""
    batched = q.dim() == 4
    B = q.shape[0] if batched else 1
    n_q, H, d_qk = q.shape[-3:]
    n_k = kv.shape[-2]
    d_v = d_out.shape[-1]
    k = idx.shape[-1]
    dt = _attn_dtype(q)
    d_q = torch.empty_like(q)
    d_kv = torch.empty(kv.shape, dtype=torch.float32, device=q.device)
    d_v_out = torch.empty(v.shape, dtype=torch.float32, device=q.device) if v is not None else None
    if ws is None:
        ws = _workspace(workspace_size(DSA_OP_MLA_BWD, B, n_q, n_k, H, d_v, k, dt), q.device)
    _check(lib().dsa_sparse_mla_backward(_ptr(q), _ptr(kv), _ptr(v), _ptr(idx), _ptr(out), _ptr(lse), _ptr(d_out),
                                         B, n_q, n_k, H, d_qk, d_v, k, float(sm_scale), dt, _ptr(d_q), _ptr(d_kv),
                                         _ptr(d_v_out), _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    return d_q, d_kv, d_v_out


def indexer_scores_at(q_idx, q_scale, k_idx, k_scale, w, idx, out=None) -> torch.Tensor:
    """Index scores of the listed keys: q_idx [n_q, H_I, d_I] or [B, n_q, H_I, d_I], idx
    [.., n_q, k] -> scores [.., n_q, k] fp32 (-inf for ids outside the keys)."""
    batched = q_idx.dim() == 4
    B = q_idx.shape[0] if batched else 1
    n_q, H_I, d_I = q_idx.shape[-3:]
    n_k = k_idx.shape[-2]
    k = idx.shape[-1]
    if out is None:
        out = torch.empty(idx.shape, dtype=torch.float32, device=idx.device)
    _check(lib().dsa_indexer_scores_at(_ptr(q_idx), _ptr(q_scale), _ptr(k_idx), _ptr(k_scale), _ptr(w), _ptr(idx),
                                       B, n_q, n_k, H_I, d_I, k, _idx_dtype(q_idx), _ptr(out), _stream()))
    return out


def indexer_kl(q, kv, idx, lse, idx_scores, sm_scale: float, p_out: bool = False, kl=None):
    """Per-row KL(p_t || softmax of the index scores) over each row's selected keys, with
    p_t the heads' attention probabilities (from lse) summed and L1-normalised.
    q [n_q, H, d_qk] or [B, n_q, H, d_qk] -> (kl [.., n_q], p [.., n_q, k] or None)."""
    batched = q.dim() == 4
    B = q.shape[0] if batched else 1
    n_q, H, d_qk = q.shape[-3:]
    n_k = kv.shape[-2]
    k = idx.shape[-1]
    if kl is None:
        kl = torch.empty(idx.shape[:-1], dtype=torch.float32, device=q.device)
    p = torch.empty(idx.shape, dtype=torch.float32, device=q.device) if p_out else None
    _check(lib().dsa_indexer_kl(_ptr(q), _ptr(kv), _ptr(idx), _ptr(lse), _ptr(idx_scores), B, n_q, n_k, H, d_qk, k,
                                float(sm_scale), _attn_dtype(q), _ptr(kl), _ptr(p), _stream()))
    return kl, p


def indexer_kl_dense(q_idx, q_scale, k_idx, k_scale, w, q, kv, sm_scale: float, q_pos=None, want_lse=False,
                     kl=None, ws=None):
    """Dense warm-up KL loss: per query row, KL(head-averaged dense attention distribution
    over every key up to its position || softmax of its index scores over the same keys).
    Indexer operands as for ``indexer`` and attention operands q [n_q, H, d_qk] / kv
    [n_k, d_qk] (or with a leading B) -> (kl [.., n_q], lse [.., n_q, H] or None)."""
    squeeze = q_idx.dim() == 3
    if squeeze:
        q_idx, q_scale, w, k_idx, k_scale, q, kv = (x.unsqueeze(0) for x in (q_idx, q_scale, w, k_idx, k_scale,
                                                                             q, kv))
    B, n_q, H_I, d_I = q_idx.shape
    n_k = k_idx.shape[1]
    H, d_qk = q.shape[-2:]
    at = _attn_dtype(q)
    if kl is None:
        kl = torch.empty((B, n_q), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, n_q, H), dtype=torch.float32, device=q.device) if want_lse else None
    if ws is None:
        ws = _workspace(workspace_size(DSA_OP_KL_DENSE, B, n_q, n_k, H, 1, 1, at), q.device)
    _check(lib().dsa_indexer_kl_dense(_ptr(q_idx), _ptr(q_scale), _ptr(k_idx), _ptr(k_scale), _ptr(w), _ptr(q),
                                      _ptr(kv), B, n_q, n_k, _ptr(q_pos), H_I, d_I, H, d_qk, float(sm_scale),
                                      _idx_dtype(q_idx), at, _ptr(kl), _ptr(lse), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream()))
    if squeeze:
        return kl[0], (lse[0] if lse is not None else None)
    return kl, lse


def _x_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.float32:
        return DSA_F32
    raise TypeError(f"quantiser input must be bfloat16 or float32, got {t.dtype}")


def fp8_quantize_rows(x, repeat: int = 1, codes=None, scale=None):
    """Per-row FP8 E4M3FN quantisation of a [n_rows, ...] tensor (each row flattened):
    returns (codes uint8 of x's shape, scale fp32 [n_rows, repeat]); the row's scale is
    written `repeat` times (a query token's scale for each of its H_I heads)."""
    assert x.is_cuda and x.is_contiguous()
    n_rows = x.shape[0]
    width = x.numel() // n_rows
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((n_rows, repeat), dtype=torch.float32, device=x.device)
    _check(lib().dsa_fp8_quantize_rows(_ptr(x), _x_dtype(x), n_rows, width, width, _ptr(codes), width,
                                       _ptr(scale), repeat, repeat, _stream()))
    return codes, scale


def kcache_append(k_new, pos, k_cache, k_cache_scale):
    """Quantise k_new [B, n_new, d_I] into k_cache [B, n_k_max, d_I] / k_cache_scale
    [B, n_k_max] at rows pos[b] .. pos[b] + n_new - 1 (in place; the caches may be
    [:, :n_k_max] views of longer per-sequence buffers)."""
    assert k_new.is_cuda and k_new.is_contiguous()
    B, n_new, d_I = k_new.shape
    kc_p, kc_bs = _key_cache(k_cache, k_cache_scale)
    _check(lib().dsa_kcache_append(_ptr(k_new), _x_dtype(k_new), B, n_new, d_I, _ptr(pos), k_cache.shape[1],
                                   kc_bs, kc_p, k_cache_scale.data_ptr(), _stream()))
