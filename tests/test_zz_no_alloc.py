"""dsa_forward_decode_noalloc (the decode entry point whose scratch is a fixed device array
of the library, for callers that cannot allocate) against dsa_forward_decode with a
caller-supplied workspace: the same kernels, so the results must be bit-identical.  Two
calls in a row, the second smaller than the first (the array keeps the first call's
contents), then a shape whose scratch would exceed the array, which must be refused."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from sparse_attention_long_02_amd import dsa
from sparse_attention_long_02_amd import synth as S
from tests.helpers import dev_bf16, dev_f32, dev_u8

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _decode_case(B, L, ctx_l, seed):
    cfg = S.CONFIGS["decode_64x128k"].with_(L=L, batch=B, seed=seed)
    inp = S.make_decode(cfg)
    ctx = torch.tensor(ctx_l, dtype=torch.int32, device="cuda")
    ops = (ctx, dev_u8(inp.qi), dev_f32(inp.q_scale), dev_f32(inp.w), dev_u8(inp.ki), dev_f32(inp.k_scale),
           dev_bf16(inp.q), dev_bf16(inp.kv))
    return cfg, ops


def _noalloc(cfg, ops):
    ctx, qi, qs, w, kc, kcs, q, kvc = ops
    B, L = cfg.batch, cfg.L
    idx = torch.full((B, cfg.k), -7, dtype=torch.int32, device="cuda")
    out = torch.zeros((B, cfg.H, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, cfg.H), dtype=torch.float32, device="cuda")
    st = dsa.lib().dsa_forward_decode_noalloc(
        B, ctx.data_ptr(), L, qi.data_ptr(), qs.data_ptr(), w.data_ptr(), kc.data_ptr(), kcs.data_ptr(), L,
        q.data_ptr(), cfg.d_qk, kvc.data_ptr(), cfg.d_qk, L * cfg.d_qk, None, 0, 0, cfg.H_I, cfg.d_I, cfg.H,
        cfg.d_qk, cfg.d_v, cfg.k, ctypes.c_float(cfg.sm_scale), dsa.DSA_FP8_E4M3, dsa.DSA_BF16, idx.data_ptr(),
        out.data_ptr(), lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == dsa.DSA_OK, dsa.lib().dsa_last_error()
    return idx, out, lse


def test_noalloc_decode_matches_workspace_decode():
    for B, L, ctx_l, seed in [(8, 40000, [40000, 39999, 20000, 16385, 2049, 2048, 1, 33333], 81),
                              (3, 5000, [5000, 4097, 100], 82)]:
        _say(f"[no-alloc decode] B={B}, n_k_max={L}")
        cfg, ops = _decode_case(B, L, ctx_l, seed)
        ctx, qi, qs, w, kc, kcs, q, kvc = ops
        r_idx, r_out, r_lse = dsa.forward_decode(ctx, qi, qs, w, kc, kcs, q, kvc, cfg.k, cfg.sm_scale, cfg.d_v)
        g_idx, g_out, g_lse = _noalloc(cfg, ops)
        torch.cuda.synchronize()
        assert torch.equal(g_idx, r_idx)
        assert torch.equal(g_out, r_out)
        assert torch.equal(g_lse, r_lse)


def test_noalloc_decode_refuses_oversized_scratch():
    L = dsa.lib()
    B, n = 128, 262144
    # the pointers below are placeholders that must never reach a kernel: the call has to be
    # refused on the host, so the shape's scratch must exceed the 128 MiB array
    need = dsa.workspace_size(dsa.DSA_OP_DECODE, B, 1, n, 128, 512, 2048, dsa.DSA_BF16)
    assert need > (128 << 20), f"shape needs only {need} bytes: pick a larger one"
    st = L.dsa_forward_decode_noalloc(B, 1 << 20, n, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, n, 1 << 20, 576,
                                      1 << 20, 576, n * 576, None, 0, 0, 64, 128, 128, 576, 512, 2048,
                                      ctypes.c_float(0.04), dsa.DSA_FP8_E4M3, dsa.DSA_BF16, 1 << 20, 1 << 20, None,
                                      None)
    assert st == dsa.DSA_ERR_UNSUPPORTED
    assert b"scratch" in L.dsa_last_error()
