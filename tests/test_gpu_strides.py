"""Strided operands at the C ABI: padded query rows (ld_q), padded key-value rows (ld_kv,
ld_v) and per-sequence cache strides (kc_seq_stride, kv_seq_stride, v_seq_stride).

The padded calls must return exactly what the dense calls return on the same values (the
kernels only read the rows elsewhere), and the decode result is also checked against the
float64 oracle.  The pad bytes hold NaN bit patterns, so a read of a pad would show."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_long_02_amd import dsa
from sparse_attention_long_02_amd import synth as S
from tests.helpers import dev_bf16, dev_f32, dev_u8, out_to_f64, overlap

pytestmark = pytest.mark.gpu

ATOL_BF16 = 2e-2
OVERLAP_MIN = 0.995
NAN_BF16 = 0x7FC1


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _padded(x, width):
    """A view of x (last dim d) inside a buffer whose last dim is `width`, pads NaN."""
    shape = tuple(x.shape[:-1]) + (width,)
    if x.dtype == torch.bfloat16:
        buf = torch.full(shape, NAN_BF16, dtype=torch.int16, device=x.device).view(torch.bfloat16)
    else:
        buf = torch.full(shape, float("nan"), dtype=x.dtype, device=x.device)
    buf[..., : x.shape[-1]] = x
    return buf[..., : x.shape[-1]]


def _padded_rows(x, n_alloc, fill, width=None):
    """x [B, n, (d)] as the view buf[:, :n, (:d)] of a per-sequence buffer of n_alloc >= n
    rows per sequence (rows `width` >= d values wide), pads `fill`."""
    shape = (x.shape[0], n_alloc) + tuple(x.shape[2:])
    if width is not None:
        shape = shape[:-1] + (width,)
    buf = torch.full(shape, fill, dtype=torch.int16 if x.dtype == torch.bfloat16 else x.dtype, device=x.device)
    if x.dtype == torch.bfloat16:
        buf = buf.view(torch.bfloat16)
    if width is None:
        buf[:, : x.shape[1]] = x
        return buf[:, : x.shape[1]]
    buf[:, : x.shape[1], : x.shape[2]] = x
    return buf[:, : x.shape[1], : x.shape[2]]


@pytest.fixture(scope="module")
def seq3k():
    cfg = S.CONFIGS["prefill_8k"].with_(L=3000)
    return cfg, S.make_prefill(cfg)


@pytest.mark.parametrize("n_q", [300, 4])
def test_sparse_mla_padded_rows(seq3k, n_q):
    """q rows 640 values apart and kv rows 640 apart (bf16); n_q = 4 splits keys over blocks."""
    cfg, inp = seq3k
    _say(f"[strides] sparse_mla bf16, ld_q = ld_kv = 640, n_q={n_q}")
    q, kv = dev_bf16(inp.q[-n_q:]), dev_bf16(inp.kv)
    rng = np.random.default_rng(3)
    idx = torch.from_numpy(np.stack([np.sort(rng.choice(3000, 2048, replace=False)) for _ in range(n_q)])
                           .astype(np.int32)).cuda()
    o_d, l_d = dsa.sparse_mla(q, kv, idx, cfg.sm_scale, 512)
    qp, kvp = _padded(q, 640), _padded(kv, 640)
    assert qp.stride(-2) == 640 and kvp.stride(-2) == 640
    o_p, l_p = dsa.sparse_mla(qp, kvp, idx, cfg.sm_scale, 512)
    torch.cuda.synchronize()
    assert torch.equal(o_d, o_p) and torch.equal(l_d, l_p)


def test_sparse_mla_fp32_strides():
    """fp32 path with a separate V and strides that are not multiples of anything."""
    cfg = S.CONFIGS["tiny_fp32_512"]
    _say("[strides] sparse_mla fp32, ld_q=67, ld_kv=65, ld_v=70")
    inp = S.make_prefill(cfg)
    q, kv, v = dev_f32(inp.q), dev_f32(inp.kv), dev_f32(inp.v)
    rng = np.random.default_rng(4)
    idx = torch.from_numpy(np.stack([np.sort(rng.choice(t + 1, min(t + 1, 64), replace=False)).tolist() +
                                     [-1] * (64 - min(t + 1, 64)) for t in range(cfg.L)]).astype(np.int32)).cuda()
    o_d, l_d = dsa.sparse_mla(q, kv, idx, cfg.sm_scale, cfg.d_v, v=v)
    o_p, l_p = dsa.sparse_mla(_padded(q, 67), _padded(kv, 65), idx, cfg.sm_scale, cfg.d_v, v=_padded(v, 70))
    torch.cuda.synchronize()
    assert torch.equal(o_d, o_p) and torch.equal(l_d, l_p)
    W = O.widen_inputs(inp)
    o_ref, _ = O.sparse_mqa(W["q"], W["kv"], W["v"], idx.cpu().numpy(), cfg.sm_scale)
    assert np.abs(o_p.double().cpu().numpy() - o_ref).max() <= 1e-5


def test_prefill_padded_rows(seq3k):
    cfg, inp = seq3k
    _say("[strides] forward_prefill, ld_q = 1024, ld_kv = 584")
    qi, qs, ki, ks, w = dev_u8(inp.qi), dev_f32(inp.q_scale), dev_u8(inp.ki), dev_f32(inp.k_scale), dev_f32(inp.w)
    q, kv = dev_bf16(inp.q), dev_bf16(inp.kv)
    ref = dsa.forward_prefill(qi, qs, ki, ks, w, q, kv, cfg.k, cfg.sm_scale, cfg.d_v)
    got = dsa.forward_prefill(qi, qs, ki, ks, w, _padded(q, 1024), _padded(kv, 584), cfg.k, cfg.sm_scale, cfg.d_v)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_decode_padded_caches_vs_dense_and_oracle():
    """Caches allocated for more rows than n_k_max (sequence strides of 5200 / 5100 rows),
    kv rows 640 values apart, q rows 640 apart."""
    cfg = S.CONFIGS["decode_64x128k"].with_(L=5000, batch=3)
    _say("[strides] forward_decode, kv_seq_stride = 5200 x 640, kc_seq_stride = 5100, ld_q = 640")
    inp = S.make_decode(cfg)
    ctx_l = [5000, 4097, 1777]
    ctx = torch.tensor(ctx_l, dtype=torch.int32, device="cuda")
    qi, qs, w = dev_u8(inp.qi), dev_f32(inp.q_scale), dev_f32(inp.w)
    kc, kcs = dev_u8(inp.ki), dev_f32(inp.k_scale)
    q, kvc = dev_bf16(inp.q), dev_bf16(inp.kv)
    r_idx, r_out, r_lse = dsa.forward_decode(ctx, qi, qs, w, kc, kcs, q, kvc, cfg.k, cfg.sm_scale, cfg.d_v)
    kc_p = _padded_rows(kc, 5100, 0x7F)
    kcs_p = _padded_rows(kcs, 5100, float("nan"))
    kv_p = _padded_rows(kvc, 5200, NAN_BF16, width=640)
    assert kv_p.stride(0) == 5200 * 640 and kv_p.stride(1) == 640 and kc_p.stride(0) == 5100 * 128
    idx, out, lse = dsa.forward_decode(ctx, qi, qs, w, kc_p, kcs_p, _padded(q, 640), kv_p, cfg.k, cfg.sm_scale,
                                       cfg.d_v)
    torch.cuda.synchronize()
    assert torch.equal(idx, r_idx) and torch.equal(out, r_out) and torch.equal(lse, r_lse)
    g_idx, g_out = idx.cpu().numpy(), out_to_f64(out)
    for b in range(cfg.batch):
        qhat = O.dequant(inp.qi[b][None], inp.q_scale[b][None])
        khat = O.dequant(inp.ki[b], inp.k_scale[b])
        kvf = O.bf16_to_f64(inp.kv[b])
        qf = O.bf16_to_f64(inp.q[b])[None]
        r = O.dsa_rows(qhat, inp.w[b][None].astype(np.float64), khat, qf, kvf, kvf[:, :512],
                       np.array([ctx_l[b] - 1]), cfg.k, cfg.sm_scale)
        ov, _ = overlap(g_idx[b][None], r["idx"])
        assert ov >= OVERLAP_MIN, (b, ov)
        o, _ = O.sparse_mqa(qf, kvf, kvf[:, :512], g_idx[b][None], cfg.sm_scale)
        assert np.abs(g_out[b] - o[0]).max() <= ATOL_BF16, b


def test_chunk_padded_caches_vs_dense():
    cfg = S.CONFIGS["prefill_8k"].with_(L=4000)
    _say("[strides] forward_chunk, B=2, padded caches and q rows")
    inps = [S.make_prefill(cfg.with_(seed=70 + b)) for b in range(2)]
    q_pos = [1000, 3900]
    n_q = 200
    rows = [np.clip(np.arange(p, p + n_q), 0, cfg.L - 1) for p in q_pos]
    qi = dev_u8(np.stack([inp.qi[r] for inp, r in zip(inps, rows)]))
    qs = dev_f32(np.stack([inp.q_scale[r] for inp, r in zip(inps, rows)]))
    w = dev_f32(np.stack([inp.w[r] for inp, r in zip(inps, rows)]))
    q = dev_bf16(np.stack([inp.q[r] for inp, r in zip(inps, rows)]))
    kc = dev_u8(np.stack([inp.ki for inp in inps]))
    kcs = dev_f32(np.stack([inp.k_scale for inp in inps]))
    kv = dev_bf16(np.stack([inp.kv for inp in inps]))
    pos = torch.tensor(q_pos, dtype=torch.int32, device="cuda")
    ref = dsa.forward_chunk(pos, qi, qs, w, kc, kcs, q, kv, cfg.k, cfg.sm_scale, cfg.d_v)
    got = dsa.forward_chunk(pos, qi, qs, w, _padded_rows(kc, 4100, 0x7F), _padded_rows(kcs, 4100, float("nan")),
                            _padded(q, 704), _padded_rows(kv, 4003, NAN_BF16, width=600), cfg.k, cfg.sm_scale,
                            cfg.d_v)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


def test_kcache_append_padded_cache():
    _say("[strides] kcache_append into a cache of 300 rows per sequence, n_k_max = 256")
    B, n_new, d_I = 3, 40, 128
    g = torch.Generator(device="cuda").manual_seed(5)
    k_new = torch.randn((B, n_new, d_I), generator=g, device="cuda").to(torch.bfloat16)
    pos = torch.tensor([0, 100, 230], dtype=torch.int32, device="cuda")
    kc = torch.full((B, 256, d_I), 0xAB, dtype=torch.uint8, device="cuda")
    kcs = torch.full((B, 256), -7.0, dtype=torch.float32, device="cuda")
    dsa.kcache_append(k_new, pos, kc, kcs)
    buf_c = torch.full((B, 300, d_I), 0xAB, dtype=torch.uint8, device="cuda")
    buf_s = torch.full((B, 300), -7.0, dtype=torch.float32, device="cuda")
    dsa.kcache_append(k_new, pos, buf_c[:, :256], buf_s[:, :256])
    torch.cuda.synchronize()
    assert torch.equal(buf_c[:, :256], kc) and torch.equal(buf_s[:, :256], kcs)
    assert torch.all(buf_c[:, 256:] == 0xAB) and torch.all(buf_s[:, 256:] == -7.0)
