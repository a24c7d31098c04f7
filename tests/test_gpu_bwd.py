"""GPU parity of the sparse-attention backward (dsa_sparse_mla_backward) against the float64
oracle's chain rule, on the forward's own lse and output.

bf16 bar: the kernels round P and dZ to bf16 for the matrix cores (relative 2^-9 each) and
take D_h = dO_h . O_h from the bf16 forward output (itself formed from bf16 P), so every
gradient element carries an error of a few 2^-9 of the magnitudes summed into it.  Each
element is held to its own bound: 2^-7 times the sum of the absolute values of the terms
that make it (|dZ| |kv| for dq; |dZ| |q| and P |dO| for dkv), plus the effect of an error of
2^-8 sum_d |dO_hd| (P |V|)_hd in D_h, plus 1e-6 of the tensor's largest value for the fp32
accumulation.  The Frobenius error relative to the reference is also held to 1e-2.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_long_02_amd import dsa
from sparse_attention_long_02_amd import synth as S
from tests.helpers import dev_bf16, dev_f32, out_to_f64

pytestmark = pytest.mark.gpu

FROB_REL = 1e-2
ELEM_REL = 2e-2


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _idx(rng, n_q, n_k, k, causal_offset=None):
    """k distinct ids per row; rows keep fewer than k (-1 padded) now and then."""
    idx = np.full((n_q, k), -1, dtype=np.int32)
    for t in range(n_q):
        hi = n_k if causal_offset is None else min(n_k, causal_offset + t + 1)
        m = min(k, hi) if t % 7 else min(k, hi) // 2
        idx[t, :m] = np.sort(rng.choice(hi, m, replace=False))
    return idx


def _compare(name, got, ref, bound=None):
    err = got - ref
    frob = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-30))
    elem = float(np.abs(err).max() / max(np.abs(ref).max(), 1e-30))
    msg = f"  {name}: relative Frobenius error {frob:.2e}, max element error / max {elem:.2e}"
    ok = frob <= FROB_REL and elem <= ELEM_REL
    if bound is not None:
        tol = bound + 1e-6 * np.abs(ref).max()
        ratio = float((np.abs(err) / tol).max())
        msg += f", worst element error / own bound {ratio:.2e}"
        ok = ok and ratio <= 1.0
    _say(msg)
    assert ok, (name, frob, elem)


U = 2.0 ** -8   # a bf16 rounding (2^-9) with a factor 2 of slack


def _element_bounds(q, kv, v, idx, do, sm_scale):
    """Per-element error bounds of the bf16 kernels' dq and dkv (see the module docstring),
    from the float64 operands: 2U times the magnitudes of the summed terms, plus the
    propagated D_h error."""
    n_q, n_k = q.shape[0], kv.shape[0]
    Bq = np.zeros(q.shape)
    Bkv = np.zeros(kv.shape)
    akv, av = np.abs(kv), np.abs(v)
    for t in range(n_q):
        sel = idx[t][(idx[t] >= 0) & (idx[t] < n_k)]
        if len(sel) == 0:
            continue
        z = sm_scale * (q[t] @ kv[sel].T)
        P = np.exp(z - z.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        dP = do[t] @ v[sel].T
        dZ = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
        dD = U * np.sum(np.abs(do[t]) * (P @ av[sel]), axis=1)        # bound on the D_h error
        PdD = P * dD[:, None]
        Bq[t] = 2 * U * sm_scale * (np.abs(dZ) @ akv[sel]) + sm_scale * (PdD @ akv[sel])
        contrib = 2 * U * sm_scale * (np.abs(dZ).T @ np.abs(q[t])) + sm_scale * (PdD.T @ np.abs(q[t]))
        contrib[:, : v.shape[1]] += 2 * U * (P.T @ np.abs(do[t]))
        Bkv[sel] += contrib
    return Bq, Bkv


def _bf16_case(B, n_q, n_k, k, seed, idx=None):
    cfg = S.CONFIGS["prefill_8k"].with_(L=n_k, seed=seed)
    inps = [S.make_prefill(cfg.with_(seed=seed + b)) for b in range(B)]
    rng = np.random.default_rng(seed)
    q_bits = np.stack([inp.q[:n_q] for inp in inps])
    kv_bits = np.stack([inp.kv for inp in inps])
    if idx is None:
        idx = np.stack([_idx(rng, n_q, n_k, k) for _ in range(B)])
    do_bits = S.bf16_bits(rng.standard_normal((B, n_q, 128, 512)).astype(np.float32))
    q, kv, do = dev_bf16(q_bits), dev_bf16(kv_bits), dev_bf16(do_bits)
    idx_d = torch.from_numpy(idx).cuda()
    out, lse = dsa.sparse_mla(q, kv, idx_d, cfg.sm_scale, 512)
    dq, dkv, dv = dsa.sparse_mla_backward(q, kv, idx_d, out, lse, do, cfg.sm_scale)
    torch.cuda.synchronize()
    assert dv is None
    g_dq, g_dkv = out_to_f64(dq), dkv.double().cpu().numpy()
    for b in range(B):
        q64, kv64, do64 = O.bf16_to_f64(q_bits[b]), O.bf16_to_f64(kv_bits[b]), O.bf16_to_f64(do_bits[b])
        r_dq, r_dkv, _ = O.sparse_mqa_backward(q64, kv64, kv64[:, :512], idx[b], do64, cfg.sm_scale, True)
        b_dq, b_dkv = _element_bounds(q64, kv64, kv64[:, :512], idx[b], do64, cfg.sm_scale)
        _compare(f"dq[{b}]", g_dq[b], r_dq, b_dq)
        _compare(f"dkv[{b}]", g_dkv[b], r_dkv, b_dkv)
        # keys no query selected get exactly zero
        unused = np.setdiff1d(np.arange(n_k), idx[b][idx[b] >= 0])
        assert np.all(g_dkv[b][unused] == 0)
    return g_dq, g_dkv


def test_backward_bf16_vs_oracle():
    _say("[sparse MLA backward, bf16] n_q=300, n_k=2000, k=256")
    _bf16_case(1, 300, 2000, 256, seed=61)


def test_backward_bf16_two_passes_and_batch():
    """4200 queries (two passes of at most 4096) with k = 64, and B = 2 sequences."""
    _say("[sparse MLA backward, bf16] n_q=4200 (two passes), k=64")
    _bf16_case(1, 4200, 4400, 64, seed=62)
    _say("[sparse MLA backward, bf16] B=2, n_q=96, k=128")
    _bf16_case(2, 96, 1500, 128, seed=63)


def test_backward_bf16_dkv_subpasses_across_sequences():
    """B = 5 sequences of 900 queries: the key-gradient sub-passes of at most 2048 queries
    (rows 0-2047, 2048-4095, then the second pass's 404) each span three sequences and
    start or end inside one, so their key ranges and pair lists cover several sequences."""
    _say("[sparse MLA backward, bf16] B=5, n_q=900, n_k=1200, k=32")
    _bf16_case(5, 900, 1200, 32, seed=68)


def test_backward_bf16_k2048_across_a_pass_boundary():
    """k = 2048 (the workload's k: 64 chunks per row, every iteration of the row scan, the
    full P / dZ workspace) over 4100 queries, so the second pass of at most 4096 queries
    runs too.  Every 41st row keeps 2048 distinct ids with -1 holes inside later chunks;
    the other rows keep 32 to 96 ids, also with holes (the oracle's cost stays small)."""
    n_q, n_k, k = 4100, 8192, 2048
    _say(f"[sparse MLA backward, bf16] n_q={n_q}, n_k={n_k}, k={k} (two passes)")
    rng = np.random.default_rng(66)
    idx = np.full((n_q, k), -1, dtype=np.int32)
    for t in range(n_q):
        full = t % 41 == 0 or t in (4095, 4096, 4099)
        m = k if full else int(rng.integers(32, 97))
        ids = np.sort(rng.choice(n_k, m, replace=False)).astype(np.int32)
        slots = np.arange(m) if full else np.sort(rng.choice(k, m, replace=False))
        idx[t, slots] = ids
        if full:   # holes in later chunks (ids are ignored wherever a -1 sits)
            idx[t, rng.choice(np.arange(k // 2, k), 40, replace=False)] = -1
    _bf16_case(1, n_q, n_k, k, seed=67, idx=idx[None])


def test_backward_bf16_rows_without_keys():
    """A row with no valid id has zero dq and adds nothing."""
    _say("[sparse MLA backward, bf16] empty rows")
    cfg = S.CONFIGS["prefill_8k"].with_(L=500)
    inp = S.make_prefill(cfg)
    rng = np.random.default_rng(64)
    idx = _idx(rng, 64, 500, 64)
    idx[5] = -1
    idx[9, :] = 700          # out of range: ignored
    q, kv = dev_bf16(inp.q[:64]), dev_bf16(inp.kv)
    do = dev_bf16(S.bf16_bits(rng.standard_normal((64, 128, 512)).astype(np.float32)))
    idx_d = torch.from_numpy(idx).cuda()
    out, lse = dsa.sparse_mla(q, kv, idx_d, cfg.sm_scale, 512)
    dq, dkv, _ = dsa.sparse_mla_backward(q, kv, idx_d, out, lse, do, cfg.sm_scale)
    torch.cuda.synchronize()
    assert torch.all(dq[5] == 0) and torch.all(dq[9] == 0)
    r_dq, r_dkv, _ = O.sparse_mqa_backward(O.bf16_to_f64(inp.q[:64]), O.bf16_to_f64(inp.kv),
                                           O.bf16_to_f64(inp.kv)[:, :512], idx, O.bf16_to_f64(
                                               do.view(torch.int16).cpu().numpy().view(np.uint16)),
                                           cfg.sm_scale, True)
    q64, kv64 = O.bf16_to_f64(inp.q[:64]), O.bf16_to_f64(inp.kv)
    do64 = O.bf16_to_f64(do.view(torch.int16).cpu().numpy().view(np.uint16))
    b_dq, b_dkv = _element_bounds(q64, kv64, kv64[:, :512], idx, do64, cfg.sm_scale)
    _compare("dq", out_to_f64(dq), r_dq, b_dq)
    _compare("dkv", dkv.double().cpu().numpy(), r_dkv, b_dkv)


def test_backward_fp32_vs_oracle():
    cfg = S.CONFIGS["tiny_fp32_512"]
    _say("[sparse MLA backward, fp32] L=512, separate V")
    inp = S.make_prefill(cfg)
    rng = np.random.default_rng(65)
    idx = _idx(rng, cfg.L, cfg.L, cfg.k, causal_offset=0)
    q, kv, v = dev_f32(inp.q), dev_f32(inp.kv), dev_f32(inp.v)
    do_np = (rng.standard_normal((cfg.L, cfg.H, cfg.d_v)) / 4).astype(np.float32)
    idx_d = torch.from_numpy(idx).cuda()
    out, lse = dsa.sparse_mla(q, kv, idx_d, cfg.sm_scale, cfg.d_v, v=v)
    dq, dkv, dv = dsa.sparse_mla_backward(q, kv, idx_d, out, lse, dev_f32(do_np), cfg.sm_scale, v=v)
    torch.cuda.synchronize()
    W = O.widen_inputs(inp)
    r_dq, r_dkv, r_dv = O.sparse_mqa_backward(W["q"], W["kv"], W["v"], idx, do_np.astype(np.float64),
                                              cfg.sm_scale, False)
    for name, got, ref in (("dq", dq, r_dq), ("dkv", dkv, r_dkv), ("dv", dv, r_dv)):
        g = got.double().cpu().numpy()
        err = float(np.abs(g - ref).max())
        _say(f"  {name}: max-abs error {err:.2e} (max |ref| {np.abs(ref).max():.2e})")
        assert err <= 1e-5 * (1 + np.abs(ref).max()), name
