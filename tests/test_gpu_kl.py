"""GPU parity of the indexer KL-alignment loss (sparse stage) and of the index scores at
selected keys.

* dsa_indexer_scores_at returns, bit for bit, the scores dsa_indexer writes for the same
  (row, key), and -inf for ignored slots.
* dsa_indexer_kl, fed the forward's selection, lse and those scores, matches the float64
  oracle's KL (and its target distribution p) on the same selection and scores.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from sparse_attention_long_02_amd import dsa
from sparse_attention_long_02_amd import synth as S
from tests.helpers import dev_bf16, dev_f32, dev_u8, indexer_inputs_dev

pytestmark = pytest.mark.gpu

P_RTOL = 2e-4   # target distribution p, relative (fp32 logits, hardware exp2, fp32 lse input)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _kl_tol(p_ref, log_q_gap):
    """Bound on the KL difference: p carries a relative error of at most P_RTOL, which moves
    each term p (ln p - ln q) by P_RTOL p (|ln p - ln q| + 1), plus fp32 rounding of the
    index-score log-sum-exp (1e-6 of the loss scale)."""
    return P_RTOL * float(np.sum(p_ref * (np.abs(log_q_gap) + 1.0))) + 1e-6


def _check_rows(rows, q_f64, kv_f64, g_idx, g_sc, g_kl, g_p, sm_scale):
    worst = 0.0
    for j, t in enumerate(rows):
        kl_ref, p_ref = O.indexer_kl_row(q_f64[j], kv_f64, g_idx[t], g_sc[t].astype(np.float64), sm_scale)
        valid = (g_idx[t] >= 0) & (g_idx[t] < kv_f64.shape[0])
        sc = g_sc[t][valid].astype(np.float64)
        log_q = sc - (sc.max() + np.log(np.sum(np.exp(sc - sc.max())))) if valid.any() else sc
        pv = p_ref[valid]
        gap = np.where(pv > 0, np.log(np.where(pv > 0, pv, 1.0)) - log_q, 0.0)
        tol = _kl_tol(pv, gap)
        err = abs(float(g_kl[t]) - kl_ref)
        worst = max(worst, err / tol)
        assert err <= tol, (t, float(g_kl[t]), kl_ref, tol)
        assert np.allclose(g_p[t], p_ref, rtol=P_RTOL, atol=1e-30), t
    return worst


@pytest.fixture(scope="module")
def layer6k():
    cfg = S.CONFIGS["prefill_8k"].with_(L=6000)
    inp = S.make_prefill(cfg)
    qi, qs, ki, ks, w = indexer_inputs_dev(inp)
    q, kv = dev_bf16(inp.q), dev_bf16(inp.kv)
    idx, out, lse = dsa.forward_prefill(qi, qs, ki, ks, w, q, kv, cfg.k, cfg.sm_scale, cfg.d_v)
    return cfg, inp, (qi, qs, ki, ks, w, q, kv), idx, lse


def test_scores_at_equal_dense_scores(layer6k):
    cfg, inp, (qi, qs, ki, ks, w, q, kv), idx, lse = layer6k
    _say("[scores at selected keys == dense scores] L=6000")
    sc = dsa.indexer_scores_at(qi, qs, ki, ks, w, idx)
    dense = dsa.indexer(qi, qs, ki, ks, w)
    torch.cuda.synchronize()
    valid = idx >= 0
    want = torch.where(valid, torch.gather(dense, 1, idx.clamp(min=0).long()), torch.full_like(sc, -np.inf))
    assert torch.equal(sc, want)
    # arbitrary ids (not a selection, past the causal position, out of range) score too
    ids = torch.tensor([[5999, 0, -1, 6000, 17, 17] + [3] * 26] * 2, dtype=torch.int32, device="cuda")
    sc2 = dsa.indexer_scores_at(qi[:2], qs[:2], ki, ks, w[:2], ids)
    full = dsa.indexer(qi, qs, ki, ks, w, q_pos=torch.tensor([5999], dtype=torch.int32, device="cuda"),
                       row_begin=0, n_rows=2)
    torch.cuda.synchronize()
    assert sc2[0, 0] == full[0, 5999] and sc2[1, 4] == full[1, 17] and sc2[0, 5] == sc2[0, 4]
    assert sc2[0, 2] == -np.inf and sc2[0, 3] == -np.inf


def test_kl_bf16_vs_oracle(layer6k):
    cfg, inp, (qi, qs, ki, ks, w, q, kv), idx, lse = layer6k
    _say("[indexer KL, bf16] L=6000")
    sc = dsa.indexer_scores_at(qi, qs, ki, ks, w, idx)
    kl, p = dsa.indexer_kl(q, kv, idx, lse, sc, cfg.sm_scale, p_out=True)
    kl2, _ = dsa.indexer_kl(q, kv, idx, lse, sc, cfg.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(kl, kl2), "not deterministic"
    g_kl, g_p, g_idx, g_sc = kl.cpu().numpy(), p.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    assert np.all(np.isfinite(g_kl)) and np.all(g_kl >= -1e-5)
    # each row's p sums to one (the heads' distributions over the same keys)
    assert np.allclose(g_p.sum(axis=1), 1.0, atol=1e-4)
    rng = np.random.default_rng(23)
    rows = np.array(sorted(set([0, 1, 31, 32, 33, cfg.k - 1, cfg.k, 5999]) |
                           set(int(x) for x in rng.integers(0, cfg.L, 16))))
    W = O.widen_inputs(inp, rows)
    worst = _check_rows(rows, W["q"], W["kv"], g_idx, g_sc, g_kl, g_p, cfg.sm_scale)
    _say(f"  worst KL error / bound {worst:.3e}; mean KL {g_kl.mean():.4f}")
    # row 0 keeps one key: p = 1 there and the loss is 0
    assert g_p[0, 0] == pytest.approx(1.0, abs=1e-5) and abs(g_kl[0]) <= 1e-6


def test_kl_batched_and_empty_rows():
    """B = 2 sequences through forward_chunk, including rows before the first key (no valid
    id: loss 0, p 0)."""
    n_k, n_q = 3000, 96
    q_pos = [-3, 2904]
    cfg = S.CONFIGS["prefill_8k"].with_(L=n_k)
    _say(f"[indexer KL, batched] B=2, n_q={n_q}, q_pos={q_pos}")
    inps = [S.make_prefill(cfg.with_(seed=50 + b)) for b in range(2)]
    rows = [np.clip(np.arange(p, p + n_q), 0, n_k - 1) for p in q_pos]
    qi = dev_u8(np.stack([inp.qi[r] for inp, r in zip(inps, rows)]))
    qs = dev_f32(np.stack([inp.q_scale[r] for inp, r in zip(inps, rows)]))
    w = dev_f32(np.stack([inp.w[r] for inp, r in zip(inps, rows)]))
    q = dev_bf16(np.stack([inp.q[r] for inp, r in zip(inps, rows)]))
    kc, kcs = dev_u8(np.stack([inp.ki for inp in inps])), dev_f32(np.stack([inp.k_scale for inp in inps]))
    kv = dev_bf16(np.stack([inp.kv for inp in inps]))
    pos = torch.tensor(q_pos, dtype=torch.int32, device="cuda")
    idx, out, lse = dsa.forward_chunk(pos, qi, qs, w, kc, kcs, q, kv, cfg.k, cfg.sm_scale, cfg.d_v)
    sc = dsa.indexer_scores_at(qi, qs, kc, kcs, w, idx)
    kl, p = dsa.indexer_kl(q, kv, idx, lse, sc, cfg.sm_scale, p_out=True)
    torch.cuda.synchronize()
    g_kl, g_p, g_idx, g_sc = kl.cpu().numpy(), p.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    assert np.all(g_kl[0, :3] == 0) and np.all(g_p[0, :3] == 0)
    for b in range(2):
        kv64 = O.bf16_to_f64(inps[b].kv)
        pick = np.array([3, 4, 50, n_q - 1])
        q64 = O.bf16_to_f64(inps[b].q[rows[b][pick]])
        _check_rows(pick, q64, kv64, g_idx[b], g_sc[b], g_kl[b], g_p[b], cfg.sm_scale)


def test_kl_fp32_vs_oracle():
    cfg = S.CONFIGS["tiny_fp32_512"]
    _say("[indexer KL, fp32] L=512")
    inp = S.make_prefill(cfg)
    qi, qs, ki, ks, w = indexer_inputs_dev(inp)
    q, kv, v = dev_f32(inp.q), dev_f32(inp.kv), dev_f32(inp.v)
    idx, out, lse = dsa.forward_prefill(qi, qs, ki, ks, w, q, kv, cfg.k, cfg.sm_scale, cfg.d_v, v=v)
    sc = dsa.indexer_scores_at(qi, qs, ki, ks, w, idx)
    dense = dsa.indexer(qi, qs, ki, ks, w)
    kl, p = dsa.indexer_kl(q, kv, idx, lse, sc, cfg.sm_scale, p_out=True)
    torch.cuda.synchronize()
    valid = idx >= 0
    want = torch.where(valid, torch.gather(dense, 1, idx.clamp(min=0).long()), torch.full_like(sc, -np.inf))
    assert torch.equal(sc, want)
    W = O.widen_inputs(inp)
    g_kl, g_p, g_idx, g_sc = kl.cpu().numpy(), p.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    for t in range(cfg.L):
        kl_ref, p_ref = O.indexer_kl_row(W["q"][t], W["kv"], g_idx[t], g_sc[t].astype(np.float64), cfg.sm_scale)
        assert abs(float(g_kl[t]) - kl_ref) <= 1e-5 * (1 + abs(kl_ref)), t
        assert np.allclose(g_p[t], p_ref, rtol=1e-5, atol=1e-12), t


def test_kl_dense_warmup_when_k_covers_the_context():
    """With k >= L every row keeps all keys 0..t, so the loss is the dense warm-up's:
    the oracle's KL over {0..t} with the oracle's own scores stays within the indexer's
    score tolerance of the GPU's (the GPU's scores carry the FP8 fold's error)."""
    cfg = S.CONFIGS["prefill_8k"].with_(L=1024, k=1024)
    _say("[indexer KL, dense warm-up reading] L=1024, k=1024")
    inp = S.make_prefill(cfg)
    qi, qs, ki, ks, w = indexer_inputs_dev(inp)
    q, kv = dev_bf16(inp.q), dev_bf16(inp.kv)
    idx, out, lse = dsa.forward_prefill(qi, qs, ki, ks, w, q, kv, cfg.k, cfg.sm_scale, cfg.d_v)
    sc = dsa.indexer_scores_at(qi, qs, ki, ks, w, idx)
    kl, p = dsa.indexer_kl(q, kv, idx, lse, sc, cfg.sm_scale, p_out=True)
    torch.cuda.synchronize()
    g_idx, g_sc, g_kl, g_p = idx.cpu().numpy(), sc.cpu().numpy(), kl.cpu().numpy(), p.cpu().numpy()
    for t in (0, 1, 511, 1023):
        assert np.array_equal(g_idx[t][: t + 1], np.arange(t + 1)) and np.all(g_idx[t][t + 1:] == -1)
    rows = np.array([1, 2, 100, 511, 1000, 1023])
    W = O.widen_inputs(inp, rows)
    _check_rows(rows, W["q"], W["kv"], g_idx, g_sc, g_kl, g_p, cfg.sm_scale)
    # end to end against the oracle's own dense indexer scores: |I_gpu - I| <= 1e-2 A moves
    # ln q by at most 2 * 1e-2 * max_s A_s, so the loss by at most that much
    for j, t in enumerate(rows):
        I = O.indexer_row(W["qhat"][j], W["w"][j], W["khat"], int(t))
        A = O.indexer_magnitude_row(W["qhat"][j], W["w"][j], W["khat"], int(t))
        kl_ref, _ = O.indexer_kl_row(W["q"][j], W["kv"], np.arange(t + 1), I, cfg.sm_scale)
        assert abs(float(g_kl[t]) - kl_ref) <= 2e-2 * float(A.max()) + 1e-4, (t, float(g_kl[t]), kl_ref)


def _check_dense_rows(rows, pos, q_f64, kv_f64, g_sc, g_kl, g_lse, sm_scale, v_f64=None):
    """Dense warm-up rows: KL against the oracle over keys 0 .. pos on the GPU's own scores,
    and the dense attention lse against the oracle's."""
    worst = 0.0
    n_k = kv_f64.shape[0]
    for j, t in enumerate(rows):
        p_ = int(pos[j])
        n = max(0, min(p_ + 1, n_k))
        if n == 0:
            assert float(g_kl[j]) == 0.0 and np.all(np.isneginf(g_lse[j])), t
            continue
        ids = np.arange(n, dtype=np.int32)
        sc = g_sc[j][:n].astype(np.float64)
        kl_ref, p_ref = O.indexer_kl_row(q_f64[j], kv_f64, ids, sc, sm_scale)
        log_q = sc - (sc.max() + np.log(np.sum(np.exp(sc - sc.max()))))
        gap = np.where(p_ref > 0, np.log(np.where(p_ref > 0, p_ref, 1.0)) - log_q, 0.0)
        tol = _kl_tol(p_ref, gap)
        err = abs(float(g_kl[j]) - kl_ref)
        worst = max(worst, err / tol)
        assert err <= tol, (t, float(g_kl[j]), kl_ref, tol)
        _, l_ref = O.sparse_mqa_row(q_f64[j], kv_f64, kv_f64 if v_f64 is None else v_f64, ids, sm_scale)
        assert np.allclose(g_lse[j], l_ref, atol=1e-4, rtol=1e-5), t
    return worst


def test_kl_dense_warmup_every_key_bf16():
    """The dense warm-up over every key s <= t at L = 8192 (far more keys than k = 2048):
    KL per row and the dense attention lse against the float64 oracle, on the index scores
    the library itself produces (dsa_indexer's, bit-identical to the ones the loss uses)."""
    cfg = S.CONFIGS["prefill_8k"]
    L = cfg.L
    _say(f"[indexer KL, dense warm-up] L={L}, every key up to each row")
    inp = S.make_prefill(cfg)
    qi, qs, ki, ks, w = indexer_inputs_dev(inp)
    q, kv = dev_bf16(inp.q), dev_bf16(inp.kv)
    kl, lse = dsa.indexer_kl_dense(qi, qs, ki, ks, w, q, kv, cfg.sm_scale, want_lse=True)
    kl2, _ = dsa.indexer_kl_dense(qi, qs, ki, ks, w, q, kv, cfg.sm_scale)
    scores = dsa.indexer(qi, qs, ki, ks, w)
    torch.cuda.synchronize()
    assert torch.equal(kl, kl2), "not deterministic"
    rng = np.random.default_rng(17)
    rows = np.array(sorted({0, 1, 31, 32, 2047, 2048, 4095, 6143, L - 1} | set(rng.integers(0, L, 24).tolist())))
    g_sc = scores[torch.from_numpy(rows).cuda()].cpu().numpy()
    del scores
    g_kl, g_lse = kl.cpu().numpy()[rows], lse.cpu().numpy()[rows]
    assert np.all(np.isfinite(kl.cpu().numpy())) and float(kl.min()) >= -1e-4
    W = O.widen_inputs(inp, rows)
    worst = _check_dense_rows(rows, rows, W["q"], W["kv"], g_sc, g_kl, g_lse, cfg.sm_scale)
    _say(f"  worst KL error / bound {worst:.3e} over {len(rows)} rows; mean KL {float(kl.mean()):.4f}")


def test_kl_dense_warmup_offsets_and_batch():
    """B = 2 sequences of 300 query rows at offsets -10 (rows before the first key: KL 0,
    lse -inf) and 2900 against 3000 keys (rows past the last key see every key)."""
    n_q, n_k = 300, 3000
    q_pos = [-10, 2900]
    _say(f"[indexer KL, dense warm-up] B=2, n_q={n_q}, n_k={n_k}, q_pos={q_pos}")
    cfg = S.CONFIGS["prefill_8k"].with_(L=n_k)
    inps = [S.make_prefill(cfg.with_(seed=90 + b)) for b in range(2)]
    rows = [np.clip(np.arange(p, p + n_q), 0, n_k - 1) for p in q_pos]
    qi = dev_u8(np.stack([inp.qi[r] for inp, r in zip(inps, rows)]))
    qs = dev_f32(np.stack([inp.q_scale[r] for inp, r in zip(inps, rows)]))
    w = dev_f32(np.stack([inp.w[r] for inp, r in zip(inps, rows)]))
    q = dev_bf16(np.stack([inp.q[r] for inp, r in zip(inps, rows)]))
    ki = dev_u8(np.stack([inp.ki for inp in inps]))
    ks = dev_f32(np.stack([inp.k_scale for inp in inps]))
    kv = dev_bf16(np.stack([inp.kv for inp in inps]))
    pos_d = torch.tensor(q_pos, dtype=torch.int32, device="cuda")
    kl, lse = dsa.indexer_kl_dense(qi, qs, ki, ks, w, q, kv, cfg.sm_scale, q_pos=pos_d, want_lse=True)
    scores = dsa.indexer(qi, qs, ki, ks, w, q_pos=pos_d)
    torch.cuda.synchronize()
    g_kl, g_lse, g_sc = kl.cpu().numpy(), lse.cpu().numpy(), scores.cpu().numpy()
    for b in range(2):
        pick = np.array([0, 5, 9, 10, 11, 99, 100, 101, 150, 299])
        W = O.widen_inputs(inps[b], rows[b][pick])
        _check_dense_rows(pick, q_pos[b] + pick, W["q"], W["kv"], g_sc[b][pick], g_kl[b][pick], g_lse[b][pick],
                          cfg.sm_scale)


def test_kl_dense_warmup_fp32_every_row():
    cfg = S.CONFIGS["tiny_fp32_512"]
    _say("[indexer KL, dense warm-up, fp32] L=512, every row")
    inp = S.make_prefill(cfg)
    qi, qs, ki, ks, w = indexer_inputs_dev(inp)
    q, kv = dev_f32(inp.q), dev_f32(inp.kv)
    kl, lse = dsa.indexer_kl_dense(qi, qs, ki, ks, w, q, kv, cfg.sm_scale, want_lse=True)
    scores = dsa.indexer(qi, qs, ki, ks, w)
    torch.cuda.synchronize()
    W = O.widen_inputs(inp)
    rows = np.arange(cfg.L)
    g_kl, g_lse, g_sc = kl.cpu().numpy(), lse.cpu().numpy(), scores.cpu().numpy()
    for t in rows:
        ids = np.arange(t + 1, dtype=np.int32)
        kl_ref, _ = O.indexer_kl_row(W["q"][t], W["kv"], ids, g_sc[t][: t + 1].astype(np.float64), cfg.sm_scale)
        assert abs(float(g_kl[t]) - kl_ref) <= 1e-5 * (1 + abs(kl_ref)), (t, float(g_kl[t]), kl_ref)
        _, l_ref = O.sparse_mqa_row(W["q"][t], W["kv"], W["kv"], ids, cfg.sm_scale)
        assert np.allclose(g_lse[t], l_ref, atol=1e-5, rtol=1e-6), t
