"""Float64 CPU oracle for the DSA layer: lightning indexer -> top-k -> sparse MLA (MQA).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import or call this module.  The library never does: it has no
CPU fallback.  This file shares no code with the HIP path (no helpers, tables or
constants); its only common ground with it is the seeded input generator, which holds
none of the arithmetic below.

Everything here is the plain definition, written out in float64 with numpy, in the
order the pages give the steps: score the preceding tokens with the lightning indexer,
keep the top-k of them, then run attention over the kept keys only.

Sources (page title, section):
  [P1] "DeepSeek-V3.2：用稀疏注意力和大规模智能体后训练，把开源大模型往前推"
       (paperbridge.wiki), sections "DeepSeek Sparse Attention：只让该看的部分参与注意力"
       and "论文证据": 2048 key-value tokens kept per query; core attention O(L^2) -> O(Lk);
       DSA runs in MLA's MQA mode.
  [P3] WeChat explainer reposted on juhe.plus, sections "第一步：Lightning Indexer" and
       "第二步：Fine-grained Token Selection": the indexer scores every history token,
       uses ReLU and may run in FP8; the top-k by those scores go to attention; k = 2048.
  [P4] "DeepSeek-V3.2-Exp 技术报告解读！..." (53ai.com), section
       "创新架构：DeepSeek稀疏注意力的核心设计" and Figure 1: index scores are taken between a
       query and its preceding tokens by a multi-head indexer with ReLU in FP8; the top-k
       key-value entries are then attended; in MQA mode one key-value entry serves every
       query head.
  [P5] "解析DeepSeek-V3.2核心技术：..." (yunpan.plus), section "1.1 DSA": the indexer scans
       all previous tokens in FP8.

Readings where the pages are silent (each is listed with its reason in the design notes):
  * index score:  I[t,s] = sum_j w[t,j] * ReLU(qhat[t,j] . khat[s]), where qhat/khat are
    the FP8 operands times their fp32 scales (the pages name multi-head + ReLU + weights
    implicitly; no 1/sqrt(d) factor: top-k is invariant to a positive scale);
  * "preceding tokens" includes s = t (so a first token has a key and k >= t+1 means dense
    causal attention);
  * ties in the top-k go to the lower key index; the kept set is emitted in ascending key
    order, padded with -1 when fewer than k keys exist;
  * attention logits are sm_scale * q . kv (sm_scale a parameter, 1/sqrt(d_qk) by default);
    V is kv[:, :d_v] unless a separate V is supplied; lse is the natural log-sum-exp of the
    scaled logits; an empty key set gives O = 0 and lse = -inf.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------------
# storage formats -> float64 (the oracle's own decoders)
# ----------------------------------------------------------------------------------------


def e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 E4M3FN code, from the format's definition.

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is subnormal
    (mantissa/8 * 2^-6); S.1111.111 is NaN; there is no infinity.
    """
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def fp8_to_f64(codes: np.ndarray) -> np.ndarray:
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (a bf16 is the high half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def dequant(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """FP8 codes times their fp32 scale (broadcast over the trailing axis), in float64."""
    return fp8_to_f64(codes) * np.asarray(scale, dtype=np.float64)[..., None]


# ----------------------------------------------------------------------------------------
# step 0: FP8 quantisation of the indexer operands  [P4 "创新架构"; P3 "第一步"; P5 "1.1 DSA"]
# ----------------------------------------------------------------------------------------
# The pages say the indexer runs in FP8 and give no quantiser.  Reading: one fp32 scale per
# row (a key; a query token over all its heads), scale = amax / 448 (1 for an all-zero
# row), code = the E4M3FN value nearest to x / scale, ties to the even mantissa,
# saturating at +-448.  Where floating point decides the code, the decision is taken in
# fp32 as the kernel takes it: scale and x / scale are correctly rounded fp32 divisions.


def _e4m3fn_positive_grid() -> tuple:
    """The finite non-negative E4M3FN values in increasing order, and their codes."""
    codes = np.array([c for c in range(0x7F)], dtype=np.int64)  # 0x7F is NaN
    return E4M3FN_TABLE[codes], codes


def e4m3fn_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code of each finite value, ties to the even mantissa (even code),
    saturating at +-448; the sign bit follows the value's sign (so -0.0 -> 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    vals, codes = _e4m3fn_positive_grid()
    a = np.minimum(np.abs(v), vals[-1])
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    mag = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    return mag | (np.signbit(v).astype(np.uint8) << np.uint8(7))


def fp8_quantize_row(x: np.ndarray) -> tuple:
    """One row (any shape, all its values share the scale): (codes uint8, scale fp32)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    scale = np.float32(amax) / np.float32(448.0) if amax > 0 else np.float32(1.0)
    q = x32 / scale  # fp32 division, correctly rounded
    return e4m3fn_encode(q.astype(np.float64)), np.float32(scale)


def fp8_quantize_rows(x: np.ndarray) -> tuple:
    """Rows along the first axis: (codes of x's shape, scales [n_rows] fp32)."""
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[0], dtype=np.float32)
    for r in range(x.shape[0]):
        codes[r], scales[r] = fp8_quantize_row(x[r])
    return codes, scales


# ----------------------------------------------------------------------------------------
# step 1: lightning indexer  [P3 "第一步"; P4 "创新架构"; P5 "1.1 DSA"]
# ----------------------------------------------------------------------------------------


def indexer_row(qhat_t: np.ndarray, w_t: np.ndarray, khat: np.ndarray, pos: int) -> np.ndarray:
    """Index scores of one query against keys 0..pos.

    qhat_t [H_I, d_I], w_t [H_I], khat [n_k, d_I] (float64, already dequantised).
    Returns I [pos+1]: I[s] = sum_j w_t[j] * max(0, qhat_t[j] . khat[s]).
    """
    x = qhat_t @ khat[: pos + 1].T                 # [H_I, pos+1]: per-head dot products
    return w_t @ np.maximum(x, 0.0)                # weighted sum of the ReLU'd head scores


def indexer_magnitude_row(qhat_t, w_t, khat, pos) -> np.ndarray:
    """sum_j |w_t[j]| * max(0, qhat_t[j] . khat[s]): the size the score tolerance is relative to."""
    x = qhat_t @ khat[: pos + 1].T
    return np.abs(w_t) @ np.maximum(x, 0.0)


def indexer(qhat: np.ndarray, w: np.ndarray, khat: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Dense score matrix for query rows with absolute positions ``pos`` (causal mask: -inf).

    qhat [n_q, H_I, d_I], w [n_q, H_I], khat [n_k, d_I]; returns [n_q, n_k] float64.
    """
    n_q, n_k = qhat.shape[0], khat.shape[0]
    out = np.full((n_q, n_k), -np.inf)
    for i in range(n_q):
        p = int(pos[i])
        if p >= 0:
            out[i, : p + 1] = indexer_row(qhat[i], w[i], khat, min(p, n_k - 1))
    return out


# ----------------------------------------------------------------------------------------
# step 2: fine-grained top-k selection  [P1 "DeepSeek Sparse Attention"; P3 "第二步"]
# ----------------------------------------------------------------------------------------


def topk_row(scores: np.ndarray, pos: int, k: int) -> np.ndarray:
    """Top-k of keys 0..pos by (score descending, key index ascending), as int32 [k].

    The kept indices are emitted in ascending order and padded with -1.  A full sort is
    the definition; -0.0 and +0.0 compare equal, as floats do.  A query at a negative
    position has no key before it and keeps nothing.
    """
    n = max(0, min(pos + 1, scores.shape[0]))
    s = np.arange(n)
    order = np.lexsort((s, -np.asarray(scores[:n], dtype=np.float64)))   # primary: -score
    keep = np.sort(order[: min(k, n)])
    out = np.full(k, -1, dtype=np.int32)
    out[: len(keep)] = keep
    return out


def topk(scores: np.ndarray, pos: np.ndarray, k: int) -> np.ndarray:
    return np.stack([topk_row(scores[i], int(pos[i]), k) for i in range(scores.shape[0])])


def topk_row_bruteforce(scores, pos: int, k: int) -> list:
    """Pure-Python version of ``topk_row`` for tiny inputs (pins the numpy sort)."""
    n = max(0, min(pos + 1, len(scores)))
    ranked = sorted(range(n), key=lambda s: (-float(scores[s]), s))
    keep = sorted(ranked[: min(k, n)])
    return keep + [-1] * (k - len(keep))


# ----------------------------------------------------------------------------------------
# step 3: attention over the kept keys, MLA in MQA mode  [P1; P4 "创新架构", Figure 1]
# ----------------------------------------------------------------------------------------


def sparse_mqa_row(q_t: np.ndarray, kv: np.ndarray, v: np.ndarray, idx_t: np.ndarray,
                   sm_scale: float) -> tuple:
    """Attention of every head of one query over the keys listed in idx_t (-1 = unused).

    q_t [H, d_qk], kv [n_k, d_qk] (shared by all heads), v [n_k, d_v].
    Returns O [H, d_v] and lse [H].
    """
    sel = idx_t[idx_t >= 0]
    H = q_t.shape[0]
    if len(sel) == 0:
        return np.zeros((H, v.shape[1])), np.full(H, -np.inf)
    z = sm_scale * (q_t @ kv[sel].T)               # [H, |S|]
    m = z.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
    p = np.exp(z - lse[:, None])
    return p @ v[sel], lse


def sparse_mqa(q: np.ndarray, kv: np.ndarray, v: np.ndarray, idx: np.ndarray,
               sm_scale: float) -> tuple:
    outs = [sparse_mqa_row(q[i], kv, v, idx[i], sm_scale) for i in range(q.shape[0])]
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


def sparse_mqa_backward(q: np.ndarray, kv: np.ndarray, v: np.ndarray, idx: np.ndarray, d_out: np.ndarray,
                        sm_scale: float, v_in_kv: bool) -> tuple:
    """Gradients of ``sparse_mqa`` for the loss sum(O * d_out), by the chain rule through the
    softmax over each row's kept keys (the sparse training stage trains the main model on
    the selected keys: P3 "阶段二：Sparse Training"; P4 "持续预训练").

    q [n_q, H, d_qk], kv [n_k, d_qk], v [n_k, d_v], idx [n_q, k] (-1 = unused; a repeated id
    counts once per slot), d_out [n_q, H, d_v].  Returns (dq, dkv, dv): dkv sums every
    query's contribution to each key row; with ``v_in_kv`` (V = kv[:, :d_v]) the value
    gradient is added into dkv[:, :d_v] and dv is None.
    """
    n_q = q.shape[0]
    dq = np.zeros_like(q, dtype=np.float64)
    dkv = np.zeros(kv.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for i in range(n_q):
        sel = idx[i][(idx[i] >= 0) & (idx[i] < kv.shape[0])]
        if len(sel) == 0:
            continue
        z = sm_scale * (q[i] @ kv[sel].T)                       # [H, |S|]
        P = np.exp(z - _logsumexp(z, axis=1)[:, None])         # softmax over the kept keys
        dP = d_out[i] @ v[sel].T                                # dL/dP
        dZ = P * (dP - np.sum(P * dP, axis=1, keepdims=True))   # through the softmax
        dq[i] = sm_scale * (dZ @ kv[sel])
        np.add.at(dkv, sel, sm_scale * (dZ.T @ q[i]))
        np.add.at(dv, sel, P.T @ d_out[i])
    if v_in_kv:
        dkv[:, : v.shape[1]] += dv
        return dq, dkv, None
    return dq, dkv, dv


def dense_causal_mqa(q: np.ndarray, kv: np.ndarray, v: np.ndarray, pos: np.ndarray,
                     sm_scale: float) -> tuple:
    """Ordinary causal attention (every head attends to keys 0..pos) for comparison."""
    outs = []
    for i in range(q.shape[0]):
        idx = np.arange(int(pos[i]) + 1, dtype=np.int32)
        outs.append(sparse_mqa_row(q[i], kv, v, idx, sm_scale))
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


# ----------------------------------------------------------------------------------------
# indexer KL-alignment loss  [P3 "阶段一：Dense Warm-up", "阶段二：Sparse Training";
#                             P4 "持续预训练"; P2 "DeepSeek Sparse Attention (DSA)"]
# ----------------------------------------------------------------------------------------


def _logsumexp(x: np.ndarray, axis=None) -> np.ndarray:
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return np.squeeze(m, axis=axis) + np.log(np.sum(np.exp(x - m), axis=axis))


def indexer_kl_row(q_t: np.ndarray, kv: np.ndarray, idx_t: np.ndarray, scores_t: np.ndarray,
                   sm_scale: float) -> tuple:
    """The indexer's KL loss for one query over its key set S (the valid ids of idx_t).

    Target: the main attention's distribution, summed over the heads and L1-normalised,
    p(s) = (1/H) sum_h softmax_{s in S}(sm_scale q_h . kv_s).  Indexer side: the softmax
    over S of the index scores scores_t (one per slot of idx_t).  Returns
    (sum_{s in S} p(s) (ln p(s) - ln q(s)), p per slot (0 for ids outside the keys)).
    An empty S gives (0, zeros).  The dense warm-up is the case S = {0, .., t}.
    """
    idx_t = np.asarray(idx_t)
    valid = (idx_t >= 0) & (idx_t < kv.shape[0])
    p_slots = np.zeros(idx_t.shape[0])
    if not valid.any():
        return 0.0, p_slots
    z = sm_scale * (q_t @ kv[idx_t[valid]].T)                 # [H, |S|]
    P = np.exp(z - _logsumexp(z, axis=1)[:, None])           # each head's softmax over S
    p = P.sum(axis=0) / P.sum()                              # summed over heads, L1-normalised
    I = np.asarray(scores_t, dtype=np.float64)[valid]
    log_q = I - _logsumexp(I)
    pos = p > 0
    kl = float(np.sum(p[pos] * (np.log(p[pos]) - log_q[pos])))
    p_slots[valid] = p
    return kl, p_slots


# ----------------------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------------------


def dsa_rows(qhat, w, khat, q, kv, v, pos, k: int, sm_scale: float) -> dict:
    """Indexer -> top-k -> sparse attention for query rows at absolute positions ``pos``.

    All arrays float64.  Returns scores (the rows' index scores, -inf beyond pos), idx,
    O and lse.
    """
    scores = indexer(qhat, w, khat, pos)
    idx = topk(scores, pos, k)
    o, lse = sparse_mqa(q, kv, v, idx, sm_scale)
    return {"scores": scores, "idx": idx, "out": o, "lse": lse}


def widen_inputs(inp, rows_sel=None) -> dict:
    """Storage-format inputs (as the generator returns them) -> float64 operands.

    Works on one prefill sequence; pass ``rows_sel`` to keep a subset of its query rows.
    """
    cfg = inp.cfg
    sel = slice(None) if rows_sel is None else rows_sel
    if cfg.fp32:
        qhat = inp.qi[sel].astype(np.float64) * inp.q_scale[sel].astype(np.float64)[..., None]
        khat = inp.ki.astype(np.float64) * inp.k_scale.astype(np.float64)[:, None]
        q = inp.q[sel].astype(np.float64)
        kv = inp.kv.astype(np.float64)
        v = inp.v.astype(np.float64) if inp.v is not None else kv[:, : cfg.d_v]
    else:
        qhat = dequant(inp.qi[sel], inp.q_scale[sel])
        khat = dequant(inp.ki, inp.k_scale)
        q = bf16_to_f64(inp.q[sel])
        kv = bf16_to_f64(inp.kv)
        v = bf16_to_f64(inp.v) if inp.v is not None else kv[:, : cfg.d_v]
    return {"qhat": qhat, "w": inp.w[sel].astype(np.float64), "khat": khat, "q": q,
            "kv": kv, "v": v}
