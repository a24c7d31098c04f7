"""Seeded synthetic inputs for the DSA layer (indexer -> top-k -> sparse MLA).

This module draws random numbers and rounds them into the storage formats the
library consumes: bf16 bit patterns, FP8 E4M3FN codes with per-token fp32 scales,
or plain fp32.  It holds none of the attention arithmetic.  The GPU tests, the
benchmark and the float64 oracle all consume exactly what it returns, so both
sides see bit-identical inputs.

Determinism and addressability
------------------------------
Every tensor is cut into blocks of ``BLOCK`` = 64 rows.  Block ``b`` of tensor
``tid`` (of sequence ``seq``) is drawn from its own Philox stream keyed by
``SeedSequence([seed, tid, seq, b])``, so any row block can be regenerated alone
(the oracle re-draws only the query rows it checks at 128K).  Draws are float32
normals; the planted mix is evaluated in float32 and then rounded once into the
storage format (bf16 RNE, or FP8 E4M3FN RNE after the per-token scale).

Workload structure (used where ``Config.planted``)
--------------------------------------------------
Queries come in blocks of 64 consecutive tokens.  Block ``b >= 1`` owns a unit
direction ``u_b`` in the indexer space (d_I) and ``u'_b`` in the attention space
(d_qk), and plants itself in 64 earlier keys drawn without replacement from
``[0, 64 b)`` (a key claimed by several blocks belongs to the latest).  Every
indexer head and every attention head of the block's queries, and the owned
rows of k_I and kv, are ``sqrt(.5) sqrt(d) u + sqrt(.5) n`` with ``n ~ N(0, I)``:
unit-variance marginals and an expected cosine of 0.5 between a query and its
planted keys.  Decode plants 64 keys per sequence for its single query.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Optional, Sequence

import numpy as np

BLOCK = 64

# stream identifiers (part of the seed key; never reorder)
T_QI, T_KI, T_W, T_Q, T_KV, T_V, T_PLANT, T_DIR_I, T_DIR_Q = range(1, 10)


@dataclass(frozen=True)
class Config:
    """One DSA workload: shapes, dtypes and the synthetic recipe."""

    name: str
    L: int                 # keys per sequence (prefill: also the number of queries)
    batch: int             # sequences (decode) or 1 (prefill)
    H: int                 # attention query heads (all share one KV row: MQA)
    d_qk: int              # q / kv row width
    d_v: int               # value width (kv[:, :d_v] unless v_separate)
    H_I: int               # indexer heads
    d_I: int               # indexer head width
    k: int                 # keys kept per query
    fp32: bool             # fp32 indexer and attention (else FP8 indexer, bf16 attention)
    decode: bool           # one query per sequence at position L-1
    planted: bool          # plant correlated keys (see module docstring)
    v_separate: bool       # separate V tensor instead of kv[:, :d_v]
    qkv_std: float = 1.0   # std of q, kv (and v)
    w_std: Optional[float] = None   # std of w; default 1/sqrt(H_I)
    seed: int = 0

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    @property
    def w_sigma(self) -> float:
        return self.w_std if self.w_std is not None else 1.0 / math.sqrt(self.H_I)

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    "tiny_fp32_512": Config("tiny_fp32_512", L=512, batch=1, H=4, d_qk=64, d_v=64, H_I=2,
                            d_I=32, k=64, fp32=True, decode=False, planted=False,
                            v_separate=True, qkv_std=1.0 / 8, w_std=1.0 / math.sqrt(2)),
    "prefill_8k": Config("prefill_8k", L=8192, batch=1, H=128, d_qk=576, d_v=512, H_I=64,
                         d_I=128, k=2048, fp32=False, decode=False, planted=True,
                         v_separate=False),
    "prefill_32k": Config("prefill_32k", L=32768, batch=1, H=128, d_qk=576, d_v=512, H_I=64,
                          d_I=128, k=2048, fp32=False, decode=False, planted=True,
                          v_separate=False),
    "prefill_128k": Config("prefill_128k", L=131072, batch=1, H=128, d_qk=576, d_v=512,
                           H_I=64, d_I=128, k=2048, fp32=False, decode=False, planted=True,
                           v_separate=False),
    "decode_64x128k": Config("decode_64x128k", L=131072, batch=64, H=128, d_qk=576, d_v=512,
                             H_I=64, d_I=128, k=2048, fp32=False, decode=True, planted=True,
                             v_separate=False),
}
CONFIG_ORDER = ["tiny_fp32_512", "prefill_8k", "prefill_32k", "prefill_128k", "decode_64x128k"]


# ----------------------------------------------------------------------------------------
# storage-format rounding (input preparation only)
# ----------------------------------------------------------------------------------------

FP8_MAX = 448.0


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return the bit patterns.

    Inputs are finite.  Works on the fp32 bit pattern: add 0x7FFF plus the lowest kept
    bit, then drop the low 16 bits (a carry into the exponent is the correct rounding).
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def fp8_e4m3fn_codes(x: np.ndarray) -> np.ndarray:
    """Encode float64 values as OCP FP8 E4M3FN codes: round-to-nearest-even, saturate at 448."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), FP8_MAX)
    # quantum of the binade a falls in (normals: 3 mantissa bits; subnormals: 2^-9)
    _, e = np.frexp(a)                       # a = m * 2^e, m in [0.5, 1)
    e = np.maximum(e - 1, -6)                # unbiased exponent, clamped to the subnormal binade
    q = np.ldexp(1.0, e - 3)
    y = np.rint(a / q) * q                   # np.rint rounds half to even
    y = np.minimum(y, FP8_MAX)
    # pack y into bits
    _, ey = np.frexp(y)
    ey = ey - 1
    normal = y >= 2.0 ** -6
    expf = np.where(normal, ey + 7, 0)
    mant = np.where(normal, y / np.ldexp(1.0, ey) - 1.0, y / 2.0 ** -9) * np.where(normal, 8, 1)
    mant = np.rint(mant).astype(np.int64)
    code = (np.where(y == 0, 0, (expf << 3) | mant)).astype(np.uint8)
    return code | (sign.astype(np.uint8) << np.uint8(7))


def fp8_quantize_rows(x: np.ndarray, n_axes: int) -> tuple:
    """Per-row FP8 quantisation: one scale per leading index over the last ``n_axes`` axes.

    scale = amax / 448 (1.0 where amax == 0); code = E4M3FN(x / scale).
    Returns (codes uint8, scales float32).  The scale is rounded to fp32 first and the
    codes are computed from that fp32 scale, so code * scale is what both sides use.
    """
    x = np.asarray(x, dtype=np.float64)
    axes = tuple(range(x.ndim - n_axes, x.ndim))
    amax = np.max(np.abs(x), axis=axes)
    scale = np.where(amax > 0, amax / FP8_MAX, 1.0).astype(np.float32)
    sc = scale.astype(np.float64).reshape(scale.shape + (1,) * n_axes)
    return fp8_e4m3fn_codes(x / sc), scale


# ----------------------------------------------------------------------------------------
# streams
# ----------------------------------------------------------------------------------------

def _rng(seed: int, tid: int, seq: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([seed, tid, seq, block])))


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _normal_rows(cfg: Config, tid: int, seq: int, rows: np.ndarray, width: tuple) -> np.ndarray:
    """N(0,1) float64 rows ``rows`` (sorted unique) of tensor ``tid`` with trailing shape ``width``."""
    out = np.empty((len(rows),) + width, dtype=np.float32)
    blocks = np.unique(rows // BLOCK)
    for b in blocks:
        sel = np.nonzero(rows // BLOCK == b)[0]
        blk = _rng(cfg.seed, tid, seq, int(b)).standard_normal((BLOCK,) + width, dtype=np.float32)
        out[sel] = blk[rows[sel] - b * BLOCK]
    return out


def _unit(cfg: Config, tid: int, seq: int, block: int, d: int) -> np.ndarray:
    u = _rng(cfg.seed, tid, seq, block).standard_normal(d)
    return (u / np.linalg.norm(u)).astype(np.float32)


def plant_owner(cfg: Config, seq: int = 0) -> np.ndarray:
    """owner[s] = query block whose direction key s carries, or -1 (prefill layout).

    For decode the single query of each sequence plants 64 keys in [0, L-1); owner is 0
    for those.
    """
    owner = np.full(cfg.L, -1, dtype=np.int64)
    if not cfg.planted:
        return owner
    if cfg.decode:
        pos = _rng(cfg.seed, T_PLANT, seq, 0).choice(cfg.L - 1, size=min(64, cfg.L - 1),
                                                     replace=False)
        owner[pos] = 0
        return owner
    nblk = (cfg.L + BLOCK - 1) // BLOCK
    for b in range(1, nblk):
        pos = _rng(cfg.seed, T_PLANT, seq, b).choice(BLOCK * b, size=BLOCK, replace=False)
        owner[pos] = b
    return owner


def _query_block_of(cfg: Config, rows: np.ndarray) -> np.ndarray:
    if cfg.decode:
        return np.zeros_like(rows)
    return rows // BLOCK


def _mix(n: np.ndarray, u: np.ndarray, d: int) -> np.ndarray:
    """sqrt(.5) sqrt(d) u + sqrt(.5) n, evaluated in float32 (n is overwritten)."""
    n *= np.float32(math.sqrt(0.5))
    n += np.float32(math.sqrt(0.5) * math.sqrt(d)) * u
    return n


# ----------------------------------------------------------------------------------------
# float32 draws (before rounding)
# ----------------------------------------------------------------------------------------

def draw_query_rows(cfg: Config, rows: Sequence[int], seq: int = 0) -> dict:
    """float32 query-side rows (before rounding): qi [n, H_I, d_I], w [n, H_I], q [n, H, d_qk].

    For decode, ``rows`` must be [0] (the single query of sequence ``seq``).
    """
    rows = np.asarray(rows, dtype=np.int64)
    qi = _normal_rows(cfg, T_QI, seq, rows, (cfg.H_I, cfg.d_I))
    w = _normal_rows(cfg, T_W, seq, rows, (cfg.H_I,)) * np.float32(cfg.w_sigma)
    q = _normal_rows(cfg, T_Q, seq, rows, (cfg.H, cfg.d_qk))
    if cfg.planted:
        qb = _query_block_of(cfg, rows)
        for b in np.unique(qb):
            if b == 0 and not cfg.decode:
                continue
            sel = np.nonzero(qb == b)[0]
            lo, hi = sel[0], sel[-1] + 1
            if hi - lo == len(sel):       # contiguous rows: mix in place
                _mix(qi[lo:hi], _unit(cfg, T_DIR_I, seq, int(b), cfg.d_I), cfg.d_I)
                _mix(q[lo:hi], _unit(cfg, T_DIR_Q, seq, int(b), cfg.d_qk), cfg.d_qk)
            else:
                qi[sel] = _mix(qi[sel], _unit(cfg, T_DIR_I, seq, int(b), cfg.d_I), cfg.d_I)
                q[sel] = _mix(q[sel], _unit(cfg, T_DIR_Q, seq, int(b), cfg.d_qk), cfg.d_qk)
    q *= np.float32(cfg.qkv_std)
    return {"qi": qi, "w": w, "q": q}


def draw_key_rows(cfg: Config, seq: int = 0, rows: Optional[np.ndarray] = None) -> dict:
    """float32 key-side rows (before rounding): ki [n, d_I], kv [n, d_qk], v [n, d_v] (v only if v_separate)."""
    if rows is None:
        rows = np.arange(cfg.L, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    ki = _normal_rows(cfg, T_KI, seq, rows, (cfg.d_I,))
    kv = _normal_rows(cfg, T_KV, seq, rows, (cfg.d_qk,))
    if cfg.planted:
        owner = plant_owner(cfg, seq)[rows]
        for b in np.unique(owner[owner >= 0]):
            sel = owner == b
            ki[sel] = _mix(ki[sel], _unit(cfg, T_DIR_I, seq, int(b), cfg.d_I), cfg.d_I)
            kv[sel] = _mix(kv[sel], _unit(cfg, T_DIR_Q, seq, int(b), cfg.d_qk), cfg.d_qk)
    kv *= np.float32(cfg.qkv_std)
    out = {"ki": ki, "kv": kv}
    if cfg.v_separate:
        out["v"] = _normal_rows(cfg, T_V, seq, rows, (cfg.d_v,)) * np.float32(cfg.qkv_std)
    return out


# ----------------------------------------------------------------------------------------
# rounded inputs, as the library consumes them
# ----------------------------------------------------------------------------------------

@dataclass
class Inputs:
    """One sequence's (prefill) or one batch's (decode) inputs in storage formats.

    fp32 configs: qi/ki/q/kv/v are float32 arrays and the FP8 scales are all 1.
    Otherwise: qi [n, H_I, d_I] and ki [L, d_I] are uint8 E4M3FN codes with fp32 scales
    q_scale [n, H_I] (one per token, repeated over heads) and k_scale [L]; q [n, H, d_qk]
    and kv [L, d_qk] are uint16 bf16 bit patterns; v is None (V = kv[:, :d_v]).
    Decode inputs carry a leading batch axis on every array.
    """

    cfg: Config
    rows: np.ndarray
    qi: np.ndarray
    q_scale: np.ndarray
    w: np.ndarray
    q: np.ndarray
    ki: Optional[np.ndarray] = None
    k_scale: Optional[np.ndarray] = None
    kv: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None


def _round_query(cfg: Config, d: dict) -> tuple:
    if cfg.fp32:
        qi = d["qi"].astype(np.float32)
        q_scale = np.ones(qi.shape[:2], dtype=np.float32)
        q = d["q"].astype(np.float32)
    else:
        qi, s = fp8_quantize_rows(d["qi"], 2)
        q_scale = np.repeat(s[:, None], cfg.H_I, axis=1)
        q = bf16_bits(d["q"])
    return qi, q_scale, d["w"].astype(np.float32), q


def _round_keys(cfg: Config, d: dict) -> tuple:
    if cfg.fp32:
        ki = d["ki"].astype(np.float32)
        k_scale = np.ones(ki.shape[0], dtype=np.float32)
        kv = d["kv"].astype(np.float32)
        v = d["v"].astype(np.float32) if "v" in d else None
    else:
        ki, k_scale = fp8_quantize_rows(d["ki"], 1)
        kv = bf16_bits(d["kv"])
        v = bf16_bits(d["v"]) if "v" in d else None
    return ki, k_scale, kv, v


def query_rows(cfg: Config, rows: Sequence[int], seq: int = 0) -> tuple:
    """Rounded (qi, q_scale, w, q) for the given query rows; blocks are drawn in parallel."""
    rows = np.asarray(rows, dtype=np.int64)
    if len(rows) <= 4 * BLOCK:
        return _round_query(cfg, draw_query_rows(cfg, rows, seq))
    chunks = np.array_split(rows, max(1, (len(rows) + 4 * BLOCK - 1) // (4 * BLOCK)))
    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(lambda r: _round_query(cfg, draw_query_rows(cfg, r, seq)), chunks))
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(4))


def key_rows(cfg: Config, seq: int = 0) -> tuple:
    """Rounded (ki, k_scale, kv, v) for all L key rows of sequence ``seq``."""
    rows = np.arange(cfg.L, dtype=np.int64)
    if cfg.L <= 8 * BLOCK:
        return _round_keys(cfg, draw_key_rows(cfg, seq, rows))
    chunks = np.array_split(rows, (cfg.L + 16 * BLOCK - 1) // (16 * BLOCK))
    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(lambda r: _round_keys(cfg, draw_key_rows(cfg, seq, r)), chunks))
    out = []
    for i in range(4):
        out.append(None if parts[0][i] is None else np.concatenate([p[i] for p in parts]))
    return tuple(out)


def make_prefill(cfg: Config, rows: Optional[Sequence[int]] = None) -> Inputs:
    """Prefill inputs of one sequence; ``rows`` restricts the query side (default: all L)."""
    assert not cfg.decode
    rows = np.arange(cfg.L, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    qi, q_scale, w, q = query_rows(cfg, rows)
    ki, k_scale, kv, v = key_rows(cfg)
    return Inputs(cfg, rows, qi, q_scale, w, q, ki, k_scale, kv, v)


def make_decode(cfg: Config, seqs: Optional[Sequence[int]] = None, with_keys: bool = True) -> Inputs:
    """Decode inputs: one query per sequence at position L-1, caches of L rows each."""
    assert cfg.decode
    seqs = list(range(cfg.batch)) if seqs is None else list(seqs)
    qparts = [query_rows(cfg, [0], s) for s in seqs]
    qi, q_scale, w, q = (np.stack([p[i][0] for p in qparts]) for i in range(4))
    inp = Inputs(cfg, np.asarray(seqs), qi, q_scale, w, q)
    if with_keys:
        kparts = [key_rows(cfg, s) for s in seqs]
        inp.ki = np.stack([p[0] for p in kparts])
        inp.k_scale = np.stack([p[1] for p in kparts])
        inp.kv = np.stack([p[2] for p in kparts])
        inp.v = None if kparts[0][3] is None else np.stack([p[3] for p in kparts])
    return inp
