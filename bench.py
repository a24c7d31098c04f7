"""Benchmark of the DSA layer on one MI355X: prefill tokens/s at L = 131072, k = 2048
(lightning indexer + top-k + sparse MLA), plus decode microseconds per step for 64
sequences of 131072 cached tokens.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_128k]
                    [--decode-workload decode_64x128k | none] [--no-cpu-baseline]
                    [--other-workloads prefill_8k,prefill_32k | none]

Prints ONE JSON line.  Inputs are seeded synthetic tensors from the generator shared with
the tests, already resident in HBM when timing starts.  A step is one call of
dsa_forward_prefill over the whole sequence; `value` is the sequence length over the mean
step time of the K timed steps (their median and minimum are reported beside it).  The
roofline object describes the slower of the two prefill stages, timed separately with HIP
events on the stream they run on.  The 8K and 32K prefill rates and the decode step time
are reported as fields of the same line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA prefill tokens/s at L=128K, k=2048 (indexer+top-k+sparse MLA); decode µs/step"
PEAK_FP8 = 5.0e15      # MI355X dense FP8 MFMA, flop/s
PEAK_BF16 = 2.5e15     # MI355X dense BF16 MFMA, flop/s
PEAK_HBM = 8.0e12      # MI355X HBM3E, bytes/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------ inputs

def prefill_inputs_on_gpu(cfg, torch):
    """Stream the generator's row blocks straight into device tensors."""
    from sparse_attention_long_02_amd import synth as S
    L = cfg.L
    dev = "cuda"
    qi = torch.empty((L, cfg.H_I, cfg.d_I), dtype=torch.uint8, device=dev)
    qs = torch.empty((L, cfg.H_I), dtype=torch.float32, device=dev)
    w = torch.empty((L, cfg.H_I), dtype=torch.float32, device=dev)
    q = torch.empty((L, cfg.H, cfg.d_qk), dtype=torch.bfloat16, device=dev)
    step = 8192
    t0 = time.time()
    for r0 in range(0, L, step):
        rows = np.arange(r0, min(L, r0 + step))
        a, b, c, d = S.query_rows(cfg, rows)
        sl = slice(r0, r0 + len(rows))
        qi[sl].copy_(torch.from_numpy(a))
        qs[sl].copy_(torch.from_numpy(b))
        w[sl].copy_(torch.from_numpy(c))
        q[sl].copy_(torch.from_numpy(d.view(np.int16)).view(torch.bfloat16))
    ki, ks, kv, _ = S.key_rows(cfg)
    ki = torch.from_numpy(ki).to(dev)
    ks = torch.from_numpy(ks).to(dev)
    kv = torch.from_numpy(kv.view(np.int16)).to(dev).view(torch.bfloat16)
    torch.cuda.synchronize()
    log(f"[bench] generated {cfg.name} inputs in {time.time() - t0:.1f}s")
    return qi, qs, ki, ks, w, q, kv


def decode_inputs_on_gpu(cfg, torch):
    from sparse_attention_long_02_amd import synth as S
    dev = "cuda"
    t0 = time.time()
    inp = S.make_decode(cfg, with_keys=False)
    kc = torch.empty((cfg.batch, cfg.L, cfg.d_I), dtype=torch.uint8, device=dev)
    kcs = torch.empty((cfg.batch, cfg.L), dtype=torch.float32, device=dev)
    kvc = torch.empty((cfg.batch, cfg.L, cfg.d_qk), dtype=torch.bfloat16, device=dev)
    for b in range(cfg.batch):
        ki, ks, kv, _ = S.key_rows(cfg, b)
        kc[b].copy_(torch.from_numpy(ki))
        kcs[b].copy_(torch.from_numpy(ks))
        kvc[b].copy_(torch.from_numpy(kv.view(np.int16)).view(torch.bfloat16))
    qi = torch.from_numpy(inp.qi).to(dev)
    qs = torch.from_numpy(inp.q_scale).to(dev)
    w = torch.from_numpy(inp.w).to(dev)
    q = torch.from_numpy(inp.q.view(np.int16)).to(dev).view(torch.bfloat16)
    ctx = torch.full((cfg.batch,), cfg.L, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] generated {cfg.name} inputs in {time.time() - t0:.1f}s")
    return ctx, qi, qs, w, kc, kcs, q, kvc


# ------------------------------------------------------------------------------ work model

def indexer_flops(L, H_I, d_I):
    """sum over tokens t of (t+1) * H_I * d_I * 2 (every causal pair, all heads)."""
    return L * (L + 1) / 2 * H_I * d_I * 2


def kept_keys(L, k):
    """sum over tokens t of min(t+1, k)."""
    m = min(L, k)
    return m * (m + 1) / 2 + max(0, L - k) * k


def gather_bytes(L, k, d_qk):
    return kept_keys(L, k) * d_qk * 2


def mla_flops(L, k, H, d_qk, d_v):
    return kept_keys(L, k) * H * (d_qk + d_v) * 2


# ------------------------------------------------------------------------------ counters

def sources_sha256(paths):
    """sha256 over the named files (repository-relative, comma-separated) read in order."""
    import hashlib
    h = hashlib.sha256()
    for rel in paths.split(","):
        with open(os.path.join(ROOT, rel), "rb") as g:
            h.update(g.read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch recorded from the FETCH_SIZE / WRITE_SIZE counter passes under
    profiles/ (calibrated on a copy of known size), or None when none is recorded or the
    kernel's sources (its .hip file and the headers it includes) have changed since: their
    sha256 no longer matches."""
    import glob
    import re
    pat = re.compile(r"^traffic (\S+) (\S+) bytes=(\d+) source=(\S+) sha256=([0-9a-f]+)\s*$")
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                m = pat.match(line)
                if not m or m.group(1) != kernel or m.group(2) != workload:
                    continue
                if not all(os.path.exists(os.path.join(ROOT, r)) for r in m.group(4).split(",")):
                    return None
                if sources_sha256(m.group(4)) != m.group(5):
                    return None
                return int(m.group(3))
    return None


# ------------------------------------------------------------------------------ timing

def time_calls(torch, fn, reps):
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / reps


def time_each(torch, fn, reps):
    """Seconds of each of `reps` back-to-back calls (an event pair around every call, all on
    the current stream): (mean over the whole run, median, min)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(reps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    each = sorted(ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(reps))
    return ev[0].elapsed_time(ev[reps]) / 1e3 / reps, float(np.median(each)), each[0]


def prefill_rate(cfg, torch, dsa, warmup, reps):
    """Whole-layer prefill rate of one more workload (its own inputs, same entry point)."""
    qi, qs, ki, ks, w, q, kv = prefill_inputs_on_gpu(cfg, torch)
    L, k = cfg.L, cfg.k
    idx = torch.empty((L, k), dtype=torch.int32, device="cuda")
    out = torch.empty((L, cfg.H, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((L, cfg.H), dtype=torch.float32, device="cuda")
    ws_n = dsa.workspace_size(dsa.DSA_OP_PREFILL, 1, L, L, cfg.H, cfg.d_v, k, dsa.DSA_BF16)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda") if ws_n else None

    def step():
        dsa.forward_prefill(qi, qs, ki, ks, w, q, kv, k, cfg.sm_scale, cfg.d_v, idx=idx, out=out, lse=lse, ws=ws)
    for _ in range(warmup):
        step()
    mean, med, mn = time_each(torch, step, reps)
    return {"workload": cfg.name, "seq_len": L, "tokens_per_s": L / mean, "ms_per_step": mean * 1e3,
            "ms_median": med * 1e3, "ms_min": mn * 1e3, "steps": reps, "warmup": warmup}


def cpu_baseline(cfg, budget_s=15.0):
    """The float64 oracle, as it stands, on a bounded sample of query rows of the same
    workload: rows drawn uniformly from the sequence, whole layer per row, until about
    budget_s seconds of oracle time have been spent."""
    import oracle as O
    from sparse_attention_long_02_amd import synth as S
    rng = np.random.default_rng(1234)
    L, k = cfg.L, cfg.k
    t0 = time.time()
    ki, ks, kv, v = S.key_rows(cfg)
    khat = O.dequant(ki, ks)
    kvf = O.bf16_to_f64(kv)
    vf = kvf[:, : cfg.d_v]
    setup = time.time() - t0
    spent, n_rows = 0.0, 0
    while spent < budget_s:
        rows = np.sort(rng.integers(0, L, 64))
        qi, qs, w, q = S.query_rows(cfg, rows)
        qhat = O.dequant(qi, qs)
        qf = O.bf16_to_f64(q)
        for j, t in enumerate(rows):
            a = time.time()
            O.dsa_rows(qhat[j:j + 1], w[j:j + 1].astype(np.float64), khat, qf[j:j + 1], kvf, vf,
                       np.array([int(t)]), k, cfg.sm_scale)
            spent += time.time() - a
            n_rows += 1
            if spent >= budget_s:
                break
    cores = len(os.sched_getaffinity(0))
    return {"value": n_rows / spent, "unit": "tokens/s", "cores": cores, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{n_rows} query rows drawn uniformly from the {L}-token sequence (mean cost of a "
                      f"uniform row equals the per-token mean of the whole sequence); float64 numpy oracle, "
                      f"whole layer (indexer, top-k, attention) per row; tokens/s = rows / oracle seconds "
                      f"({spent:.1f}s of CPU work, key setup {setup:.1f}s not counted)"}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo; "unknown" where it is not readable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_128k")
    ap.add_argument("--decode-workload", default="decode_64x128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage-reps", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=8192, help="tokens of the chunked-prefill stage")
    ap.add_argument("--dense-kl", type=int, default=32768, help="rows of the dense warm-up KL stage (0: skip)")
    ap.add_argument("--other-workloads", default="prefill_8k,prefill_32k",
                    help="comma-separated prefill workloads also timed (whole layer), or none")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs the DSA layer on a single MI355X "
              "(the multi-GPU sharding is described in the design notes, not implemented).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_long_02_amd import dsa
    from sparse_attention_long_02_amd import synth as S

    cfg = S.CONFIGS[args.workload]
    assert not cfg.decode and not cfg.fp32
    dsa.lib()
    qi, qs, ki, ks, w, q, kv = prefill_inputs_on_gpu(cfg, torch)
    L, k = cfg.L, cfg.k
    idx = torch.empty((L, k), dtype=torch.int32, device="cuda")
    out = torch.empty((L, cfg.H, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((L, cfg.H), dtype=torch.float32, device="cuda")
    ws_n = dsa.workspace_size(dsa.DSA_OP_PREFILL, 1, L, L, cfg.H, cfg.d_v, k, dsa.DSA_BF16)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda") if ws_n else None

    def step():
        dsa.forward_prefill(qi, qs, ki, ks, w, q, kv, k, cfg.sm_scale, cfg.d_v, idx=idx, out=out, lse=lse, ws=ws)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    mean_s, med_s, min_s = time_each(torch, step, args.steps)
    wall = time.perf_counter() - t0
    ms_step = mean_s * 1e3
    log(f"[bench] {args.steps} timed steps: {ms_step:.3f} ms/step, median {med_s * 1e3:.3f}, "
        f"min {min_s * 1e3:.3f} (wall {wall:.2f}s)")

    # the two stages alone (same stream, HIP events)
    t_sel = time_calls(torch, lambda: dsa.select_prefill(qi, qs, ki, ks, w, k, idx=idx), args.stage_reps)
    t_mla = time_calls(torch, lambda: dsa.sparse_mla(q, kv, idx, cfg.sm_scale, cfg.d_v), args.stage_reps)
    log(f"[bench] stages: select {t_sel * 1e3:.3f} ms, sparse MLA {t_mla * 1e3:.3f} ms")
    f_idx = indexer_flops(L, cfg.H_I, cfg.d_I)
    g_bytes = gather_bytes(L, k, cfg.d_qk)
    f_mla = mla_flops(L, k, cfg.H, cfg.d_qk, cfg.d_v)
    stages = {
        "select": {"ms": t_sel * 1e3, "fp8_flop": f_idx, "mfma_frac": f_idx / t_sel / PEAK_FP8},
        "sparse_mla": {"ms": t_mla * 1e3, "gather_bytes": g_bytes, "hbm_frac": g_bytes / t_mla / PEAK_HBM,
                       "bf16_flop": f_mla, "mfma_frac": f_mla / t_mla / PEAK_BF16},
    }
    f_traffic = recorded_traffic("idx_dense_fp8_kernel_filter", cfg.name)
    n_chunks = -(-L // 16384)
    stages["select"]["filter_kernel_traffic_bytes_per_step"] = f_traffic * n_chunks if f_traffic else None
    if t_sel >= t_mla:
        # the selection stage as a whole (key sample, thresholds, filtering indexer and
        # candidate top-k per chunk of 16384 rows): its work over its time per step
        a = f_idx / t_sel
        roof = {"kernel": "threshold-filtered FP8 selection (idx_dense_fp8_kernel + sel_* kernels, one step)",
                "bound": "mfma", "achieved": a / 1e12, "peak": PEAK_FP8 / 1e12, "unit": "TFLOP/s",
                "frac": a / PEAK_FP8, "traffic": stages["select"]["filter_kernel_traffic_bytes_per_step"]}
    else:
        a = g_bytes / t_mla
        roof = {"kernel": "sparse_mla_bf16_kernel (gathered KV rows)", "bound": "hbm",
                "achieved": a / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": a / PEAK_HBM,
                "traffic": recorded_traffic("sparse_mla_bf16_kernel", cfg.name)}
    roof["traffic_unit"] = "bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE)"

    # the FP8 quantisation of the indexer operands (the step before the indexer; not part
    # of the metric, which starts from FP8 operands): seeded bf16 activations of the
    # workload's shape, quantised per query token (all its heads) and per key
    gq = torch.Generator(device="cuda").manual_seed(0)
    xq = torch.randn((L, cfg.H_I, cfg.d_I), generator=gq, device="cuda").to(torch.bfloat16)
    xk = torch.randn((L, cfg.d_I), generator=gq, device="cuda").to(torch.bfloat16)
    cq = torch.empty_like(xq, dtype=torch.uint8)
    sq = torch.empty((L, cfg.H_I), dtype=torch.float32, device="cuda")
    ck = torch.empty_like(xk, dtype=torch.uint8)
    sk = torch.empty((L, 1), dtype=torch.float32, device="cuda")

    def quant():
        dsa.fp8_quantize_rows(xq, repeat=cfg.H_I, codes=cq, scale=sq)
        dsa.fp8_quantize_rows(xk, codes=ck, scale=sk)
    quant()
    t_q = time_calls(torch, quant, args.stage_reps)
    q_bytes = L * (cfg.H_I * cfg.d_I * 3 + cfg.H_I * 4) + L * (cfg.d_I * 3 + 4)
    stages["quantize"] = {"ms": t_q * 1e3, "bytes": q_bytes, "hbm_frac": q_bytes / t_q / PEAK_HBM,
                          "note": "bf16 indexer activations -> FP8 codes + fp32 scales (q_I and k_I); "
                                  "not in the metric"}
    log(f"[bench] FP8 quantisation of q_I and k_I: {t_q * 1e3:.3f} ms ({q_bytes / t_q / 1e9:.0f} GB/s)")
    del xq, xk, cq, sq, ck, sk

    # chunked prefill: the sequence's last CHUNK tokens as one chunk against the cache that
    # holds all L rows (the most expensive chunk: its rows see the most keys)
    C = min(args.chunk, L)
    p0 = L - C
    pos_c = torch.tensor([p0], dtype=torch.int32, device="cuda")
    cidx = torch.empty((1, C, k), dtype=torch.int32, device="cuda")
    cout = torch.empty((1, C, cfg.H, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    clse = torch.empty((1, C, cfg.H), dtype=torch.float32, device="cuda")
    ws_c_n = dsa.workspace_size(dsa.DSA_OP_CHUNK, 1, C, L, cfg.H, cfg.d_v, k, dsa.DSA_BF16)
    ws_c = torch.empty(ws_c_n, dtype=torch.uint8, device="cuda") if ws_c_n else None

    def chunk():
        dsa.forward_chunk(pos_c, qi[None, p0:], qs[None, p0:], w[None, p0:], ki[None], ks[None], q[None, p0:],
                          kv[None], k, cfg.sm_scale, cfg.d_v, idx=cidx, out=cout, lse=clse, ws=ws_c)
    chunk()
    t_c = time_calls(torch, chunk, args.stage_reps)
    f_c = indexer_flops(L, cfg.H_I, cfg.d_I) - indexer_flops(p0, cfg.H_I, cfg.d_I)
    stages["chunk"] = {"ms": t_c * 1e3, "tokens": C, "q_pos": p0, "n_k": L, "tokens_per_s": C / t_c,
                       "indexer_fp8_flop": f_c, "indexer_mfma_frac_of_step": f_c / t_c / PEAK_FP8,
                       "note": "the last chunk of the sequence through dsa_forward_chunk"}
    log(f"[bench] chunk of {C} tokens at q_pos {p0}: {t_c * 1e3:.3f} ms ({C / t_c:.0f} tokens/s)")
    del cidx, cout, clse, ws_c

    # indexer KL loss of the sparse training stage over this step's selection: the index
    # scores of the selected keys, then the loss (one pass over the gathered rows)
    isc = torch.empty((L, k), dtype=torch.float32, device="cuda")
    klv = torch.empty((L,), dtype=torch.float32, device="cuda")
    dsa.forward_prefill(qi, qs, ki, ks, w, q, kv, k, cfg.sm_scale, cfg.d_v, idx=idx, out=out, lse=lse, ws=ws)
    t_sa = time_calls(torch, lambda: dsa.indexer_scores_at(qi, qs, ki, ks, w, idx, out=isc), args.stage_reps)
    t_kl = time_calls(torch, lambda: dsa.indexer_kl(q, kv, idx, lse, isc, cfg.sm_scale, kl=klv), args.stage_reps)
    kept = kept_keys(L, k)
    sa_bytes = kept * (cfg.d_I + 4) + 2 * L * k * 4
    stages["indexer_kl"] = {
        "scores_at_ms": t_sa * 1e3, "scores_at_algorithmic_bytes": sa_bytes,
        "scores_at_algorithmic_GBps": sa_bytes / t_sa / 1e9,
        "scores_at_bound": "L2/MALL: the per-pair key bytes are algorithmic, the 16.5 MiB key cache stays on "
                           "chip, so this rate is not a fraction of HBM (HBM bytes: the counter table under "
                           "profiles/)",
        "kl_ms": t_kl * 1e3, "kl_gather_bytes": g_bytes, "kl_gather_frac_of_hbm_peak": g_bytes / t_kl / PEAK_HBM,
        "mean_kl": float(klv.mean()), "note": "sparse-stage indexer loss forward over the step's selection"}
    log(f"[bench] indexer KL: scores at selected keys {t_sa * 1e3:.3f} ms, KL {t_kl * 1e3:.3f} ms "
        f"({g_bytes / t_kl / 1e9:.0f} GB/s gathered), mean KL {float(klv.mean()):.4f}")
    del isc, klv

    # indexer KL loss of the dense warm-up stage over the sequence's first rows: dense index
    # scores (FP8 indexer) and two sweeps of dense attention over every key up to the row
    Ld = min(args.dense_kl, L)
    if Ld > 0:
        kld = torch.empty((Ld,), dtype=torch.float32, device="cuda")
        ws_kd = torch.empty(dsa.workspace_size(dsa.DSA_OP_KL_DENSE, 1, Ld, Ld, cfg.H, 1, 1, dsa.DSA_BF16),
                            dtype=torch.uint8, device="cuda")

        def kl_dense():
            dsa.indexer_kl_dense(qi[:Ld], qs[:Ld], ki[:Ld], ks[:Ld], w[:Ld], q[:Ld], kv[:Ld], cfg.sm_scale,
                                 kl=kld, ws=ws_kd)
        kl_dense()
        t_kd = time_calls(torch, kl_dense, args.stage_reps)
        keys = kept_keys(Ld, Ld)
        f_kd = 2 * 2 * cfg.H * cfg.d_qk * keys
        stages["indexer_kl_dense"] = {
            "ms": t_kd * 1e3, "rows": Ld, "keys": keys, "bf16_flop": f_kd, "mfma_frac": f_kd / t_kd / PEAK_BF16,
            "indexer_fp8_flop": indexer_flops(Ld, cfg.H_I, cfg.d_I),
            "gather_bytes": 2 * keys * cfg.d_qk * 2, "mean_kl": float(kld.mean()),
            "note": "dense warm-up indexer loss: dense FP8 index scores, then two sweeps of dense attention "
                    "(head lse, then the KL terms) over every key up to the row"}
        log(f"[bench] dense warm-up KL over {Ld} rows: {t_kd * 1e3:.3f} ms "
            f"({f_kd / t_kd / 1e12:.0f} TFLOP/s bf16), mean KL {float(kld.mean()):.4f}")
        del kld, ws_kd

    # backward of the sparse attention over the step's selection (the sparse training
    # stage): seeded bf16 output gradients of the workload's shape
    dout = torch.empty((L, cfg.H, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    gb = torch.Generator(device="cuda").manual_seed(1)
    for r0 in range(0, L, 8192):
        dout[r0:r0 + 8192] = torch.randn((min(8192, L - r0), cfg.H, cfg.d_v), generator=gb, device="cuda")
    ws_b = torch.empty(dsa.workspace_size(dsa.DSA_OP_MLA_BWD, 1, L, L, cfg.H, cfg.d_v, k, dsa.DSA_BF16),
                       dtype=torch.uint8, device="cuda")
    t_bwd = time_calls(torch, lambda: dsa.sparse_mla_backward(q, kv, idx, out, lse, dout, cfg.sm_scale, ws=ws_b),
                       args.stage_reps)
    f_bwd = kept * cfg.H * 2 * (3 * cfg.d_qk + 2 * cfg.d_v)
    stages["sparse_mla_backward"] = {
        "ms": t_bwd * 1e3, "bf16_flop": f_bwd, "mfma_frac": f_bwd / t_bwd / PEAK_BF16,
        "gather_bytes": g_bytes, "dkv_contribution_bytes": kept * cfg.d_qk * 4,
        "note": "dq and dkv of the step's attention for seeded output gradients; dkv from fp32 "
                "per-pair contribution rows (written once, read once) summed per key"}
    log(f"[bench] sparse MLA backward: {t_bwd * 1e3:.3f} ms ({f_bwd / t_bwd / 1e12:.0f} TFLOP/s bf16)")
    del dout, ws_b
    torch.cuda.empty_cache()

    decode = None
    if args.decode_workload != "none":
        del out, lse, q
        torch.cuda.empty_cache()
        dcfg = S.CONFIGS[args.decode_workload]
        ctx, dqi, dqs, dw, kc, kcs, dq, kvc = decode_inputs_on_gpu(dcfg, torch)
        ws_d = torch.empty(dsa.workspace_size(dsa.DSA_OP_DECODE, dcfg.batch, 1, dcfg.L, dcfg.H, dcfg.d_v, dcfg.k,
                                              dsa.DSA_BF16), dtype=torch.uint8, device="cuda")
        didx = torch.empty((dcfg.batch, dcfg.k), dtype=torch.int32, device="cuda")
        dout = torch.empty((dcfg.batch, dcfg.H, dcfg.d_v), dtype=torch.bfloat16, device="cuda")
        dlse = torch.empty((dcfg.batch, dcfg.H), dtype=torch.float32, device="cuda")

        def dstep():
            dsa.forward_decode(ctx, dqi, dqs, dw, kc, kcs, dq, kvc, dcfg.k, dcfg.sm_scale, dcfg.d_v, idx=didx,
                               out=dout, lse=dlse, ws=ws_d)
        for _ in range(args.warmup):
            dstep()
        t_dec, t_dec_med, t_dec_min = time_each(torch, dstep, max(args.steps, 10))
        icache = dcfg.batch * dcfg.L * (dcfg.d_I + 4)
        log(f"[bench] decode {t_dec * 1e6:.1f} us/step (median {t_dec_med * 1e6:.1f}, min {t_dec_min * 1e6:.1f})")
        decode = {"workload": dcfg.name, "us_per_step": t_dec * 1e6, "us_median": t_dec_med * 1e6,
                  "us_min": t_dec_min * 1e6, "steps": max(args.steps, 10), "batch": dcfg.batch, "ctx": dcfg.L,
                  "index_cache_bytes": icache, "index_cache_hbm_frac": icache / t_dec / PEAK_HBM}

        # the same step over paged caches: the caches' 64-token pages copied into pools in a
        # seeded random order, read through the block table
        P = dsa.DSA_PAGE_ROWS
        pps = (dcfg.L + P - 1) // P
        n_pages = dcfg.batch * pps
        perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(7)).view(dcfg.batch, pps)
        table = perm.to(torch.int32).cuda()
        s_idx = torch.arange(dcfg.L)
        rows = (perm[:, s_idx // P] * P + s_idx % P).reshape(-1).cuda()
        kp = torch.empty((n_pages * P, dcfg.d_I), dtype=kc.dtype, device="cuda")
        ksp = torch.empty((n_pages * P,), dtype=kcs.dtype, device="cuda")
        kvp = torch.empty((n_pages * P, dcfg.d_qk), dtype=kvc.dtype, device="cuda")
        kp[rows] = kc.reshape(-1, dcfg.d_I)
        ksp[rows] = kcs.reshape(-1)
        kvp[rows] = kvc.reshape(-1, dcfg.d_qk)
        del rows
        ref_out = dout.clone()
        pidx = torch.empty_like(didx)
        pout = torch.empty_like(dout)
        plse = torch.empty_like(dlse)

        def pstep():
            dsa.forward_decode_paged(ctx, dqi, dqs, dw, kp, ksp, dq, kvp, table, dcfg.L, dcfg.k, dcfg.sm_scale,
                                     dcfg.d_v, idx=pidx, out=pout, lse=plse, ws=ws_d)
        for _ in range(args.warmup):
            pstep()
        t_pg, t_pg_med, t_pg_min = time_each(torch, pstep, max(args.steps, 10))
        same = bool(torch.equal(pout.view(torch.int16), ref_out.view(torch.int16)))
        log(f"[bench] paged decode {t_pg * 1e6:.1f} us/step (median {t_pg_med * 1e6:.1f}); output equal to "
            f"the contiguous decode: {same}")
        decode["paged"] = {"us_per_step": t_pg * 1e6, "us_median": t_pg_med * 1e6, "us_min": t_pg_min * 1e6,
                           "page_rows": P, "output_equal_to_contiguous": same}
        del ctx, dqi, dqs, dw, kc, kcs, dq, kvc, ws_d, didx, dout, dlse, kp, ksp, kvp, table, pidx, pout, plse
        del ref_out
        torch.cuda.empty_cache()

    others = []
    if args.other_workloads != "none":
        for name in args.other_workloads.split(","):
            r = prefill_rate(S.CONFIGS[name], torch, dsa, args.warmup, args.steps)
            log(f"[bench] {name}: {r['tokens_per_s']:.0f} tokens/s ({r['ms_per_step']:.3f} ms/step)")
            others.append(r)
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg)
        log(f"[bench] cpu baseline {cpu['value']:.3f} tokens/s on {cpu['cores']} cores")

    value = L / (ms_step / 1e3)
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8+bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "seq_len": L, "batch": 1, "topk": k, "heads": cfg.H,
                   "d_qk": cfg.d_qk, "d_v": cfg.d_v, "indexer_heads": cfg.H_I, "indexer_dim": cfg.d_I,
                   "parallelism": "single GPU"},
        "ms_per_step_median": med_s * 1e3, "ms_per_step_min": min_s * 1e3,
        "roofline": roof, "stages": stages, "decode": decode, "other_prefill_workloads": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
