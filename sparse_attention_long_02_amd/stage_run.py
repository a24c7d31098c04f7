"""Runs each prefill stage once, at a benchmark workload, for hardware-counter profiling.

    python -m sparse_attention_long_02_amd.stage_run [--workload prefill_128k] [--copy-mib 4096]
                                                     [--training] [--dense-kl L] [--decode]

Order of the dispatches: one device-to-device copy of --copy-mib MiB (its FETCH_SIZE and
WRITE_SIZE readings calibrate the counters against a known byte count), then
dsa_select_prefill (per chunk of rows: key-sample indexer, thresholds, filtering indexer,
candidate top-k; then the streaming selection of any undecided rows), then dsa_sparse_mla on
that selection.  With --training, then the sparse-stage indexer loss (dsa_indexer_scores_at,
dsa_indexer_kl) and dsa_sparse_mla_backward for seeded output gradients, as the benchmark
runs them.  With --dense-kl L, the dense warm-up loss (dsa_indexer_kl_dense) over the first L
rows and keys of the same sequence.  With --decode, one dsa_forward_decode of the 64 x 131072
decode workload.  Inputs are the seeded synthetic tensors the benchmark uses.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="prefill_128k")
    ap.add_argument("--copy-mib", type=int, default=4096)
    ap.add_argument("--training", action="store_true")
    ap.add_argument("--dense-kl", type=int, default=0)
    ap.add_argument("--decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    args = ap.parse_args()

    import torch
    import bench
    from sparse_attention_long_02_amd import dsa
    from sparse_attention_long_02_amd import synth as S

    cfg = S.CONFIGS[args.workload]
    dsa.lib()
    n = args.copy_mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[stage_run] copy of {n} bytes done", flush=True)
    del src, dst

    if not args.no_prefill:
        prefill(args, cfg, torch, bench, dsa)
    if args.decode:
        decode(torch, bench, dsa, S)


def decode(torch, bench, dsa, S):
    dcfg = S.CONFIGS["decode_64x128k"]
    ctx, qi, qs, w, kc, kcs, q, kvc = bench.decode_inputs_on_gpu(dcfg, torch)
    dsa.forward_decode(ctx, qi, qs, w, kc, kcs, q, kvc, dcfg.k, dcfg.sm_scale, dcfg.d_v)
    torch.cuda.synchronize()
    print("[stage_run] forward_decode done", flush=True)


def prefill(args, cfg, torch, bench, dsa):
    qi, qs, ki, ks, w, q, kv = bench.prefill_inputs_on_gpu(cfg, torch)
    if args.dense_kl:
        n = min(args.dense_kl, cfg.L)
        dsa.indexer_kl_dense(qi[:n], qs[:n], ki[:n], ks[:n], w[:n], q[:n], kv[:n], cfg.sm_scale)
        torch.cuda.synchronize()
        print(f"[stage_run] indexer_kl_dense over {n} rows done", flush=True)
    idx = torch.empty((cfg.L, cfg.k), dtype=torch.int32, device="cuda")
    dsa.select_prefill(qi, qs, ki, ks, w, cfg.k, idx=idx)
    torch.cuda.synchronize()
    print("[stage_run] select_prefill done", flush=True)
    out, lse = dsa.sparse_mla(q, kv, idx, cfg.sm_scale, cfg.d_v)
    torch.cuda.synchronize()
    print("[stage_run] sparse_mla done", flush=True)
    if not args.training:
        return
    isc = dsa.indexer_scores_at(qi, qs, ki, ks, w, idx)
    dsa.indexer_kl(q, kv, idx, lse, isc, cfg.sm_scale)
    torch.cuda.synchronize()
    print("[stage_run] indexer KL done", flush=True)
    del isc
    dout = torch.empty((cfg.L, cfg.H, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    gb = torch.Generator(device="cuda").manual_seed(1)
    for r0 in range(0, cfg.L, 8192):
        dout[r0:r0 + 8192] = torch.randn((min(8192, cfg.L - r0), cfg.H, cfg.d_v), generator=gb, device="cuda")
    dsa.sparse_mla_backward(q, kv, idx, out, lse, dout, cfg.sm_scale)
    torch.cuda.synchronize()
    print("[stage_run] sparse_mla_backward done", flush=True)


if __name__ == "__main__":
    main()
