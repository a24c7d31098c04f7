"""Build libdsa.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m sparse_attention_long_02_amd.build [--verbose]

The library is written next to this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
SOURCES = ["api.cpp", "indexer.hip", "topk.hip", "prefill_topk.hip", "sparse_mla.hip", "quant.hip",
           "attn_kl.hip", "sparse_mla_bwd.hip", "indexer_dense.hip", "noalloc.hip"]
# sources whose kernels keep MFMA accumulators in the accumulation registers (the backward's
# dq accumulators do not fit next to its operands in the vector registers)
AGPR_ACC = {"sparse_mla_bwd.hip"}
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms stay off in every device build
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in the VGPR form: the attention kernel rescales them with
    # VALU ops, and AGPR<->VGPR copies otherwise push it into scratch
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdsa)")


def build(verbose: bool = False, extra: list | None = None) -> str:
    """Compile every source into libdsa.so; returns the library path."""
    os.makedirs(os.path.join(HERE, "_build"), exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(HERE, "_build", os.path.splitext(src)[0] + ".o")
        flags = HIPCC_FLAGS
        if src in AGPR_ACC:
            flags = [f for f in HIPCC_FLAGS if f not in ("-mllvm", "-amdgpu-mfma-vgpr-form")]
        cmd = [hipcc(), *flags, *(extra or []), "-I", os.path.join(ROOT, "include"), "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, flush=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
