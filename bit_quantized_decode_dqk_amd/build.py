"""Build libdqk.so for gfx950 in-tree with hipcc (no JIT cache, no pip install).

    python -m bit_quantized_decode_dqk_amd.build

Every call recompiles.  Sources whose results must be reproducible bit for bit
(append, select, dequant, host API) are compiled with -ffp-contract=off; the
decode kernels may contract.  All HIP code is compiled with packed-fp32 ops
disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdqk.so")
ARCH = os.environ.get("DQK_OFFLOAD_ARCH", "gfx950")

SOURCES = {
    "dqk_api.cpp": ["-ffp-contract=off"],
    "dqk_append.hip": ["-ffp-contract=off"],
    "dqk_select.hip": ["-ffp-contract=off"],
    "dqk_step.hip": ["-ffp-contract=off"],
    "dqk_dequant.hip": ["-ffp-contract=off"],
    "dqk_decode.hip": ["-fno-honor-nans"],   # inputs are finite; only -inf is used
    # the chunk loops (up to ten blocks, with a run-time exit) must unroll fully,
    # or the chunk's logits would be indexed at run time and go to scratch memory
    "dqk_decode4.hip": ["-fno-honor-nans", "-mllvm", "-unroll-max-upperbound=16"],
    "dqk_decode8.hip": ["-fno-honor-nans", "-mllvm", "-unroll-max-upperbound=16"],
    "dqk_bf16.hip": [],
    "dqk_combine.hip": [],
    "dqk_probe.hip": [],
    "dqk_noalloc.hip": [],
    "dqk_grow.hip": [],
}

COMMON = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-fast-math", "-fno-gpu-rdc"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, extra) -> str:
    obj = os.path.join(OUT_DIR, src + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if warn.strip() and os.environ.get("DQK_BUILD_VERBOSE"):
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
