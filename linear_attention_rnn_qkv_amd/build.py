"""Build the C-ABI library ``libgdn.so`` in-tree with hipcc for gfx950.

Usage: ``python -m linear_attention_rnn_qkv_amd.build``. Compiles every source
under ``csrc/`` (in parallel) and links one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
OBJ = os.path.join(HERE, "_build")
ARCH = "gfx950"
SOURCES = ["gdn_api.cpp", "prologue.hip", "chunk_rule.hip", "chunk_prep.hip",
           "chunk_state.hip", "gated_norm.hip", "decode.hip",
           "chunk_state_wide.hip", "backward.hip", "chunk_bwd.hip", "chunk_bwd_mma.hip", "chunk_bwd_state_mma.hip",
           "noalloc.hip"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         # no packed-FP32 instructions in generated device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA sources and results in VGPRs (gfx950 has no separate
         # accumulator file requirement): avoids AGPR<->VGPR copies around
         # every VALU use of an accumulator
         "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
