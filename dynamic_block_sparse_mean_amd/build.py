"""Build libsparse_attn.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m dynamic_block_sparse_mean_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsparse_attn.so")
SOURCES = ["api.hip", "pool.hip", "select.hip", "quant.hip", "attn.hip", "ulysses.hip", "nvfp4.hip"]
ARCH = "gfx950"

# Packed fp32 VALU ops are kept out of the generated code on purpose (the hipcc host pass
# warns that it does not know the feature; that warning is harmless).
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# MFMA accumulators in ordinary VGPRs for the attention and score kernels (small accumulators,
# no copies between register files); the GEMM keeps its 256 accumulator registers in AGPRs.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
PER_FILE = {s: VGPR_FORM for s in SOURCES if s != "nvfp4.hip"}


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + err)
    return err


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[hipcc, *FLAGS, *PER_FILE.get(s, []), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        for msg in ex.map(_run, cmds):
            if verbose and msg.strip():
                print(msg)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
