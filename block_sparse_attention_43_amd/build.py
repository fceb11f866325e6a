"""Compile the HIP sources into ``libpisa.so`` for gfx950, in-tree.

    python -m block_sparse_attention_43_amd.build

Objects go to ``_build/`` at the repository root; the shared library is written next
to this file, where the Python binding loads it.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpisa.so")
SOURCES = ["abi.hip", "block_stats.hip", "select_topk.hip", "select_large.hip", "pooled_w.hip", "attention_fwd.hip", "attention_frag.hip", "attention_row.hip",
           "attention_literal.hip", "attention_bwd.hip", "attention_bwd_literal.hip", "layout.hip"]
ARCH = "gfx950"
# Packed fp32 VALU forms are disabled for all device code (hipcc emits them from plain
# float code otherwise); the host pass warns that it does not know the feature.
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


# Per-source extra flags. The register-streamed attention kernel keeps its MFMA results
# in VGPRs (the VALU reads every score tile); operands still come from AGPRs.
EXTRA = {"attention_frag.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
         "attention_row.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"],
         "attention_literal.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"]}


def build(verbose: bool = False, jobs: int = 4) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[hipcc, *FLAGS, *EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
