"""Compile the gfx950 HIP library ``libmoe_mi355x.so`` in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libmoe_mi355x.so")

SOURCES = ["api.hip", "route.hip", "permute.hip", "grouped_gemm.hip",
           "ffn_f32.hip", "combine.hip", "mx_quant.hip", "mx_gemm.hip",
           "noalloc.hip", "eplb.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep per-thread staging arrays in registers, not in LDS
    "-mllvm", "-disable-promote-alloca-to-lds",
]


def build(verbose: bool = False) -> str:
    """Always recompiles; returns the path of the shared library."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = SO + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + ["-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
