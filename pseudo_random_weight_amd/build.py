"""Build the HIP library libseedmm.so in-tree for gfx950.

    python -m pseudo_random_weight_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libseedmm.so")
SOURCES = [os.path.join(CSRC, "seedmm.hip"), os.path.join(CSRC, "search.hip"),
           os.path.join(CSRC, "expert_cache.hip")]
HEADERS = [os.path.join(CSRC, "seed_decode.hpp"), os.path.join(CSRC, "moe_layer.hpp"),
           os.path.join(ROOT, "include", "seedmm.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # no packed fp32 instructions in any device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
    # keep per-thread arrays in registers (the LDS budget belongs to the kernels' tiles)
    "-mllvm", "-disable-promote-alloca-to-lds",
]


def build(verbose: bool = False) -> str:
    tmp = SO + ".tmp"
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libseedmm.so")
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
