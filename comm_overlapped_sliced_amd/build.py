"""Builds libflashovl.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libflashovl.so")
SOURCES = ["fo_api.cpp", "fo_dma.cpp", "fo_sched.cpp", "fo_gemm.hip", "fo_mlp.hip", "fo_attn.hip"]
ARCH = "gfx950"


def hipcc_cmd(out: str) -> list:
    return [
        "hipcc", "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        # packed fp32 VALU forms are kept out of the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, "-Wl,-rpath,/opt/rocm/lib",
        *[os.path.join(CSRC, s) for s in SOURCES], "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    res = subprocess.run(hipcc_cmd(tmp), capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
