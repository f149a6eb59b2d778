"""Build libfa.so (gfx950 HIP kernels + C boundary) in-tree with hipcc.

    python -m exact_attention_90_amd.build            # build
    python -m exact_attention_90_amd.build --report   # build and print per-kernel
                                                      # VGPR/AGPR/spill/LDS/occupancy
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_fused.hip", "fa_fwd16.hip", "fa_fwd16_d128.hip", "fa_naive.hip",
           "fa_bwd.hip", "fa_bwd32.hip"]
ARCH = "gfx950"

# Packed fp32 VALU ops are kept out of every device code object.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-file code-generation choices: the d = 128 forward kernel takes its S products in
# vector-register form (its P V products accumulate in AGPRs through assembly).
FILE_FLAGS = {"fa_fwd16_d128.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(report: bool = False, verbose: bool = False) -> str:
    objs = []
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
               "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS,
               *FILE_FLAGS.get(src, []), "-c",
               os.path.join(CSRC, src), "-o", obj]
        if report:
            cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
        res = subprocess.run(cmd, capture_output=True, text=True)
        text = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                         if "packed-fp32-ops" not in line)
        if res.returncode != 0:
            sys.stderr.write(text + "\n")
            raise RuntimeError(f"hipcc failed on {src}")
        if report or verbose:
            sys.stdout.write(text + "\n")
        objs.append(obj)
    tmp = LIB + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--report", action="store_true")
    args = ap.parse_args()
    print(build(report=args.report))
