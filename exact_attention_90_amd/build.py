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
           "fa_bwd.hip", "fa_bwd_d128.hip", "fa_bwd_d256.hip", "fa_bwd32.hip"]
ARCH = "gfx950"

# Packed fp32 VALU ops are kept out of every device code object.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-file code-generation choices: the 16-bit forward kernels and the d = 128 (and the
# d = 256 dV and dQ) backward kernels take the compiler's own matrix-core products (S, dP)
# in vector-register form;
# where the accumulators do not fit beside them
# (d = 256; the backward's dV and dK at d = 128) the accumulating products go to AGPRs
# through their own assembly.  (The d = 64 kernels compile to the same code either way.)
FILE_FLAGS = {"fa_fwd16_d128.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "fa_fwd16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "fa_bwd_d128.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "fa_bwd_d256.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _compile_cmd(src: str, obj: str, report: bool) -> list:
    cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS,
           *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if report:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    return cmd


def _compile_all(build_dir: str, report: bool, echo: bool) -> tuple:
    """Compile every source into build_dir, in parallel; returns (objects, compiler text)."""
    os.makedirs(build_dir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        procs.append((src, subprocess.Popen(_compile_cmd(src, obj, report), stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    texts = []
    for src, p in procs:
        out = p.communicate()[0]
        text = "\n".join(line for line in out.splitlines() if "packed-fp32-ops" not in line)
        if p.returncode != 0:
            sys.stderr.write(text + "\n")
            raise RuntimeError(f"hipcc failed on {src}")
        if echo:
            sys.stdout.write(text + "\n")
        texts.append(text)
    return objs, "\n".join(texts)


def build(report: bool = False, verbose: bool = False) -> str:
    objs, _ = _compile_all(os.path.join(PKG, "_build"), report, report or verbose)
    tmp = LIB + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


def resource_usage(build_dir: str) -> dict:
    """Compile every source into build_dir (the library itself is not touched) and return
    the compiler's per-kernel resource record: {kernel: {"vgpr", "agpr", "scratch",
    "vgpr_spill", "sgpr_spill", "occupancy"}} (scratch in bytes per lane)."""
    _, text = _compile_all(build_dir, report=True, echo=False)
    keys = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch",
            "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill",
            "Occupancy [waves/SIMD]": "occupancy"}
    out, cur = {}, None
    for line in text.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].split("[-Rpass")[0].strip()
        if body.startswith("Function Name:"):
            cur = body.split(":", 1)[1].strip()
            out[cur] = {}
            continue
        if cur is None or ":" not in body:
            continue
        k, v = body.rsplit(":", 1)
        if k.strip() in keys:
            try:
                out[cur][keys[k.strip()]] = int(v.strip())
            except ValueError:
                pass
    return out


def device_assembly(src: str, out_path: str) -> str:
    """The gfx950 assembly of one source as the library builds it (same flags), written to
    out_path; returns its text."""
    cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-I", INCLUDE,
           "-I", CSRC, *DEVICE_FLAGS, *FILE_FLAGS.get(src, []), "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", out_path]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        sys.stderr.write(p.stdout)
        raise RuntimeError(f"hipcc -S failed on {src}")
    with open(out_path) as f:
        return f.read()


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--report", action="store_true")
    args = ap.parse_args()
    print(build(report=args.report))
