"""Compile libqmm.so (HIP, gfx950) in-tree with hipcc.

Every source is compiled with
  * -ffp-contract=off: no silent a*b+c fusion, so each fp32 step of the
    quantizers is the single IEEE operation the method states;
  * -fhip-fp32-correctly-rounded-divide-sqrt: '/' and sqrtf are correctly
    rounded (the quantizers rely on it for bit-exact codes);
  * the packed-fp32 target feature switched off (-packed-fp32-ops);
and no fast-math.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqmm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["abi.hip", "quantize.hip", "w4a16.hip", "w8a8.hip", "w8a16.hip", "formats.hip", "awq.hip"]

# Per-source extra flags.  The MFMA kernels keep their accumulators in
# ordinary VGPRs: with the default accumulator-register form the register
# allocator copies accumulators between registers on every loop iteration,
# and results folded on the vector ALUs would be copied out of AGPRs.
EXTRA = {"w8a8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "w4a16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "w8a16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
         "formats.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link libqmm.so; returns the library path."""
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
