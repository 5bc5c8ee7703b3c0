"""Build libmxsens.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m bit_gemm_hdiag_amd.build [--debug]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libmxsens.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["mxs_colsum.hip", "mxs_allocate.hip", "mxs_quantize.hip", "mxs_gemm.hip", "mxs_layerwise.hip", "mxs_attention.hip", "mxs_api.hip"]
# packed fp32 instructions are disabled for all device code; common-code
# sinking is off because merging the tails of per-width branches turned
# register arrays of the decode kernels into scratch memory
FLAGS = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-simplifycfg-sink-common=false",
         "-I", os.path.join(HERE, "..", "include")]


def _compile(src: str, debug: bool) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if debug:
        cmd.append("-g")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(debug: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, debug), SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(debug="--debug" in sys.argv))
