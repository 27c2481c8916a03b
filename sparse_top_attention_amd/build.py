"""Builds libqsa.so in-tree for gfx950 with hipcc (no JIT, no torch extension machinery)."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqsa.so")
SOURCES = ["qsa_decode.hip", "qsa_topk.hip", "qsa_prompt.hip", "qsa_chunk_d64_v8.hip", "qsa_chunk_d128_v8.hip",
           "qsa_chunk_d128_v4.hip", "qsa_chunk_d256_v8.hip", "qsa_chunk_d256_v4.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 VALU ops are switched off on purpose (-packed-fp32-ops): the kernels use scalar fp32 FMAs only.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# The decode chunk kernel's matrix-core accumulators are rescaled by the VALU between products: keeping them in
# ordinary VGPRs saves the copies to and from the accumulation registers.
EXTRA = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form"] for src in SOURCES if src.startswith("qsa_chunk_")}


def _compile(src):
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(int(os.environ.get("MAX_JOBS", "8")), len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
