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
           "qsa_chunk_d128_v4.hip", "qsa_chunk_d192_v8.hip", "qsa_chunk_d192_v4.hip", "qsa_chunk_d256_v8.hip",
           "qsa_chunk_d256_v4.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 VALU ops are switched off on purpose (-packed-fp32-ops): the kernels use scalar fp32 FMAs only.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# The decode chunk kernel's matrix-core accumulators are rescaled by the VALU between products: keeping them in
# ordinary VGPRs saves the copies to and from the accumulation registers.
EXTRA = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form"] for src in SOURCES if src.startswith("qsa_chunk_")}


# A test build of the same sources with AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (each
# sanitizer flag applies to the host pass alone; the device code is built as usual): the argument checks, scratch
# layouts and launch dispatch run under the sanitizers in the CPU tests. Never loaded by the product path.
SAN_BUILD = os.path.join(HERE, "_build_san")
SAN_LIB = os.path.join(HERE, "libqsa_san.so")
SAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src, sanitize=False):
    out_dir = SAN_BUILD if sanitize else BUILD
    obj = os.path.join(out_dir, src.replace(".hip", ".o"))
    flags = [f for f in FLAGS if f != "-O3"] + SAN_FLAGS if sanitize else FLAGS
    cmd = [HIPCC, *flags, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose=False, sanitize=False):
    out_dir, lib = (SAN_BUILD, SAN_LIB) if sanitize else (BUILD, LIB)
    os.makedirs(out_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(int(os.environ.get("MAX_JOBS", "8")), len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    tmp = lib + ".tmp"
    link = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"] if sanitize else []
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    import sys
    build(verbose=True, sanitize="--sanitize" in sys.argv)
