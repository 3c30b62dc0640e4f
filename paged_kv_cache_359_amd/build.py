"""Builds libpkv.so in-tree with hipcc for gfx950 (host allocator + HIP kernels)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpkv.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

SOURCES = ["allocator.cpp", "cache_ops.hip", "decode.hip", "prefill.hip", "probe.hip"]

# Device code is built without packed-fp32 instructions (compiler-generated v_pk_* fp32 ops
# are avoided on this target); the host pass only warns that it does not know the feature.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]

# Per-source additions.  The attention kernels keep their matrix-core accumulators in
# ordinary VGPRs: with the default heuristic the compiler placed them in AGPRs and moved
# them back and forth every chunk around the softmax rescale, and the extra registers cost a
# wave per SIMD of occupancy.
_VGPR_MFMA = ["-mllvm", "--amdgpu-mfma-vgpr-form"]
SOURCE_FLAGS = {"prefill.hip": _VGPR_MFMA, "decode.hip": _VGPR_MFMA}


def build(verbose: bool = False, extra_flags=None) -> str:
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    tmp = LIB + ".tmp"

    def compile_one(src):
        path = os.path.join(CSRC, src)
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), *(extra_flags or []), "-I", INCLUDE,
               *lang, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, capture_output=not verbose)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
