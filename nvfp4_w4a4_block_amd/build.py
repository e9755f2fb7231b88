"""Builds libnvfp4.so (the HIP kernels and the C ABI of include/nvfp4.h) in-tree for gfx950.

    python -m nvfp4_w4a4_block_amd.build

Each source is compiled with hipcc to an object under _build/, then linked
into nvfp4_w4a4_block_amd/libnvfp4.so.  The quantization kernels are built
with -ffp-contract=off and correctly rounded fp32 division, which their
bit-exact codes and scales rely on.  Every HIP object is built with packed
fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnvfp4.so")
ARCH = "gfx950"

SOURCES = {
    "quant.hip": ["-ffp-contract=off"],
    "gemm_skinny.hip": [],
    "gemv_fp4.hip": [],
    "gemm_m16.hip": [],
    "gemm_m16_stream.hip": [],
    "tree.hip": [],
    "kv_fp8.hip": [],
    "gemm_tiled.hip": [],
    "stream.hip": [],
    "scratch.hip": [],
    "abi.cpp": [],
}

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Werror",
    "-Wno-unused-command-line-argument",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the NVFP4 library)")


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that line.
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = []
    objs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        jobs.append([cc, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for cmd, fut in [(c, ex.submit(_run, c)) for c in jobs]:
            if verbose:
                print(" ".join(cmd))
            fut.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
