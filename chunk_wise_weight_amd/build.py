"""Build libttt.so (the HIP library behind the C ABI) for gfx950 with hipcc.

Usage: python -m chunk_wise_weight_amd.build [--verbose]
The library is written next to this file, in-tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libttt.so")
# a standalone program: MFMA throughput and shader clock under the power limit (not part of the library)
PROBE_SRC = os.path.join(PKG, "probes", "mfma_clock.hip")
PROBE = os.path.join(PKG, "probes", "mfma_clock")
SOURCES = ["ttt_api.hip", "kernels_bf16.hip", "kernels_f32.hip", "kernels_clip.hip", "kernels_target.hip", "kernels_misc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep fp32 arithmetic on scalar/vector FMA forms, not packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libttt.so")


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    cmd = [hipcc, *[f for f in HIPCC_FLAGS if f != "-fPIC"], "-o", PROBE + ".tmp", PROBE_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(PROBE + ".tmp", PROBE)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
