"""Build libgqa_attn.so (and the measurement microbenchmarks,
libgqa_microbench.so) in-tree with hipcc for gfx950.

    python -m mqa_flashattention_amd.build          # compile
    python -m mqa_flashattention_amd.build --asm    # also keep the gfx950 assembly

Flags: -O3, C++17, position-independent shared library, gfx950 only, and
packed-fp32 VALU instructions disabled for the device pass.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = [os.path.join(CSRC, "gqa_attn.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("attn_tile.hpp", "prefill_kernel.hpp",
                                           "decode_kernel.hpp", "decode_part.hpp",
                                           "mixed_kernel.hpp", "backward_kernel.hpp")] + [
    os.path.join(INCLUDE, "gqa_attn.h")]
LIBRARY = os.path.join(PKG, "libgqa_attn.so")
MICROBENCH_SOURCE = os.path.join(CSRC, "microbench.hip")
MICROBENCH = os.path.join(PKG, "libgqa_microbench.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # device code never produces or tests NaN (scores are finite or
            # -inf), so max needs no NaN canonicalisation; host code keeps
            # IEEE semantics for argument validation
            "-Xarch_device", "-fno-honor-nans",
            "-Wall", "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(sources, output, verbose, keep_asm=False):
    tmp = output + ".tmp"
    cmd = [hipcc(), *compile_flags(), *sources, "-o", tmp]
    if keep_asm:
        cmd += ["-save-temps=obj"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=CSRC)
    os.replace(tmp, output)


def build(verbose: bool = False, keep_asm: bool = False) -> str:
    """Compile the HIP library and the microbenchmark library; returns the
    library's path.  Always recompiles."""
    _compile(SOURCES, LIBRARY, verbose, keep_asm)
    _compile([MICROBENCH_SOURCE], MICROBENCH, verbose)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True, keep_asm="--asm" in sys.argv))
