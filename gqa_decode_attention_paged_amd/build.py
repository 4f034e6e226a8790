"""Compile the HIP library ``libgqa_paged.so`` for gfx950, in-tree.

    python -m gqa_decode_attention_paged_amd.build
"""
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgqa_paged.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed-FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # gfx950 preloads this many leading kernel-argument dwords into SGPRs (the
    # decode kernel's block-table pointer, lengths pointer and plan scalars)
    "-mllvm", "-amdgpu-kernarg-preload-count=8",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
DECODE_SOURCE = os.path.join(CSRC, "gqa_paged.hip")     # decode, append, copy and gather kernels
SOURCES = [DECODE_SOURCE, os.path.join(CSRC, "probes.hip")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libgqa_paged.so")


def build(verbose: bool = False) -> str:
    """Compile every source into the shared library; returns its path."""
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=PKG, prefix=".libgqa_paged.")
    os.close(fd)
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-6000:]}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
