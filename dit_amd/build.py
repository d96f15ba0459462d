"""Builds libfixedm.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m dit_amd.build          # or __graft_entry__.build()

Every HIP file is compiled with packed-fp32 instruction selection disabled and without
floating-point contraction, so the arithmetic is exactly what the source spells out.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfixedm.so")
SOURCES = ["api.cpp", "bounds.hip", "attn_bf16.hip", "attn_f32.hip", "finalize.hip"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


# Per-file flags.  The bf16 attention kernel keeps its MFMA accumulators in architectural
# VGPRs (so the exp2 work reads the scores without v_accvgpr_read copies) and pins the
# resident query fragments in the accumulation registers instead.
EXTRA = {"attn_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def _generate() -> None:
    """Writes the generated kernel sources (the assembly main loop of the bf16 kernel)."""
    sys.path.insert(0, CSRC)
    try:
        import gen_fixed_loop
    finally:
        sys.path.remove(CSRC)
    gen_fixed_loop.main()


def build(verbose: bool = False) -> str:
    """Generates and compiles every source and links dit_amd/libfixedm.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    _generate()
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
