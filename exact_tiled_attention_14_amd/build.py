"""Compile the HIP sources in ``csrc/`` into the in-tree ``libfa.so`` (gfx950).

Run as ``python -m exact_tiled_attention_14_amd.build``.  Each source is
compiled to an object under ``_build/`` in parallel, then linked.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libfa.so")

SOURCES = ["fa_api.hip", "fwd_bf16.hip", "fwd_f32.hip", "decode.hip", "bwd_bf16.hip", "quant_fp8.hip", "fwd_fp8.hip", "decode_mq.hip", "mla.hip"]

ARCH = "gfx950"
# Packed fp32 instructions are disabled for all device code: the compiler may
# otherwise form v_pk_* fp32 operations from ordinary float code.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Extra options for single sources.  The backward's dK/dV kernel runs one wave
# per SIMD with its gradient accumulators in AGPRs; by default the compiler
# also puts the S and dP products there and copies them back for the
# softmax arithmetic (64 register moves per step), which the VGPR form of the
# matrix-core results avoids (same-box A/B: 209.9 -> 203.7 us for the whole
# backward at B2 H16 S2048).
SOURCE_FLAGS = {"bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libfa.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
