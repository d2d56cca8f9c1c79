"""Build libvdit.so (the HIP kernels and their C ABI) in-tree for gfx950.

Usage: ``python -m spacetime_attention_amd.build`` or ``build()`` from Python.
Each .hip file is compiled on its own (in parallel) and the objects are linked
into ``spacetime_attention_amd/libvdit.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libvdit.so")
OBJDIR = os.path.join(HERE, "_build")

SOURCES = ["attn_flash.hip", "attn_flash_full.hip", "attn_temporal.hip", "attn_f32.hip", "patchify.hip",
           "rope3d.hip", "qkv_proj.hip", "vdit_abi.hip"]
# Per-file flags. The full pass's ping-pong kernel is scheduled with LLVM's
# maximum-ILP strategy (measured faster there, slower on the other passes).
FILE_FLAGS = {"attn_flash_full.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # Packed fp32 VALU ops are kept out of all device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + FILE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libvdit.so. Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    workers = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
