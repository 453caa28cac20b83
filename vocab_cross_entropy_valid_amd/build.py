"""Ahead-of-time build of liblce.so for gfx950 with hipcc.

Compiles every source in csrc/ to an object (in parallel) and links the
shared library next to this file, where the Python binding loads it.  Runs
without a GPU: hipcc cross-compiles for gfx950.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblce.so")
ARCH = os.environ.get("LCE_OFFLOAD_ARCH", "gfx950")

SOURCES = ["kernels_fwd.hip", "kernels_bwd.hip", "kernels_embed.hip", "kernels_attn.hip",
           "api.hip"]

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep the compiler from emitting packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # schedule for instruction-level parallelism (one wave per SIMD: the
    # MFMA loop cannot hide LDS latency behind other waves)
    "-mllvm", "-amdgpu-sched-strategy=max-ilp",
    f"-I{os.path.join(ROOT, 'include')}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblce)")


# The attention kernels (their operand reads are ordered by explicit
# sched_group_barriers where it matters) keep LLVM's default scheduler: with
# max-ilp both backward passes measured 8% slower, the forward 2% faster.
DEFAULT_SCHED = {"kernels_attn.hip"}


def _flags(src: str) -> list:
    if src not in DEFAULT_SCHED:
        return FLAGS
    i = FLAGS.index("-amdgpu-sched-strategy=max-ilp")
    return FLAGS[:i - 1] + FLAGS[i + 1:]


def _compile(src: str) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *_flags(src), "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx950-only feature above: drop that note
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return out


def build(verbose: bool = False) -> str:
    """Compile csrc/*.hip and link liblce.so; returns the library path."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
