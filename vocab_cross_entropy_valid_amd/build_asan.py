"""Host AddressSanitizer build of the library: liblce_asan.so.

The host code of the boundary (argument checks, workspace plans, launch
orchestration in api.hip) is compiled with AddressSanitizer; the device code
is the same as in liblce.so (no sanitizer on the GPU side).  Used on a host
without a GPU to run the host-side tests under the sanitizer:

    python -m vocab_cross_entropy_valid_amd.build_asan
    LD_PRELOAD=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so) \\
    ASAN_OPTIONS=detect_leaks=0 \\
    LCE_LIBRARY=vocab_cross_entropy_valid_amd/liblce_asan.so \\
    python -m pytest tests -m "not gpu"

(The Python interpreter is not instrumented, hence the preloaded runtime and
no leak check.)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

from . import build as _b

OBJ = os.path.join(_b.PKG, "_build_asan")
LIB = os.path.join(_b.PKG, "liblce_asan.so")
# host-only instrumentation: every sanitizer flag behind -Xarch_host
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def _compile(src: str) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    flags = _b._flags(src) + (HOST_ASAN if src == "api.hip" else [])
    cmd = [_b.hipcc(), *flags, "-c", os.path.join(_b.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return out


def build_asan(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(_b.SOURCES)) as ex:
        objs = list(ex.map(_compile, _b.SOURCES))
    cmd = [_b.hipcc(), f"--offload-arch={_b.ARCH}", "-shared", "-fPIC", "-Xarch_host",
           "-fsanitize=address", "-Xarch_host", "-shared-libasan", *objs, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_asan(verbose=True)
