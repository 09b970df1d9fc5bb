"""Build the host side of libr2l.so with AddressSanitizer and UBSan (CPU only).

    python -m reverse_selective_scan_amd.build_sanitized   # -> _build_san/libr2l_san.so

Every csrc/*.hip is compiled as for libr2l.so, plus both sanitizers on the
host compiler only: the C-ABI entry points, their argument checks, the
workspace planning and the launch code are instrumented; the device code is
the usual gfx950 code, uninstrumented.  Loading the library
into an uninstrumented Python needs the ASan runtime preloaded:
asan_runtime() returns its path (tests/test_host_sanitized.py does this).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

from reverse_selective_scan_amd.build import CFLAGS as BASE_CFLAGS, CSRC, HIPCC, ARCH

PKG = os.path.dirname(os.path.abspath(__file__))
BUILD = os.path.join(PKG, "_build_san")
LIB = os.path.join(BUILD, "libr2l_san.so")

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
CFLAGS = [*BASE_CFLAGS, "-Xarch_host", "-g", *SAN]


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to LD_PRELOAD)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    r = subprocess.run([HIPCC, *CFLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan", *SAN, *objs, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
