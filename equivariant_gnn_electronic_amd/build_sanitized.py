"""Host-only build of libegnn with AddressSanitizer and UndefinedBehaviorSanitizer.

    python -m equivariant_gnn_electronic_amd.build_sanitized

Compiles every csrc/*.hip translation unit with ASan + UBSan on the host
side (every check fatal) and its device side unoptimised (those kernels are
never launched: the library is only for host logic), into
_build/sanitized/libegnn_san.so.  What runs there is the host logic: argument
checks, workspace carving, the CG and template tables.
tests/test_host_sanitizers.py runs the C ABI tests against it with the ASan
runtime preloaded.  It is never loaded on a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

from .build import CSRC, HIPCC, INCLUDE, ROOT, SOURCES

OUT = os.path.join(ROOT, "_build", "sanitized")
LIB = os.path.join(OUT, "libegnn_san.so")
# each sanitizer flag directly after -Xarch_host: host code only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-Xarch_device", "-O0", "-Xarch_host", "-g", "-std=c++17", "-fPIC",
         "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def asan_runtime():
    """The clang ASan runtime to preload into an uninstrumented interpreter."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def _compile(src):
    obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
    r = subprocess.run([HIPCC, *FLAGS, *SAN, "-c", os.path.join(CSRC, src), "-o", obj], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build():
    os.makedirs(OUT, exist_ok=True)
    with cf.ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libasan", "-o", LIB, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return LIB


def build_if_stale():
    """The sanitized library, rebuilt when any source or header is newer."""
    srcs = glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(INCLUDE, "*.h"))
    if os.path.exists(LIB) and os.path.getmtime(LIB) >= max(os.path.getmtime(f) for f in srcs):
        return LIB
    return build()


if __name__ == "__main__":
    print(build())
