"""Build libegnn.so (HIP, gfx950) in-tree.

    python -m equivariant_gnn_electronic_amd.build

Compiles every csrc/*.hip translation unit with hipcc in parallel and links
them into equivariant_gnn_electronic_amd/libegnn.so.  Object files go to
_build/ at the repository root.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libegnn.so")

SOURCES = ["common.hip", "timing.hip", "graph.hip", "geom.hip", "gemm.hip", "layer.hip", "hblocks.hip", "labels.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 (v_pk_*_f32) instructions in the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(verbose=True, only=None):
    """Compile and link; returns the library path.  Always recompiles every
    source, or only the listed ones (their objects from an earlier build are
    reused for the rest)."""
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        raise RuntimeError("hipcc not found")
    os.makedirs(BUILD, exist_ok=True)
    todo = SOURCES if not only else [s for s in SOURCES if s in only]
    if only and len(todo) != len(set(only)):
        raise ValueError(f"unknown sources: {sorted(set(only) - set(SOURCES))}")
    jobs = min(len(todo), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, todo))
    for (obj, err), src in zip(results, todo):
        if err.strip() and verbose:
            print(f"[{src}]\n{err}", file=sys.stderr)
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"objects missing (run a full build): {missing}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--only", nargs="*", help="recompile only these csrc/*.hip files, then link")
    build(only=ap.parse_args().only)
