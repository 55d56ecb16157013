"""Build ``libtlgemm.so`` (gfx950 HIP kernels + host planner) in-tree with hipcc.

    python -m dense_gemm_transformer_amd.build [--force] [-j N]

Each source compiles to an object under ``_build/`` in parallel; the objects
link into ``dense_gemm_transformer_amd/libtlgemm.so``.  The benchmark's
hardware-ceiling probes link separately into ``libtlgceil.so``.  Works
without a GPU (hipcc cross-compiles for gfx950).
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtlgemm.so")
CEIL_LIB = os.path.join(PKG, "libtlgceil.so")
CEIL_SOURCES = ["ceilings.hip"]

ARCH = "gfx950"
SOURCES = [
    "plan.cpp",
    "run.hip",
    "kernels/generic.hip",
    "kernels/stream_f32.hip",
    "kernels/stream_f16.hip",
    "kernels/stream_bf16.hip",
    "kernels/tiled_f32.hip",
    "kernels/tiled_f16.hip",
    "kernels/tiled_bf16.hip",
    "layer.hip",
]
HEADERS = ["tlgemm_internal.h", "dispatch_table.inc", "kernels/common.h", "kernels/stream.h",
           "kernels/tiled.h"]

# Packed fp32 VALU ops are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _deps_mtime() -> float:
    paths = [os.path.join(CSRC, h) for h in HEADERS] + [os.path.join(INCLUDE, h) for h in ("tlgemm.h", "tlglayer.h")]
    paths.append(__file__)
    return max(os.path.getmtime(p) for p in paths)


def _compile(src: str, force: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
    if not force and os.path.exists(obj) and os.path.getmtime(obj) >= max(os.path.getmtime(path), _deps_mtime()):
        return obj
    cmd = [hipcc(), f"--offload-arch={ARCH}", *COMMON]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE_FLAGS]
    cmd += ["-c", path, "-o", obj + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(obj + ".tmp", obj)
    return obj


def _link(lib: str, objs: list[str]) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(force: bool = True, jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared libraries; returns the GEMM library's path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEIL_SOURCES
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, force), srcs))
    _link(LIB, objs[:len(SOURCES)])
    _link(CEIL_LIB, objs[len(SOURCES):])
    if verbose:
        print(f"built {LIB} and {CEIL_LIB}")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--force", action="store_true", help="recompile every source")
    ap.add_argument("-j", type=int, default=None)
    args = ap.parse_args(argv)
    build(force=args.force, jobs=args.j, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
