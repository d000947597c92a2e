"""Compile libfa.so (the HIP kernels and the C ABI) for gfx950, in tree.

    python -m exact_io_aware_69_amd.build

Each .hip file is compiled to an object in parallel, then linked into
``exact_io_aware_69_amd/libfa.so``. Every HIP translation unit gets
``-Xclang -target-feature -Xclang -packed-fp32-ops`` so that hipcc never
emits packed fp32 arithmetic.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

try:
    from . import _srcid
except ImportError:  # run as a script
    import _srcid

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip", "fa_std.hip", "fa_fwd_fa1.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str, build_id: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    # Only the C ABI's unit carries the source identity (fa_build_id), so the
    # kernels' objects do not depend on it.
    extra = [f'-DFA_BUILD_ID="{build_id}"'] if src == "fa_api.hip" else []
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature and says so.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l).strip()
    if msg:
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        raise RuntimeError("hipcc not found")
    os.makedirs(BUILD, exist_ok=True)
    build_id = _srcid.source_id()
    workers = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_id), SOURCES))
    tmp = LIB + ".tmp"
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "lib")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
           f"-L{rocm_lib}", f"-Wl,-rpath,{rocm_lib}", "-lrocblas"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} (sources {build_id})")
    return LIB


if __name__ == "__main__":
    build()
