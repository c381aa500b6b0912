"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m fine_grained_mixture_amd.build
The library is written in-tree next to this file so that it travels with the
source tree; the object files go to _build/ at the repository root.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "gemm.hip", "gemm_big.hip", "skinny.hip", "route.hip", "route_small.hip",
           "combine.hip", "lowrank.hip", "gemm_bwd.hip", "gemm_bwd_f32.hip", "backward.hip", "lowrank_bwd.hip",
           "fp8.hip", "noalloc.hip"]

# -packed-fp32-ops: no packed fp32 VALU instructions in the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


INFO = os.path.join(PKG, "build_info.json")


def source_digest() -> str:
    """sha256 over the library's sources (csrc and include), file names included."""
    import hashlib
    h = hashlib.sha256()
    for dname in (CSRC, os.path.join(ROOT, "include")):
        for name in sorted(os.listdir(dname)):
            if name.endswith((".hip", ".cpp", ".h")):
                h.update(name.encode())
                with open(os.path.join(dname, name), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()


def _write_info() -> None:
    """Record the commit the library was built from, so that a copy of the
    tree without its git history can still name it."""
    import json
    import time
    try:
        sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                             text=True, timeout=10).stdout.strip() or None
        dirty = bool(subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--",
                                     "fine_grained_mixture_amd/csrc", "include"],
                                    capture_output=True, text=True, timeout=10).stdout.strip())
    except (OSError, subprocess.SubprocessError):
        sha, dirty = None, None
    info = {"git_sha": sha, "sources_modified_since_commit": dirty,
            "source_sha256": source_digest(),
            "built_utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime())}
    with open(INFO, "w") as f:
        json.dump(info, f)


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library. Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    _write_info()
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
