"""Build librocketkv.so (hand-written HIP for gfx950) in-tree.

    python -m sparse_decode_attention_amd.build      # or build() from Python
    python -m sparse_decode_attention_amd.build --incremental   # changed sources only

Every .hip file under csrc/ is compiled to an object with hipcc (in parallel)
and linked into sparse_decode_attention_amd/librocketkv.so.  Packed-FP32
instructions are disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
LIB = os.path.join(PKG, "librocketkv.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; cannot build librocketkv.so")
    return exe


def _stale(src: str, obj: str) -> bool:
    """True when obj is missing or older than src or any header it may include."""
    if not os.path.exists(obj):
        return True
    deps = [src, *glob.glob(os.path.join(CSRC, "*.hpp")), *glob.glob(os.path.join(INCLUDE, "*.h")), __file__]
    return os.path.getmtime(obj) < max(os.path.getmtime(x) for x in deps)


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    if incremental and not _stale(src, obj):
        return obj
    cmd = [_hipcc(), *FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = True, incremental: bool = False) -> str:
    """Compile every csrc/*.hip and link librocketkv.so; returns its path.
    incremental: recompile only sources newer than their objects (or whose
    headers changed); the default compiles everything."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda x: _compile(x, incremental), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", flush=True)
    return LIB


if __name__ == "__main__":
    try:
        build(incremental="--incremental" in sys.argv[1:])
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
