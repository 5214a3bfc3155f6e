"""Build libswiglu.so in-tree with hipcc for gfx950.

Usage: python -m swiglu_mlp_fwd_amd.build [-v]

Every HIP source under csrc/ is compiled to an object in _build/ (in
parallel) and linked into swiglu_mlp_fwd_amd/libswiglu.so.  All device code
is compiled with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libswiglu.so")
ARCH = "gfx950"

SOURCES = ["abi.hip", "gemm.hip", "transpose.hip", "gemv.hip", "act_fwd.hip", "act_quant.hip", "act_bwd.hip",
           "count.hip", "probe.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Packed fp32 ops (v_pk_*_f32) are left out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def source_hash() -> str:
    """Hash of everything the library is built from: every file under csrc/,
    the public header and the compiler flags.  It is compiled into the
    library (swiglu_source_hash) and compared on load, so a library built
    from other sources is refused instead of silently tested."""
    h = hashlib.sha256()
    files = sorted(os.path.join("csrc", f) for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp", ".h")))
    for rel in files + [os.path.join("..", "include", "swiglu.h")]:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read() + b"\0")
    h.update(" ".join(HIPCC_FLAGS).encode())
    return h.hexdigest()[:16]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; libswiglu needs ROCm to build")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, f'-DSWIGLU_SOURCE_HASH="{source_hash()}"', "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile and link libswiglu.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
