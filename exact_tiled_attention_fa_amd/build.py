"""Build libfa.so (the C-ABI HIP library) in-tree with hipcc for gfx950.

Also builds libfa_sync.so, the race-check variant of the same sources
(-DFA_SYNC_CHECK=1: every LDS phase closed by a full wait and a barrier, with
unchanged arithmetic), which the GPU tests compare bit for bit with libfa.so.
Warnings are errors in both.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
SYNC_LIB = os.path.join(PKG, "libfa_sync.so")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_decode.hip", "fa_bwd.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wextra",
    "-Werror",
    # Packed FP32 VALU forms stay off: the compiler must not emit them.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature name; that note is harmless.
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


VARIANTS = (
    (LIB, os.path.join(PKG, "_build"), []),
    (SYNC_LIB, os.path.join(PKG, "_build", "sync"), ["-DFA_SYNC_CHECK=1"]),
)


def build(verbose: bool = False) -> str:
    """Compile every HIP source of both variants to objects in parallel, then
    link libfa.so and libfa_sync.so. Returns the path of libfa.so."""
    cc = hipcc()
    procs = []
    links = []
    for lib, objdir, defines in VARIANTS:
        os.makedirs(objdir, exist_ok=True)
        objs = []
        for src in SOURCES:
            obj = os.path.join(objdir, src.replace(".hip", ".o"))
            objs.append(obj)
            cmd = [cc, *HIPCC_FLAGS, *defines, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd))
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        links.append((lib, objs))
    failed = None
    for cmd, p in procs:
        _, err = p.communicate()
        err = "\n".join(l for l in err.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0 and failed is None:
            failed = f"build failed: {' '.join(cmd)}\n{err}"
        elif err.strip():
            sys.stderr.write(err + "\n")
    if failed:
        raise RuntimeError(failed)
    for lib, objs in links:
        tmp = lib + ".tmp"
        _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
