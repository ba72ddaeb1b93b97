"""Compile the HIP library for gfx950, in-tree.

Produces mamba_ssd_chunked_04_amd/libssd_mi355x.so from the HIP sources in
csrc/ (the SSD forward and backward, the gated RMSNorm and the causal
conv1d) with hipcc.  Packed-fp32 instruction selection is switched off for all device
code (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
SRCS = tuple(os.path.join(PKG_DIR, "csrc", f)
             for f in ("ssd_fwd.hip", "ssd_bwd.hip", "rmsnorm_gated.hip", "causal_conv1d.hip"))
HEADER = os.path.join(REPO_DIR, "include", "ssd_mi355x.h")
LIB = os.path.join(PKG_DIR, "libssd_mi355x.so")
ARCH = "gfx950"


def hipcc_command(out_path: str = LIB, extra=()) -> list:
    hipcc = os.environ.get("HIPCC", "hipcc")
    return [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-pass-failed", "-I", os.path.join(REPO_DIR, "include"), *SRCS, "-o", out_path, *extra]


def build_library(verbose: bool = True) -> str:
    """Always recompiles; writes the library atomically."""
    tmp = LIB + ".tmp%d" % os.getpid()
    t0 = time.time()
    proc = subprocess.run(hipcc_command(tmp), capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
    if proc.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"[build] {os.path.relpath(LIB, REPO_DIR)} in {time.time() - t0:.1f}s", file=sys.stderr)
        if err.strip():
            print(err, file=sys.stderr)
    return LIB


def library_is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in (*SRCS, HEADER))


if __name__ == "__main__":
    build_library()
