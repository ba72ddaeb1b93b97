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
             for f in ("ssd_fwd_q64.hip", "ssd_fwd_q128.hip", "ssd_fwd_q256.hip", "ssd_fwd.hip",
                       "ssd_bwd.hip", "rmsnorm_gated.hip", "causal_conv1d.hip"))
HEADERS = (os.path.join(REPO_DIR, "include", "ssd_mi355x.h"),
           os.path.join(PKG_DIR, "csrc", "ssd_fwd_impl.h"))
LIB = os.path.join(PKG_DIR, "libssd_mi355x.so")
# calibration kernels the benchmark measures the GPU's own peaks with (not
# part of the SSD library)
CALIB_SRC = os.path.join(PKG_DIR, "csrc", "calib.hip")
CALIB_LIB = os.path.join(PKG_DIR, "libssd_calib.so")
ARCH = "gfx950"


FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-pass-failed", "-I", os.path.join(REPO_DIR, "include")]
BUILD_DIR = os.path.join(REPO_DIR, "_build")


def hipcc_command(out_path: str = LIB, extra=()) -> list:
    """One command that compiles every source and links the library."""
    hipcc = os.environ.get("HIPCC", "hipcc")
    return [hipcc, *FLAGS, "-shared", *SRCS, "-o", out_path, *extra]


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
    return proc.returncode, err


def build_library(verbose: bool = True) -> str:
    """Always recompiles (the sources in parallel, then one link); writes the
    library atomically."""
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", "hipcc")
    os.makedirs(BUILD_DIR, exist_ok=True)
    tag = "%d" % os.getpid()
    objs = [os.path.join(BUILD_DIR, os.path.basename(src) + "." + tag + ".o") for src in SRCS]
    tmp = LIB + ".tmp" + tag
    t0 = time.time()
    jobs = min(len(SRCS), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    try:
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(lambda so: _run([hipcc, *FLAGS, "-c", so[0], "-o", so[1]]),
                                  zip(SRCS, objs)))
        err = "\n".join(e for _, e in results if e.strip())
        bad = [src for (rc, _), src in zip(results, SRCS) if rc != 0]
        if bad:
            raise RuntimeError(f"hipcc failed on {', '.join(map(os.path.basename, bad))}:\n{err}")
        rc, lerr = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
        if rc != 0:
            raise RuntimeError(f"hipcc link failed ({rc}):\n{lerr}")
        err = (err + "\n" + lerr).strip()
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
        if os.path.exists(tmp):
            os.remove(tmp)
    if verbose:
        print(f"[build] {os.path.relpath(LIB, REPO_DIR)} in {time.time() - t0:.1f}s", file=sys.stderr)
        if err.strip():
            print(err, file=sys.stderr)
    return LIB


def build_calibration(verbose: bool = True) -> str:
    """Compiles the benchmark's calibration kernels (always)."""
    hipcc = os.environ.get("HIPCC", "hipcc")
    tmp = CALIB_LIB + ".tmp%d" % os.getpid()
    t0 = time.time()
    rc, err = _run([hipcc, *FLAGS, "-shared", CALIB_SRC, "-o", tmp])
    if rc != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed on calib.hip ({rc}):\n{err}")
    os.replace(tmp, CALIB_LIB)
    if verbose:
        print(f"[build] {os.path.relpath(CALIB_LIB, REPO_DIR)} in {time.time() - t0:.1f}s",
              file=sys.stderr)
    return CALIB_LIB


def library_is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in (*SRCS, *HEADERS))


if __name__ == "__main__":
    build_library()
    build_calibration()
