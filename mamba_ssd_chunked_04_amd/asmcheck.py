"""A check of the library's gfx950 device assembly for one miscompile.

hipcc (ROCm 7.2) has been seen to place a register spill store
(`scratch_store_*`) in the join block of a divergent region before that
block's exec restore (`s_or_b64 exec, exec, sN`): the spill then runs only
for the lanes that took the region, and a value reloaded later comes back
as garbage in the others.  In the fused-norm forward this dropped the final
state of seven waves in eight.  The kernels are written to avoid the
pattern (wave-uniform branches, no accumulators held across chunks); this
module compiles the forward's translation units to assembly and reports any
kernel in which the pattern appears, so a change of code or compiler that
brings it back is caught on the CPU.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

from .build import ARCH, FLAGS, PKG_DIR

FWD_UNITS = tuple(os.path.join(PKG_DIR, "csrc", f)
                  for f in ("ssd_fwd_q64.hip", "ssd_fwd_q128.hip", "ssd_fwd_q256.hip"))


def device_asm(src: str, out_dir: str) -> str:
    """Compile one translation unit's device code to gfx950 assembly."""
    hipcc = os.environ.get("HIPCC", "hipcc")
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    flags = [f for f in FLAGS if f != "-fPIC"]
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", src, "-o", out]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{proc.stderr[-4000:]}")
    return out


def spills_before_exec_restore(asm: str):
    """(kernel, count) for every kernel with a scratch store that precedes, in
    the same basic block, that block's `s_or_b64 exec, exec, s[..]`."""
    lines = asm.splitlines()
    found = []
    starts = [(i, m.group(1)) for i, l in enumerate(lines)
              for m in [re.match(r"^(_Z\S+):\s*;", l)] if m]
    for si, name in starts:
        end = next((i for i in range(si, len(lines)) if lines[i].startswith(".Lfunc_end")),
                   len(lines))
        bad, pending = 0, 0
        for l in lines[si + 1:end]:
            if re.match(r"^\.LBB\S+:", l) or l.startswith("; %bb."):
                pending = 0           # a new basic block
                continue
            t = l.strip()
            if t.startswith("scratch_store"):
                pending += 1
            elif re.match(r"s_or_b64 exec, exec, s\[", t):
                bad += pending
                pending = 0
        if bad:
            found.append((name, bad))
    return found


def check_forward(units=FWD_UNITS):
    """Compile the forward's units (in parallel) and return the offending
    kernels, [] when the assembly is clean."""
    with tempfile.TemporaryDirectory(prefix="ssd_asm_") as tmp:
        with ThreadPoolExecutor(len(units)) as ex:
            paths = list(ex.map(lambda u: device_asm(u, tmp), units))
        bad = []
        for p in paths:
            with open(p) as f:
                bad += spills_before_exec_restore(f.read())
    return bad


if __name__ == "__main__":
    res = check_forward()
    for name, n in res:
        print(f"{n} spill store(s) before an exec restore in {name}")
    print("clean" if not res else f"{len(res)} kernel(s) affected")
    raise SystemExit(1 if res else 0)
