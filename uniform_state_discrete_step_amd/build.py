"""Build libdgd.so in-tree for gfx950 with hipcc.

Usage: ``python -m uniform_state_discrete_step_amd.build`` (or
``__graft_entry__.build()``).  Always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "dgd.hip")]
OUTPUT = os.path.join(HERE, "libdgd.so")
# the same library with the projection's phase timing recorded (a measurement
# build: dgd_phase_times reports only there)
OUTPUT_PHASE = os.path.join(HERE, "libdgd_phase.so")

HIPCC_FLAGS = [
    "-O3",
    "--offload-arch=gfx950",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, phase_timing: bool = False) -> str:
    out = OUTPUT_PHASE if phase_timing else OUTPUT
    tmp = out + ".tmp"
    defs = ["-DDGD_PHASE_TIMING"] if phase_timing else []
    cmd = [hipcc(), *HIPCC_FLAGS, *defs, "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, phase_timing="--phase-timing" in sys.argv))
