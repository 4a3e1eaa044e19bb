"""Build of libulp.so: every HIP source under csrc/ compiled for gfx950 by hipcc."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libulp.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every fp32 operation stays a separately rounded IEEE operation
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libulp)")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile libulp.so in-tree (atomically replaced) and return its path."""
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra or []), "-I", INCLUDE, "-I", CSRC, *sources(),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stderr[-6000:]}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
