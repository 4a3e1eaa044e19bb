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
# The same sources with every launch taking its streaming (non-temporal) instantiation, at
# any size: a test build, so that small parity cases exercise the code paths that
# otherwise only launches above the cache budget take.
STREAM_LIB = os.path.join(HERE, "libulp_stream.so")
STREAM_FLAGS = ["-DULP_RESIDENT_MB=0"]

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


def _start(out: str, extra: list[str] | None, verbose: bool):
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra or []), "-I", INCLUDE, "-I", CSRC, *sources(),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    return proc, tmp, out


def _finish(job) -> str:
    proc, tmp, out = job
    _, err = proc.communicate()
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err[-6000:]}")
    os.replace(tmp, out)    # atomic: a loader never sees a partial file
    return out


def build(out: str = LIB, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile libulp.so in-tree (atomically replaced) and return its path."""
    return _finish(_start(out, extra, verbose))


def build_all(verbose: bool = False) -> list[str]:
    """libulp.so and the streaming test build libulp_stream.so, compiled side by side."""
    jobs = [_start(LIB, None, verbose), _start(STREAM_LIB, STREAM_FLAGS, verbose)]
    return [_finish(j) for j in jobs]


if __name__ == "__main__":
    print(build_all(verbose=True))
