"""Properties of the consumer kernel's gfx950 code that its correctness rests on, checked
on the compiler's assembly (CPU; hipcc cross-compiles):

* M0 is written only by the kernel's own global -> LDS loads (inline asm that sets M0 to
  the LDS destination and does not declare it, since the compiler reserves M0): no code
  the compiler emits may use M0;
* no MFMA runs with part of the wave switched off: between a `s_and_saveexec` and the
  instruction that restores EXEC there is no MFMA.  (An MFMA reads operand rows from every
  lane; run under a partial EXEC mask the rows of the inactive lanes come out wrong.  The
  kernel pins its accumulators before the output branch because the compiler once moved
  the last tile's MFMAs into it.)"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from precision_attention_input_amd import _build


def kernels(asm: str) -> dict[str, list[str]]:
    out, name, body = {}, None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S*consumer_kernel\S*):", line)
        if m:
            name, body = m.group(1), []
            continue
        if name:
            body.append(line)
            if "s_endpgm" in line:
                out[name], name = body, None
    return out


def check_m0(body: list[str]) -> list[str]:
    bad, in_asm = [], False
    for line in body:
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
        elif s.startswith(";;#ASMEND"):
            in_asm = False
        elif not in_asm and not s.startswith(";") and re.search(r"\bm0\b", s):
            bad.append(s)
    return bad


def check_mfma_exec(body: list[str]) -> list[str]:
    bad, masked_from = [], None
    for i, line in enumerate(body):
        s = line.strip()
        if s.startswith(";"):
            continue
        if s.startswith("s_and_saveexec"):
            masked_from = i
        elif re.match(r"s_(or|mov|and)_b64\s+exec\s*,", s) or s.startswith("s_endpgm"):
            masked_from = None
        elif masked_from is not None and s.startswith("v_mfma"):
            bad.append(f"{s} (EXEC masked since line {masked_from})")
    return bad


@pytest.fixture(scope="module")
def consumer_asm(tmp_path_factory):
    src = os.path.join(_build.CSRC, "consumer.hip")
    out = str(tmp_path_factory.mktemp("asm") / "consumer.s")
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [_build.hipcc(), *flags, "--cuda-device-only", "-S", "-I", _build.INCLUDE,
           "-I", _build.CSRC, src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    return open(out).read()


def test_consumer_kernels_present(consumer_asm):
    ks = kernels(consumer_asm)
    assert len(ks) == 3, sorted(ks)       # D = 64 4x1, D = 128 4x1 and 8x2


def test_m0_written_only_by_the_lds_loads(consumer_asm):
    for name, body in kernels(consumer_asm).items():
        assert check_m0(body) == [], name
        assert any("s_mov_b32 m0" in l for l in body), name


def test_no_mfma_under_a_partial_exec_mask(consumer_asm):
    for name, body in kernels(consumer_asm).items():
        assert any(l.strip().startswith("v_mfma") for l in body), name
        assert check_mfma_exec(body) == [], name
