"""Pins of the oracle's caller-held V scale (CPU only).

The unpack_for_sage page (Returns) leaves the V scale with the caller.  Reading: when the
caller hands one over, a [B,H,D] float32 divisor per (batch, global head, channel), V
becomes E4M3(RN32(fp32(v) / scale)) -- one IEEE binary32 division, then the same
round-to-nearest-even saturating E4M3 conversion as the unscaled path.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import brute, pipeline
from precision_attention_input_amd import workloads as W

from helpers import check_outputs_against_definition, small

CASES = [small(B=2, P=4, L=100, H=8, D=64, used=301, scale_sequence=301, seed=11),
         small(P=2, L=65, H=6, D=128, dtype=torch.float16, used=100, seed=12),
         small(P=8, L=40, H=16, D=64, dtype=torch.float16, seed=13),
         W.BATCHED_SMALL_HEAD.with_(B=2, L=96, H=4, used=150, scale_sequence=150)]


def run(w, vs, d=None):
    d = d or W.generate(w)
    return d, pipeline.run_group(d["Q"], d["K"], d["V"], d["mean"], world_size=w.P,
                                 used_sequence=w.used, scale_sequence=w.scale_sequence,
                                 v_scale=vs)


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_v_scale_matches_definition(olib, w):
    """The per-rank oracle against the definition oracle (one library division per value
    of the whole tensor, torch's E4M3 conversion), every output."""
    vs = W.v_scale(w)
    d, res = run(w, vs)
    df = brute.define(d["Q"], d["K"], d["V"], d["mean"], world_size=w.P,
                      used_sequence=w.used, v_scale=vs)
    check_outputs_against_definition(res["outs"], df, w)


def test_unit_scale_equals_unscaled(olib):
    w = CASES[0]
    d, a = run(w, None)
    _, b = run(w, torch.ones(w.B, w.H, w.D), d)
    for r in range(w.P):
        assert torch.equal(a["sends"][r], b["sends"][r])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_power_of_two_scale_is_exact_rescaling(olib, dtype):
    """v / 2^k is exact, so the scaled path equals the unscaled path on V * 2^-k (exact in
    the input dtype for these ranges); Q and K bytes do not change."""
    w = small(B=2, P=4, L=70, H=8, D=64, dtype=dtype, used=250, seed=14)
    d = W.generate(w)
    g = torch.Generator().manual_seed(5)
    lo, hi = (-6, 7) if dtype == torch.bfloat16 else (-3, 1)   # fp16: no subnormal loss
    k = torch.randint(lo, hi, (w.B, w.H, w.D), generator=g).float()
    vs = torch.exp2(k)
    _, a = run(w, vs, d)
    d2 = dict(d)
    d2["V"] = (d["V"].float() * torch.exp2(-k)[:, None]).to(dtype)
    assert torch.equal(d2["V"].float(), d["V"].float() * torch.exp2(-k)[:, None])
    _, b = run(w, None, d2)
    for p in range(w.P):
        for i in range(5):
            assert torch.equal(a["outs"][p][i].view(torch.uint8) if i == 2 else a["outs"][p][i],
                               b["outs"][p][i].view(torch.uint8) if i == 2 else b["outs"][p][i])


def _one(v, s, dtype=torch.float16):
    """E4M3 byte of a single value through the oracle's pack with scale s."""
    w = small(B=1, P=2, L=64, H=2, D=64, dtype=dtype, seed=0)
    z = torch.zeros(1, 64, 2, 64, dtype=dtype)
    V = z.clone()
    V[0, 0, 0, 0] = v
    vs = torch.ones(1, 2, 64)
    vs[0, 0, 0] = s
    amax = torch.full((1, 2, 1), 1.0)
    send = oracle.pack(z, z, V, torch.zeros(1, 2, 64, dtype=dtype), amax, amax, rank=0,
                       world_size=2, v_scale=vs)
    cb = send.shape[1]
    sec = (64 * 1 * 64 + 255) // 256 * 256
    return int(send[0, 2 * sec])


def test_hand_worked_values(olib):
    """Worked by hand: 1/0.5 = 2 -> 0x40; 3/3 = 1 -> 0x38; RN32(1/3) = 0.3333333 lies
    between 0.3125 and 0.34375 above their midpoint 0.328125 -> 0x2B; -100/0.125 = -800
    saturates -> 0xFE; 1/512 = 2^-9 -> 0x01 (smallest subnormal); 1/1024 is the tie between
    0 and 2^-9 -> 0x00 (even); 3/2048 = 0.75 * 2^-9 -> 0x01."""
    for v, s, code in [(1.0, 0.5, 0x40), (3.0, 3.0, 0x38), (1.0, 3.0, 0x2B),
                       (-100.0, 0.125, 0xFE), (1.0, 512.0, 0x01), (1.0, 1024.0, 0x00),
                       (3.0, 2048.0, 0x01)]:
        assert _one(v, s) == code, (v, s)


def _double_rounding_pairs(mid: Fraction, above: bool, n: int = 3):
    """(v, s): integer v < 2048 (exact in fp16) and float32 s near v/mid whose exact
    quotient differs from mid, on the given side, while RN32(v/s) == mid."""
    out = []
    for vi in range(1025, 2048):
        t = np.float32(float(Fraction(vi) / mid))
        for s32 in (np.nextafter(t, np.float32(-np.inf)), t, np.nextafter(t, np.float32(np.inf))):
            q = Fraction(vi) / Fraction(float(s32))
            if q == mid or (q > mid) != above:
                continue
            if Fraction(float(np.float32(float(q)))) == mid:   # float(q): correctly rounded
                out.append((float(vi), float(s32)))
        if len(out) >= n:
            return out
    return out


def test_scale_division_rounds_to_binary32_first(olib):
    """The quotient is rounded to binary32 before the E4M3 rounding.  Pairs whose exact
    quotient lies just beside an E4M3 midpoint but whose binary32 quotient IS the midpoint
    take the tie-to-even code, not the code the exact quotient is nearest to:
    1.0625 (between 1.0 = 0x38 and 1.125 = 0x39) -> 0x38 even from just above;
    1.1875 (between 1.125 = 0x39 and 1.25 = 0x3A) -> 0x3A even from just below."""
    for mid, above, code, exact_code in [(Fraction(17, 16), True, 0x38, 0x39),
                                         (Fraction(19, 16), False, 0x3A, 0x39)]:
        pairs = _double_rounding_pairs(mid, above)
        assert pairs, f"no pair found for {mid}"
        for v, s in pairs:
            assert _one(v, s) == code, (v, s)
            assert code != exact_code
