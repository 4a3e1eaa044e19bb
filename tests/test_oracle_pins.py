"""Pins of the CPU oracle against facts fixed outside it (CPU only).

* E4M3: the OCP specification's table, a nearest-code brute force over every bf16 and
  fp16 input, and torch's float8_e4m3fn conversion.
* INT8 quantization: exact rational arithmetic.
* Binary16 / bfloat16 decoding: numpy's and torch's own conversions.
* The derive identity of the derive_k_boundary_amax page (description), checked on raw
  float32 arithmetic with no oracle code involved.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- E4M3

def e4m3_code_values():
    """The 256 E4M3FN codes decoded from the OCP definition (NaN codes -> None)."""
    vals = []
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 15 and m == 7:
            vals.append(None)
        elif e == 0:
            vals.append(s * m * 2.0 ** -9)
        else:
            vals.append(s * (1 + m / 8) * 2.0 ** (e - 7))
    return vals


_CODE_VALUES = None


def e4m3_nearest(x: float) -> int:
    """Brute force: the finite code of x's sign nearest to x in exact arithmetic; ties go to
    the even fraction.  Nearest-finite already saturates (448 is the nearest finite code to
    anything above it); an infinity takes the largest magnitude."""
    global _CODE_VALUES
    if _CODE_VALUES is None:
        _CODE_VALUES = [None if v is None else Fraction(v) for v in e4m3_code_values()]
    neg = math.copysign(1.0, x) < 0
    best, best_d = None, None
    for c, v in enumerate(_CODE_VALUES):
        if v is None or bool(c & 0x80) != neg:
            continue
        d = -abs(v) if math.isinf(x) else abs(v - Fraction(x))
        if best is None or d < best_d or (d == best_d and (c & 1) == 0 and (best & 1) == 1):
            best, best_d = c, d
    return best


def test_e4m3_ocp_table(olib):
    rows = 0
    for line in open(os.path.join(GOLDEN, "e4m3_ocp_values.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        lit, code = line.split()[:2]
        x = float(lit)
        assert oracle.e4m3(x) == int(code, 16), (lit, hex(oracle.e4m3(x)))
        rows += 1
    assert rows >= 15


def all_patterns(dtype):
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    x = bits.view(dtype).float()
    return x[torch.isfinite(x)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_e4m3_exhaustive_vs_brute_force_and_torch(olib, dtype):
    xs = all_patterns(dtype)
    ours = np.array([oracle.e4m3(float(v)) for v in xs.tolist()], dtype=np.uint8)
    lib_codes = xs.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, lib_codes)
    # nearest-code search on a subset that covers every binade and both signs densely
    vals = xs.tolist()
    for i in range(0, len(vals), 7):
        assert ours[i] == e4m3_nearest(vals[i]), vals[i]


def test_e4m3_nearest_code_on_every_fp8_midpoint(olib):
    """Every midpoint between adjacent codes (exact in fp32) is a tie: even fraction wins."""
    vals = sorted(v for v in e4m3_code_values() if v is not None and v >= 0)
    for a, b in zip(vals, vals[1:]):
        mid = (a + b) / 2
        for x in (mid, -mid, np.nextafter(np.float32(mid), np.float32(0)),
                  np.nextafter(np.float32(mid), np.float32(1e9))):
            assert oracle.e4m3(float(x)) == e4m3_nearest(float(x)), x


# ----------------------------------------------------------------------------- INT8

def round_half_even(r: Fraction) -> int:
    n = math.floor(r)
    frac = r - n
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def rn32(r: Fraction) -> Fraction:
    """Exact round-to-nearest-even of a rational to binary32 (no overflow in these tests)."""
    if r == 0:
        return Fraction(0)
    e = math.floor(math.log2(abs(r)))
    while Fraction(2) ** e > abs(r):
        e -= 1
    while Fraction(2) ** (e + 1) <= abs(r):
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - 23)
    return round_half_even(r / ulp) * ulp


def exact_quant(x: float, s: float) -> int:
    """clamp(rint(RN32(x / s)), -127, 127) in exact rational arithmetic."""
    return max(-127, min(127, round_half_even(rn32(Fraction(x) / Fraction(s)))))


def test_quant_i8_exact_rational(olib):
    rng = np.random.default_rng(0)
    s_vals = (rng.random(300) * 2.0 ** rng.integers(-20, 10, 300)).astype(np.float32)
    for s in s_vals:
        s = float(s)
        if s == 0:
            continue
        xs = (rng.standard_normal(20) * s * 60).astype(np.float32).tolist()
        # near-tie and exact-tie numerators: (k + 1/2) * s rounded to binary32, +- 1 ulp
        for k in (-128, -127, -3, -1, 0, 1, 2, 63, 126, 127):
            t = np.float32((k + 0.5) * s)
            xs += [float(t), float(np.nextafter(t, np.float32(1e30))),
                   float(np.nextafter(t, np.float32(-1e30)))]
        for x in xs:
            assert oracle.quant_i8(x, s) == exact_quant(x, s), (x, s)


def test_quant_i8_ties_go_to_even(olib):
    for k in range(-127, 127):
        x = k + 0.5          # exact binary32, scale 1 => quotient exactly k + 1/2
        want = k if k % 2 == 0 else k + 1
        assert oracle.quant_i8(x, 1.0) == max(-127, min(127, want))
    assert oracle.quant_i8(1e30, 1e-9) == 127
    assert oracle.quant_i8(-1e30, 1e-9) == -127


# ----------------------------------------------------------------------------- decoding

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_input_decoding_matches_library(olib, dtype):
    """The oracle's amax of a one-element shard is |value|: decode every finite pattern."""
    xs = all_patterns(dtype).to(dtype)
    # shard [B=1, L=64, H=2, D=64]: put each value alone into rank 0's first group
    vals = xs.float()
    n = vals.numel()
    got = []
    for i in range(0, n, 97):
        x = torch.zeros(1, 64, 2, 64, dtype=dtype)
        x[0, 5, 1, 7] = xs[i]
        a = oracle.k_grouped_amax(x, None, rank=0, world_size=2)
        got.append((float(a[0, 1, 0]), max(abs(float(vals[i])), float(np.float32(1e-7)))))
    for g, want in got:
        assert g == np.float32(want)


# ----------------------------------------------------------------------------- derive identity

def test_derive_identity_on_float32_arithmetic():
    """max_t |RN(k_t - m)| == max(RN(maxK - m), RN(m - minK)) for float32 RN subtraction
    (derive_k_boundary_amax description), on adversarial spreads: values straddling m,
    exponents far apart, subnormals, exact ties of |k - m|."""
    rng = np.random.default_rng(1)
    for trial in range(4000):
        n = int(rng.integers(1, 70))
        m = np.float32(rng.standard_normal() * 10.0 ** rng.integers(-30, 30))
        kind = trial % 4
        if kind == 0:
            k = (m + rng.standard_normal(n) * abs(m) * 1e-3).astype(np.float32)
        elif kind == 1:
            k = (rng.standard_normal(n) * 10.0 ** rng.integers(-38, 38, n)).astype(np.float32)
        elif kind == 2:
            k = np.array([np.nextafter(m, np.float32(np.inf)) if i % 2 else
                          np.nextafter(m, np.float32(-np.inf)) for i in range(n)], np.float32)
        else:
            k = (m + np.float32(2.0) ** rng.integers(-149, 20, n).astype(np.float32)
                 * rng.choice([-1, 1], n)).astype(np.float32)
        k = k[np.isfinite(k)]
        if k.size == 0:
            continue
        with np.errstate(over="ignore"):
            direct = np.max(np.abs(k - m))
            derived = max(np.float32(k.max() - m), np.float32(m - k.min()))
        assert direct.view(np.uint32) == np.float32(derived).view(np.uint32) or (
            np.isinf(direct) and np.isinf(derived))
