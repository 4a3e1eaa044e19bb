"""The caller-held V scale through the HIP pack (GPU), bit for bit against the oracle.

With a [B,H,D] float32 V scale the pack writes E4M3(RN32(fp32(v) / scale)) (the V scale
stays with the caller, unpack_for_sage Returns); every other output is unchanged.  Checked
on the three smaller workloads (group and per-rank entry points; the two large ones in
test_gpu_large_parity.py),
on every 16-bit input pattern, at saturation and in the E4M3 subnormal range, and on
quotients whose binary32 rounding lands exactly on an E4M3 midpoint.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import pipeline
import precision_attention_input_amd as ulp
from precision_attention_input_amd import workloads as W

from gpu_helpers import DEV, assert_bits_equal, compare_all, run_group, run_per_rank, say, \
    to_dev
from helpers import small
from test_oracle_vscale import _double_rounding_pairs

pytestmark = pytest.mark.gpu


def oracle_run(w, d, vs):
    return pipeline.run_group(d["Q"], d["K"], d["V"], d["mean"], world_size=w.P,
                              used_sequence=w.used, scale_sequence=w.scale_sequence,
                              v_scale=vs)


@pytest.mark.parametrize("wname", [W.TINY.name, W.UNALIGNED_PADDED.name,
                                   W.BATCHED_SMALL_HEAD.name])
@pytest.mark.parametrize("mode", ["group", "per_rank"])
def test_workload_v_scale_parity(olib, wname, mode):
    w = W.BY_NAME[wname]
    say(f"[v_scale] {wname} mode={mode}")
    d = W.generate(w)
    vs = W.v_scale(w)
    dd = to_dev(d, w.P)
    vsd = vs.to(DEV)
    g = (run_group(w, dd, w.aligned, v_scale=vsd) if mode == "group"
         else run_per_rank(w, dd, w.aligned, v_scale=vsd))
    compare_all(g, oracle_run(w, d, vs), w, f"{wname}/{mode}/v_scale")


def _patterns(dtype):
    bitsrc = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(dtype)
    return torch.where(torch.isfinite(bitsrc.float()), bitsrc, torch.zeros_like(bitsrc))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_every_input_pattern_with_scales(olib, dtype):
    """All 65536 16-bit patterns as V, twice, against per-channel scales spread over 2^-20 ..
    2^20 with arbitrary mantissas: saturation, normals, subnormals and zero."""
    say(f"[v_scale exhaustive] {dtype}")
    P, L, H, D = 2, 256, 2, 128
    x = _patterns(dtype).repeat(2).view(1, P * L, H, D)
    w = small(P=P, L=L, H=H, D=D, dtype=dtype)
    g = torch.Generator().manual_seed(21)
    vs = torch.exp2(torch.empty(1, H, D).uniform_(-20.0, 20.0, generator=g))
    d = dict(Q=x.clone(), K=x.clone(), V=x.clone())
    d["mean"] = W.k_mean_global(d["K"], P * L, dtype)
    dd = to_dev(d, P)
    compare_all(run_group(w, dd, v_scale=vs.to(DEV)), oracle_run(w, d, vs), w,
                "v_scale exhaustive")


def test_midpoint_quotients_and_extremes(olib):
    """Pairs (v, s) whose exact quotient is just beside an E4M3 midpoint while the binary32
    quotient is the midpoint itself (both tie directions), exact midpoints, and scales that
    push quotients past 448 or below the smallest subnormal."""
    say("[v_scale midpoints]")
    P, L, H, D = 2, 64, 2, 64
    w = small(P=P, L=L, H=H, D=D, dtype=torch.float16)
    pairs = []
    for mid, above in [(Fraction(17, 16), True), (Fraction(19, 16), False),
                       (Fraction(17, 16), False), (Fraction(19, 16), True)]:
        pairs += _double_rounding_pairs(mid, above, n=8)
    V = torch.zeros(1, P * L, H, D)
    vs = torch.ones(1, H, D)
    # channel c of head 0 carries pair c in every row (scaled by powers of two per row so the
    # rows visit other binades of the same mantissa pattern)
    for c, (v, s) in enumerate(pairs[:D]):
        vs[0, 0, c] = s
        for t in range(P * L):
            V[0, t, 0, c] = v * 2.0 ** -((t % 12))
    # head 1: fixed values against extreme scales
    ext = [2.0 ** -30, 2.0 ** -20, 1e-3, 0.3, 1.0, 3.0, 1e3, 2.0 ** 20, 2.0 ** 30, 7.5]
    for c in range(D):
        vs[0, 1, c] = float(np.float32(ext[c % len(ext)] * (1 + c / 97)))
        for t in range(P * L):
            V[0, t, 1, c] = ((t * 37 + c * 11) % 2001 - 1000) / 64.0
    V16 = V.to(torch.float16)
    assert torch.equal(V16.float(), V)
    d = dict(Q=V16.clone(), K=V16.clone(), V=V16)
    d["mean"] = W.k_mean_global(d["K"], P * L, torch.float16)
    dd = to_dev(d, P)
    compare_all(run_group(w, dd, v_scale=vs.to(DEV)), oracle_run(w, d, vs), w, "midpoints")
    compare_all(run_per_rank(w, dd, v_scale=vs.to(DEV)), oracle_run(w, d, vs), w,
                "midpoints per rank")


def test_v_scale_leaves_q_and_k_unchanged(olib):
    """Only the V section of each chunk depends on the V scale."""
    w = W.UNALIGNED_PADDED
    d = W.generate(w)
    dd = to_dev(d, w.P)
    a = run_group(w, dd)
    b = run_group(w, dd, v_scale=W.v_scale(w).to(DEV))
    for p in range(w.P):
        for i in (0, 1, 3, 4):
            assert_bits_equal(a["outs"][p][i], b["outs"][p][i], f"output {i} dest {p}")
    assert not torch.equal(a["outs"][0][2].view(torch.uint8), b["outs"][0][2].view(torch.uint8))
