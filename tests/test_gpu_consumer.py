"""The consumer check on the HIP path's outputs (GPU): attention read from the unpacked
tensors the way the Sage consumer reads them (oracle/consumer.py, float64 on the CPU),
against float64 attention on the original inputs, at the full workload shapes (sampled
heads and query rows), with and without a caller V scale.  Bounds and their rationale are
those of tests/test_oracle_consumer.py."""
from __future__ import annotations

import math

import pytest
import torch

from precision_attention_input_amd import workloads as W

import precision_attention_input_amd as ulp

from gpu_helpers import DEV, run_group, say, to_dev
from helpers import small
from test_oracle_consumer import COS, REL, caller_v_scale, grouped_inputs
from oracle import consumer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wname", [w.name for w in W.WORKLOADS])
def test_consumer_on_gpu_outputs(olib, wname):
    w, d = grouped_inputs(W.BY_NAME[wname])
    say(f"[consumer] {wname}")
    vs = caller_v_scale(d, w) if w.dtype == torch.float16 else None
    dd = to_dev(d, w.P)
    g = run_group(w, dd, w.aligned, v_scale=None if vs is None else vs.to(DEV))
    used = w.used or w.S
    qsel = sorted(set(list(range(0, used, max(1, used // 24))) + [used - 1]))
    heads = W.sample_heads(w, per_dest=1)
    worst = None
    for p, hh in enumerate(heads):
        j = hh - p * w.h
        q8, k8, v8, qs, ks = (t.cpu() for t in g["outs"][p])
        for b in range(w.B):
            o = consumer.quantized_attention(q8, k8, v8, qs, ks, b=b, j=j, queries=qsel,
                                             used=used,
                                             v_scale_row=None if vs is None else vs[b, hh])
            r = consumer.reference_attention(d["Q"], d["K"], d["V"], b=b, head=hh,
                                             queries=qsel, used=used)
            c = consumer.compare(o, r)
            if worst is None or c["rel_l2"] > worst["rel_l2"]:
                worst = c
    say(f"[consumer] {wname}: worst {worst}")
    assert worst["cos"] >= COS and worst["rel_l2"] <= REL, worst


# ----------------------------------------------------------------- the MFMA consumer kernel

# Against attention on the original inputs (ref_in) the FP8 consumer is held to a bound
# derived per (b, head), with no constant of its own: its elements lie within the
# per-element FP8-probability bound e of the float64 consumer on the same bytes (exact,
# checked first), so by the triangle inequality
#     ||got - ref_in|| <= ||exact - ref_in|| + ||e||,
# i.e. rel_l2(got) <= rel_l2(exact) + ||e|| / ||ref_in|| =: r, and cos(got, ref_in) >=
# sqrt(1 - r^2) (a vector within r |ref_in| of ref_in, r < 1, makes at most that angle).
# How far exact itself lies from ref_in is the input quantization, which
# test_consumer_on_gpu_outputs holds to COS / REL.
def mfma_exponent_error(qs, ks, b: int, j: int, D: int) -> float:
    """How far (log2 units) the MFMA kernel's exponent arguments may lie from the exact
    score * log2(e) - running maximum.  The kernel reads its dot products biased by
    1.5 * 2^23 and folds the bias into the offset 1.5 * 2^23 * scl + m - log2(448), which
    it rounds once: half an ulp of at most (1.5 * 2^23 + 127^2 D) scl + 9, where
    scl = q_scale * k_scale * log2(e) / sqrt(D) <= the largest such product of the head.
    scl itself carries three binary32 roundings, a relative 3 * 2^-24 on
    |dot * scl| <= 127^2 D scl; the fma and the exp2 each round on arguments of magnitude
    up to a few hundred.  Taken here as a full ulp of the sum, with room to spare."""
    scl = float(qs[b, j].max()) * float(ks[b, j].max()) * math.log2(math.e) / math.sqrt(D)
    return 2.0 ** -23 * ((1.5 * 2 ** 23 + 4 * 127 ** 2 * D) * scl + 256)


def _check_mfma_consumer(w, d, g, vs, dests, heads_of, nq, label):
    used = w.used or w.S
    qsel = sorted(set(list(range(0, used, max(1, used // nq))) + [used - 1, used // 2]))
    worst, e2e = 0.0, None
    for p in dests:
        q8, k8, v8, qs, ks = g["outs"][p]
        vsp = None if vs is None else vs[:, p * w.h:(p + 1) * w.h].contiguous().to(DEV)
        out = ulp.consumer_attention(q8, k8, v8, qs, ks, used=used, v_scale=vsp)
        torch.cuda.synchronize()
        out = out.cpu()
        c8 = [t.cpu() for t in (q8, k8, v8, qs, ks)]
        for b in range(w.B):
            for j in heads_of(p):
                hh = p * w.h + j
                row = None if vs is None else vs[b, hh]
                xerr = mfma_exponent_error(c8[3], c8[4], b, j, q8.shape[-1])
                ref, bound = consumer.fp8_probability_bound(*c8, b=b, j=j, queries=qsel,
                                                            used=used, v_scale_row=row,
                                                            exponent_error=xerr)
                got = out[b, qsel, j].double()
                ratio = ((got - ref).abs() / bound).max().item()
                assert ratio <= 1.0, f"{label}: dest {p} b {b} head {j}: error/bound {ratio}"
                worst = max(worst, ratio)
                ref_in = consumer.reference_attention(d["Q"], d["K"], d["V"], b=b, head=hh,
                                                      queries=qsel, used=used)
                exact = consumer.compare(ref, ref_in)
                r = exact["rel_l2"] + float(bound.norm() / ref_in.norm())
                c = consumer.compare(got, ref_in)
                c["allowed_rel_l2"] = r
                assert c["rel_l2"] <= r * (1 + 1e-9), (label, p, b, j, c)
                if r < 1:
                    assert c["cos"] >= (1 - r * r) ** 0.5 - 1e-9, (label, p, b, j, c)
                if e2e is None or c["rel_l2"] > e2e["rel_l2"]:
                    e2e = c
        assert torch.isfinite(out).all()
    say(f"[mfma consumer] {label}: worst error/bound {worst:.3f}, vs inputs {e2e}")


@pytest.mark.parametrize("wname", [w.name for w in W.WORKLOADS])
def test_mfma_consumer_within_fp8_bound(olib, wname):
    """The gfx950 MFMA consumer (INT8 Q.K, FP8 P.V) on the HIP path's unpacked tensors, every
    element of sampled query rows within the FP8-probability bound of the float64 consumer
    (oracle/consumer.py), with a caller V scale on the fp16 workloads."""
    w, d = grouped_inputs(W.BY_NAME[wname])
    vs = caller_v_scale(d, w) if w.dtype == torch.float16 else None
    dd = to_dev(d, w.P)
    g = run_group(w, dd, w.aligned, v_scale=None if vs is None else vs.to(DEV))
    big = w.S > 10000
    dests = [0, w.P - 1] if big else list(range(w.P))
    heads_of = (lambda p: [0, w.h - 1]) if big else (lambda p: range(w.h))
    _check_mfma_consumer(w, d, g, vs, dests, heads_of, 12 if big else 40, wname)


@pytest.mark.parametrize("P,L,H,D,used", [(2, 1, 2, 64, 1), (2, 33, 4, 128, 50),
                                          (4, 100, 8, 64, 257), (8, 40, 8, 128, 320),
                                          (2, 96, 2, 128, 130), (2, 4000, 32, 128, 7999)])
def test_mfma_consumer_edges(olib, P, L, H, D, used):
    """One live row, used below / at / just past a 64-row group, S not a multiple of 64.
    The last case has enough query tiles (2 x 16 heads x 32 tiles of 256 queries) for the
    launcher's 256-query workgroups, with a partial last key tile, a last workgroup whose
    waves end past `used` and past S."""
    w, d = grouped_inputs(small(B=2, P=P, L=L, H=H, D=D, dtype=torch.float16, used=used,
                                scale_sequence=used, seed=used))
    vs = caller_v_scale(d, w)
    dd = to_dev(d, w.P)
    g = run_group(w, dd, v_scale=vs.to(DEV))
    _check_mfma_consumer(w, d, g, vs, range(w.P), lambda p: range(w.h), 64, w.name)


def test_mfma_consumer_rejects_bad_arguments(olib):
    """Validation happens before any launch (no kernel runs on these)."""
    q8 = torch.zeros(1, 64, 2, 64, dtype=torch.int8, device=DEV)
    v8 = torch.zeros(1, 64, 2, 64, dtype=torch.uint8, device=DEV)
    sc = torch.ones(1, 2, 1, device=DEV)
    with pytest.raises(ValueError, match="used"):
        ulp.consumer_attention(q8, q8, v8, sc, sc, used=65)
    with pytest.raises(ValueError, match="v_scale"):
        ulp.consumer_attention(q8, q8, v8, sc, sc, used=64, v_scale=torch.ones(1, 2, 32, device=DEV))


@pytest.mark.parametrize("wname,P,L,H,D,used", [
    ("unaligned_padded_b2_p4_l1000_h16_d128_fp16", None, None, None, None, None),
    ("batched_small_head_b4_p2_l2048_h24_d64_fp16", None, None, None, None, None),
    ("edge", 2, 4000, 32, 128, 7999), ("edge", 4, 100, 8, 64, 257),
    ("edge", 2, 33, 4, 128, 50)])
def test_mfma_consumer_query_position_invariance(olib, wname, P, L, H, D, used):
    """With no causal mask a query's output depends only on its own row and on its Q scale
    group, not on where the row sits among the queries: reversing the live rows of the last
    64-row group (one Q scale) must reverse their outputs bit for bit, and leave every other
    row's bits alone.  The reversal moves queries into and out of the last, partly live,
    wave of a workgroup, so any result that depends on a lane's neighbours or on which lanes
    are active (an MFMA run with part of the wave switched off, say) shows here."""
    if wname == "edge":
        w, d = grouped_inputs(small(B=2, P=P, L=L, H=H, D=D, dtype=torch.float16, used=used,
                                    scale_sequence=used, seed=used))
    else:
        w, d = grouped_inputs(W.BY_NAME[wname])
    say(f"[mfma consumer position] {w.name}")
    g = run_group(w, to_dev(d, w.P), w.aligned)
    n = w.used or w.S
    lo = (n - 1) // 64 * 64                      # first row of the last live 64-row group
    rows = torch.arange(lo, n, device=DEV)
    for p in range(w.P):
        q8, k8, v8, qs, ks = g["outs"][p]
        out = ulp.consumer_attention(q8, k8, v8, qs, ks, used=n)
        q8r = q8.clone()
        q8r[:, rows] = q8[:, rows.flip(0)]
        outr = ulp.consumer_attention(q8r, k8, v8, qs, ks, used=n)
        torch.cuda.synchronize()
        assert torch.equal(outr[:, :lo].view(torch.int32), out[:, :lo].view(torch.int32)), p
        assert torch.equal(outr[:, rows].view(torch.int32),
                           out[:, rows.flip(0)].view(torch.int32)), (p, lo, n)


def test_mfma_consumer_launch_shape_invariance(olib):
    """Each query's output is computed with the same operations in the same order whatever
    workgroup shape the launcher picks: run over 16 heads x 2 batch entries the launch takes
    256-query workgroups (8 waves of two 16-query blocks); head 3 alone, copied out, is too
    small a launch for that and takes 64-query ones (4 waves of one block).  The two must
    give the same bits for that head."""
    w, d = grouped_inputs(small(B=2, P=2, L=2000, H=32, D=128, dtype=torch.float16,
                                used=3999, scale_sequence=3999, seed=11))
    say(f"[mfma consumer shapes] {w.name}")
    g = run_group(w, to_dev(d, w.P), w.aligned)
    n = w.used
    assert (n + 255) // 256 * w.h * w.B >= 512          # the 256-query shape
    assert (n + 255) // 256 * 1 * w.B < 512              # one head: the 64-query shape
    q8, k8, v8, qs, ks = g["outs"][1]
    full = ulp.consumer_attention(q8, k8, v8, qs, ks, used=n)
    j = 3
    one = ulp.consumer_attention(q8[:, :, j:j + 1].contiguous(), k8[:, :, j:j + 1].contiguous(),
                                 v8[:, :, j:j + 1].contiguous(), qs[:, j:j + 1].contiguous(),
                                 ks[:, j:j + 1].contiguous(), used=n)
    torch.cuda.synchronize()
    assert torch.equal(one[:, :, 0].view(torch.int32), full[:, :, j].view(torch.int32))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("scale", [1e-3, 3e-2])
def test_mfma_consumer_extreme_dot_products(olib, D, scale):
    """Q and K codes of +-127 in whole rows, so that the dot products reach +-127^2 D, the
    ends of the range the kernel's biased accumulators must hold exactly; a small scale
    gives a flat softmax, a large one a peaked one.  Held to the same FP8 bound."""
    g = torch.Generator().manual_seed(D + int(scale * 1e4))
    B, h, S = 1, 2, 300
    sign = lambda n: torch.randint(0, 2, (n,), generator=g) * 2 - 1
    q8 = (127 * sign(B * S * h)).view(B, S, h, 1).expand(B, S, h, D).to(torch.int8).contiguous()
    k8 = (127 * sign(B * S * h)).view(B, S, h, 1).expand(B, S, h, D).to(torch.int8).contiguous()
    # a few rows with mixed signs, so the dots also take values between the extremes
    k8[:, ::7] = (127 * torch.randint(-1, 2, (B, len(range(0, S, 7)), h, D), generator=g)).to(torch.int8)
    spad = (S + 63) // 64 * 64
    codes = torch.randint(0, 256, (B, D, h, spad), generator=g, dtype=torch.int32)
    codes[(codes & 0x7F) == 0x7F] = 0x38                 # no NaN codes
    codes[..., S:] = 0
    v8 = codes.to(torch.uint8)
    W = (S + 63) // 64
    qs = torch.full((B, h, W), scale, dtype=torch.float32)
    ks = torch.full((B, h, W), scale, dtype=torch.float32) * torch.linspace(0.5, 1.5, W)
    say(f"[mfma consumer extremes] D={D} scale={scale}")
    out = ulp.consumer_attention(*(t.to(DEV) for t in (q8, k8, v8, qs, ks)), used=S)
    torch.cuda.synchronize()
    out = out.cpu()
    assert torch.isfinite(out).all()
    qsel = list(range(S))
    for j in range(h):
        xerr = mfma_exponent_error(qs, ks, 0, j, D)
        ref, bound = consumer.fp8_probability_bound(q8, k8, v8, qs, ks, b=0, j=j, queries=qsel,
                                                    used=S, exponent_error=xerr)
        ratio = ((out[0, :, j].double() - ref).abs() / bound).max().item()
        assert ratio <= 1.0, (D, scale, j, ratio)


def _random_geometries(n, seed=2024):
    g = torch.Generator().manual_seed(seed)
    out = []
    for _ in range(n):
        P = [2, 4, 8][int(torch.randint(0, 3, (1,), generator=g))]
        L = int(torch.randint(1, 400, (1,), generator=g))
        D = [64, 128][int(torch.randint(0, 2, (1,), generator=g))]
        H = P * int(torch.randint(1, 4, (1,), generator=g))
        S = P * L
        used = int(torch.randint(1, S + 1, (1,), generator=g))
        dtype = [torch.bfloat16, torch.float16][int(torch.randint(0, 2, (1,), generator=g))]
        out.append((P, L, H, D, used, dtype))
    return out


@pytest.mark.parametrize("P,L,H,D,used,dtype", _random_geometries(10))
def test_mfma_consumer_random_geometries(olib, P, L, H, D, used, dtype):
    """Seeded random world sizes, shard lengths, head counts, head dims, live prefixes and
    dtypes: every element of every destination and head within the FP8 bound."""
    w, d = grouped_inputs(small(B=1, P=P, L=L, H=H, D=D, dtype=dtype, used=used,
                                scale_sequence=used, seed=P * 1000 + L))
    vs = caller_v_scale(d, w) if dtype == torch.float16 else None
    g = run_group(w, to_dev(d, w.P), v_scale=None if vs is None else vs.to(DEV))
    _check_mfma_consumer(w, d, g, vs, range(w.P), lambda p: range(w.h), 32, w.name)
