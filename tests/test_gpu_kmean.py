"""The global K mean on the GPU (ulp_k_mean) against the oracle's (GPU).

The pages take k_mean_global as an input rounded to the dtype (k_grouped_amax and
derive_k_boundary_amax, Parameters); the library also forms it, from the stacked shards.
The binary32 mean is held to a relative 1e-6 of the oracle's: on the five workloads
plainly, |mean_gpu - mean_oracle| <= 1e-6 |mean_oracle| for every channel; on constructed
shapes, whose channel means can sit near zero, against max(|mean|, mean |K|) of the
channel, so that such a channel is held to its own scale.  The dtype mean must be the
round-to-nearest-even of the GPU's binary32 mean.  Where every partial sum is exact (inputs on a bounded dyadic grid) the
result does not depend on the summation order, and there GPU and oracle agree bit for bit.
"""
from __future__ import annotations

import pytest
import torch

import oracle
from oracle import pipeline
import precision_attention_input_amd as ulp
from precision_attention_input_amd import workloads as W

from gpu_helpers import DEV, assert_bits_equal, say
from helpers import oracle_threads, sign_pattern_columns, small

pytestmark = pytest.mark.gpu

REL = 1e-6


def channel_scale(Ks: torch.Tensor, used: int) -> torch.Tensor:
    """mean |K| over the live rows per (b, h, d) of stacked shards [P,B,L,H,D]."""
    P, B, L, H, D = Ks.shape
    acc = torch.zeros(B, H, D, dtype=torch.float64)
    for r in range(P):
        n = max(0, min(L, used - r * L))
        if n:
            acc += Ks[r, :, :n].double().abs().sum(dim=1)
    return (acc / used).float()


def check(Ks: torch.Tensor, used, tag: str, exact: bool = False, plain: bool = False):
    """plain: the tolerance is 1e-6 of |mean| itself (the workloads); otherwise of
    max(|mean|, mean |K|) per channel (constructed shapes)."""
    P, B, L, H, D = Ks.shape
    u = used or P * L
    ref_f, ref_d = oracle.k_mean(Ks, used_sequence=used)
    mf, md = ulp.k_mean(Ks.to(DEV), world_size=P, used_sequence=used)
    torch.cuda.synchronize()
    mf, md = mf.cpu(), md.cpu()
    tol = REL * (ref_f.abs() if plain else torch.maximum(ref_f.abs(), channel_scale(Ks, u)))
    err = (mf.double() - ref_f.double()).abs()
    same = int((mf.view(torch.int32) == ref_f.view(torch.int32)).sum())
    say(f"[k_mean] {tag}: max err / tol {float((err / tol.double().clamp_min(1e-300)).max()):.3g}"
        f", {same}/{mf.numel()} binary32 values bit-exact")
    assert bool((err <= tol.double()).all()), f"{tag}: mean outside the 1e-6 tolerance"
    assert_bits_equal(md, mf.to(Ks.dtype), f"{tag}: dtype mean = RNE(binary32 mean)")
    if exact:
        assert_bits_equal(mf, ref_f, f"{tag}: binary32 mean")
        assert_bits_equal(md, ref_d, f"{tag}: dtype mean")
    return mf, md


@pytest.mark.parametrize("wname", [W.TINY.name, W.UNALIGNED_PADDED.name,
                                   W.BATCHED_SMALL_HEAD.name])
def test_workload_k_mean(olib, wname):
    w = W.BY_NAME[wname]
    d = W.generate(w)
    Ks = W.stacked_shards(d["K"], w.P)
    _, md = check(Ks, w.used, wname, plain=True)
    # the workload recipe's mean (the input every other parity test uses)
    diff = int((md.view(torch.int16) != d["mean"].view(torch.int16)).sum())
    say(f"[k_mean] {wname}: {diff} dtype values differ from the recipe's")


@pytest.mark.parametrize("wname", [W.VIDEO_DIT_ALIGNED.name, W.LONG_UNALIGNED.name])
def test_large_workload_k_mean(olib, wname):
    """Full-size shapes, every channel against the oracle's mean (plain 1e-6 relative
    bound), and the recipe's torch binary64 sum at the same bound."""
    w = W.BY_NAME[wname]
    say(f"[k_mean] generating {wname}")
    d = W.generate(w)
    Ks = W.stacked_shards(d["K"], w.P)
    del d["Q"], d["V"]
    mf, md = check(Ks, w.used, wname, plain=True)
    u = w.used or w.S
    acc = torch.zeros(w.B, w.H, w.D, dtype=torch.float64)
    for t0 in range(0, u, 4096):
        acc += d["K"][:, t0:min(u, t0 + 4096)].double().sum(dim=1)
    ref = (acc / u).float()
    assert bool(((mf.double() - ref.double()).abs() <= REL * ref.abs().double()).all())
    diff = int((md.view(torch.int16) != d["mean"].view(torch.int16)).sum())
    say(f"[k_mean] {wname}: {diff} of {md.numel()} dtype values differ from the recipe's")


def _edge():
    out = []
    for i, (P, L, H, D, used) in enumerate([
            (2, 1, 2, 64, None), (8, 1, 8, 128, 5), (2, 3, 2, 64, 6), (8, 3, 16, 64, 17),
            (4, 100, 4, 128, 257), (2, 128, 2, 64, 256), (2, 129, 4, 128, None),
            (6, 300, 6, 64, 1), (8, 1000, 24, 128, 7999), (2, 1000, 40, 128, 1999),
            (4, 517, 20, 128, 2068), (2, 2048, 34, 64, 4095)]):
        dtype = (torch.bfloat16, torch.float16)[i % 2]
        out.append((small(B=1 + i % 3, P=P, L=L, H=H, D=D, dtype=dtype, used=used,
                          seed=900 + i), used))
    return out


EDGE = _edge()


@pytest.mark.parametrize("w,used", EDGE, ids=[f"{w.name}_u{u}" for w, u in EDGE])
def test_edge_shapes_k_mean(olib, w, used):
    """Ragged column blocks (H*D not a multiple of 2048), row chunks that end mid-shard,
    shards shorter than the 8-row load batch, one live row, B > 1."""
    d = W.generate(w)
    check(W.stacked_shards(d["K"], w.P), used, f"{w.name} used={used}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_exact_sums_bit_exact_and_deterministic(olib, dtype):
    """Inputs k * 2^-6 with integer |k| < 256 around a per-channel offset: exact in both
    dtypes, and every partial sum is an exact binary64 value, so any summation order gives
    the oracle's result.  Rows past used hold nonzero values that must be ignored.  The
    workspace starts as garbage; a second call gives the same bits."""
    g = torch.Generator().manual_seed(77)
    P, B, L, H, D = 4, 2, 700, 8, 128
    base = torch.randint(-200, 201, (H, D), generator=g)
    k = base + torch.randint(-50, 51, (P, B, L, H, D), generator=g)
    Ks = (k.double() * 2.0 ** -6).to(dtype)
    assert torch.equal(Ks.double(), k.double() * 2.0 ** -6)   # exactly representable
    used = 2500
    mf1, md1 = check(Ks, used, f"exact {dtype}", exact=True)
    need = ulp.lib().ulp_k_mean_workspace_bytes(B, L, H, D, P, used)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)      # NaN patterns
    mf2, md2 = ulp.k_mean(Ks.to(DEV), world_size=P, used_sequence=used, workspace=ws)
    assert_bits_equal(mf2, mf1, "second call, binary32")
    assert_bits_equal(md2, md1, "second call, dtype")


def test_k_mean_feeds_the_pipeline(olib):
    """The GPU mean is a valid k_mean_global: the group pipeline run with it gives the
    oracle's bytes for the same mean."""
    from gpu_helpers import compare_all, run_group, to_dev
    from oracle import pipeline
    w = W.UNALIGNED_PADDED
    d = W.generate(w)
    dd = to_dev(d, w.P)
    _, md = ulp.k_mean(dd["K"], world_size=w.P, used_sequence=w.used)
    dd["mean"] = md
    d["mean"] = md.cpu()
    ref = pipeline.run_group(d["Q"], d["K"], d["V"], d["mean"], world_size=w.P,
                             used_sequence=w.used, scale_sequence=w.scale_sequence)
    compare_all(run_group(w, dd), ref, w, "pipeline with the GPU mean")


# ----------------------------------------------------------------- statistics with the mean

def _check_with_mean(w, Ks_dev, Qs_dev, label, plain=False):
    """group_stats_with_mean against (a) the oracle's mean within its tolerance (plain:
    1e-6 of |mean|, else of max(|mean|, mean |K|)), (b) the oracle's statistics of every
    rank, Q and K, run with the GPU's dtype mean, bit for bit, and (c) ulp_group_stats fed
    the same mean."""
    P = w.P
    qa, ka, qm, km, mf, md = ulp.group_stats_with_mean(Qs_dev, Ks_dev, world_size=P,
                                                       used_sequence=w.used)
    ra = ulp.group_stats(Qs_dev, Ks_dev, md, world_size=P, used_sequence=w.used)
    torch.cuda.synchronize()
    for got, ref, name in zip((qa, ka, qm, km), ra, ("q_amax", "k_amax", "q_minmax",
                                                     "k_minmax")):
        assert_bits_equal(got, ref, f"{label}: {name} vs group_stats with the same mean")
    Ks = Ks_dev.cpu()
    of, _ = oracle.k_mean(Ks, used_sequence=w.used)
    tol = REL * (of.abs() if plain else torch.maximum(of.abs(), channel_scale(Ks, w.used or w.S)))
    assert bool(((mf.cpu().double() - of.double()).abs() <= tol.double()).all()), label
    assert_bits_equal(md, mf.cpu().to(Ks.dtype), f"{label}: dtype mean = RNE(fp32 mean)")
    Qs = Qs_dev.cpu()
    oqm, okm, oqa, oka = pipeline.run_stats(list(Qs), list(Ks), md.cpu(), world_size=P,
                                            used_sequence=w.used, threads=oracle_threads())
    assert_bits_equal(qm, oqm, f"{label} q_minmax")
    assert_bits_equal(km, okm, f"{label} k_minmax")
    for r in range(P):
        assert_bits_equal(qa[r], oqa[r], f"{label} q_amax r{r}")
        assert_bits_equal(ka[r], oka[r], f"{label} k_amax r{r}")
    say(f"[stats+mean] {label}: ok")


@pytest.mark.parametrize("wname", [w.name for w in W.WORKLOADS])
def test_stats_with_mean_workloads(olib, wname):
    w = W.BY_NAME[wname]
    d = W.generate(w)
    Ks = W.stacked_shards(d["K"], w.P).to(DEV)
    Qs = W.stacked_shards(d["Q"], w.P).to(DEV)
    del d
    _check_with_mean(w, Ks, Qs, wname, plain=True)


@pytest.mark.parametrize("w,used", EDGE, ids=[f"{w.name}_u{u}" for w, u in EDGE])
def test_stats_with_mean_edges(olib, w, used):
    w = w.with_(used=used)
    d = W.generate(w)
    _check_with_mean(w, W.stacked_shards(d["K"], w.P).to(DEV),
                     W.stacked_shards(d["Q"], w.P).to(DEV), f"{w.name} used={used}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [64, 128])
def test_stats_with_mean_sign_and_zero_patterns(olib, dtype, D):
    """Channels of all -0, mixed zeros, one sign, +-max and subnormals (the raw 16-bit
    ordering of the one-read pass), 65-row shards and a live prefix ending mid-group."""
    P, L, H, used = 4, 65, 4, 200
    w = small(P=P, L=L, H=H, D=D, dtype=dtype, used=used)
    K = sign_pattern_columns(P * L, H, D, used, dtype, 2)
    Q = sign_pattern_columns(P * L, H, D, used, dtype, 1)
    _check_with_mean(w, W.stacked_shards(K, P).to(DEV), W.stacked_shards(Q, P).to(DEV),
                     f"sign patterns {w.name}")

