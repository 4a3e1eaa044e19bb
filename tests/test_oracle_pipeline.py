"""The per-rank C oracle against the global definition, and the invariants the pages state
(CPU only)."""
from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

import oracle
from oracle import brute, pipeline
from precision_attention_input_amd import workloads as W

from helpers import (check_amax_against_definition, check_outputs_against_definition,
                     first_group, last_group, small)

FLOOR32 = float(np.float32(1e-7))


def run(w: W.Workload, data=None):
    d = data or W.generate(w)
    res = pipeline.run_group(d["Q"], d["K"], d["V"], d["mean"], world_size=w.P,
                             used_sequence=w.used, scale_sequence=w.scale_sequence)
    df = brute.define(d["Q"], d["K"], d["V"], d["mean"], world_size=w.P,
                      used_sequence=w.used)
    return d, res, df


def _enumeration():
    Ps = [2, 4, 6, 8]
    Ls = [1, 2, 31, 63, 64, 65, 96, 100, 127, 128, 129, 200]
    cases = []
    for i, (P, L) in enumerate(itertools.product(Ps, Ls)):
        S = P * L
        B = 1 + (i % 2)
        D = (64, 128)[(i // 2) % 2]
        dtype = (torch.bfloat16, torch.float16)[(i // 4) % 2]
        H = P * (1 + (i // 3) % 2)
        rng = np.random.default_rng(i)
        useds = {None, 1, S, max(1, S - 1), min(S, 64 * (S // 128) + 1),
                 int(rng.integers(1, S + 1))}
        for used in sorted(useds, key=lambda u: -1 if u is None else u):
            ss = None if used is None else (used if i % 3 else None)
            cases.append(small(B=B, P=P, L=L, H=H, D=D, dtype=dtype, used=used,
                               scale_sequence=ss, seed=1000 + i))
    return cases


ENUM = _enumeration()


@pytest.mark.parametrize("w", ENUM, ids=[f"{w.name}_u{w.used}" for w in ENUM])
def test_pipeline_matches_definition(olib, w):
    d, res, df = run(w)
    check_outputs_against_definition(res["outs"], df, w)
    check_amax_against_definition(res["k_amax"], df["k_amax"], w)
    check_amax_against_definition(res["q_amax"], df["q_amax"], w)


def test_workload_mix_matches_definition(olib):
    """Heavy tails, outlier channels and fp16 as in the batched small-head workload."""
    w = W.BATCHED_SMALL_HEAD.with_(B=1, L=160, H=4, used=250, scale_sequence=250)
    d, res, df = run(w)
    check_outputs_against_definition(res["outs"], df, w)
    check_amax_against_definition(res["k_amax"], df["k_amax"], w)


# ------------------------------------------------------------------ invariants of the pages

def test_used_none_equals_used_s(olib):
    """k_grouped_amax description: used None or used == S leaves the result bit-identical."""
    w = small(P=4, L=100, H=4, D=128, dtype=torch.float16, seed=7)
    d = W.generate(w)
    for r, x in enumerate(pipeline.shards(d["K"], w.P)):
        a = oracle.k_grouped_amax(x, d["mean"], rank=r, world_size=w.P)
        b = oracle.k_grouped_amax(x, d["mean"], rank=r, world_size=w.P, used_sequence=w.S)
        assert torch.equal(a, b)


@pytest.mark.parametrize("used", [1, 63, 64, 65, 150, 195, 250, 399])
def test_only_partial_live_group_changes(olib, used):
    """k_grouped_amax description: with padding only slot (used-1)//64 differs from the
    unfixed kernel output, and it then equals the amax over its live rows only."""
    w = small(P=4, L=100, H=4, D=64, used=used, seed=11)
    d = W.generate(w)
    pl = (used - 1) // 64
    df = brute.define(d["Q"], d["K"], d["V"], d["mean"], world_size=w.P, used_sequence=used)
    for r, x in enumerate(pipeline.shards(d["K"], w.P)):
        unfixed = oracle.k_grouped_amax(x, d["mean"], rank=r, world_size=w.P)
        fixed = oracle.k_grouped_amax(x, d["mean"], rank=r, world_size=w.P, used_sequence=used)
        g0, g1 = first_group(r, w.L), last_group(r, w.L)
        for j in range(fixed.shape[-1]):
            if g0 + j != pl or g0 + j > g1:
                assert torch.equal(unfixed[..., j], fixed[..., j]), (r, j)
        if g0 <= pl <= g1:
            lo, hi = max(64 * pl, r * w.L), min(64 * pl + 64, r * w.L + w.L, used)
            if hi > lo:
                kc = brute.rn32_sub(x[:, lo - r * w.L:hi - r * w.L].float(),
                                    d["mean"].float()[:, None])
                want = torch.maximum(kc.abs().amax(dim=(1, 3)), torch.tensor(FLOOR32))
                assert torch.equal(fixed[..., pl - g0], want)
            else:   # this rank's slice of the partial group is padding only
                assert (fixed[..., pl - g0] == FLOOR32).all()


def test_padding_only_slice_contributes_floor(olib):
    """derive_k_boundary_amax description: sentinels (+inf, -inf) contribute exactly 1e-7.
    L=100, used=195: group 3 = rows [192,256) has live rows 192..194 on rank 1 only; rank 2's
    slice [200,256) is all padding."""
    w = small(P=4, L=100, H=4, D=64, used=195, seed=5)
    d = W.generate(w)
    ks = pipeline.shards(d["K"], w.P)
    mm = oracle.boundary_minmax(ks[2], rank=2, world_size=w.P, used_sequence=195)
    assert (mm[:, :, 0, 0] == float("inf")).all() and (mm[:, :, 0, 1] == float("-inf")).all()
    # a gather in which every toucher is padding only yields exactly the floor
    gathered = torch.stack([oracle.boundary_minmax(k, rank=r, world_size=w.P,
                                                   used_sequence=195)
                            for r, k in enumerate(ks)])
    gathered[1] = float("nan")   # rank 1 is a toucher of group 3: replace by sentinels
    gathered[1, :, :, :, 0] = float("inf")
    gathered[1, :, :, :, 1] = float("-inf")
    a = oracle.k_grouped_amax(ks[2], d["mean"], rank=2, world_size=w.P, used_sequence=195)
    oracle.derive_k_boundary_amax(a, gathered, d["mean"], rank=2, local_sequence=w.L,
                                  world_size=w.P)
    assert (a[..., 0] == FLOOR32).all()


def test_derive_bit_neutral_on_non_crossing_and_identical_on_touchers(olib):
    """derive_k_boundary_amax description: single-toucher live groups keep the kernel's
    partial; every toucher of a crossing group ends with the same bits."""
    w = small(P=4, L=100, H=8, D=128, dtype=torch.float16, used=370, seed=3)
    d, res, df = run(w)
    for r in range(w.P):
        for g in (first_group(r, w.L), last_group(r, w.L)):
            touchers = [r2 for r2 in range(w.P)
                        if r2 * w.L < 64 * g + 64 and 64 * g < r2 * w.L + w.L]
            vals = [res["k_amax"][r2][..., g - first_group(r2, w.L)] for r2 in touchers]
            for v in vals[1:]:
                assert torch.equal(v, vals[0]), (r, g)
            if len(touchers) == 1 and g <= (370 - 1) // 64:
                j = g - first_group(r, w.L)
                assert torch.equal(res["k_amax"][r][..., j], res["k_amax_kernel"][r][..., j])



def _waits_for_derive(r, L, S, used, j, n):
    """The slots the one-read pack leaves for after derive: a rank's first or last slot whose
    group another rank also touches or whose rows all lie in the zero tail."""
    if j not in (0, n - 1):
        return False
    g = first_group(r, L) + j
    lo, hi = max(64 * g, r * L), min(64 * g + 64, r * L + L)
    shared = 64 * g < r * L or min(64 * g + 64, S) > hi
    return shared or min(hi, used) <= lo


def test_derive_changes_only_slots_that_wait(olib):
    """The premise of packing from one read (statistics and pack in one pass, then derive
    and the pack of the waiting slots): on every enumerated shape, derive (derive page,
    description) leaves every slot outside the waiting set bit for bit as the grouped amax
    wrote it, for Q and for K; and the waiting set is not vacuous (derive does change some
    of its slots: crossing groups and boundary groups in the zero tail)."""
    changed_waiting = 0
    for w in ENUM[::3]:
        d, res, _ = run(w)
        S, used = w.S, w.used or w.S
        for r in range(w.P):
            n = last_group(r, w.L) - first_group(r, w.L) + 1
            for t in ("q", "k"):
                before, after = res[f"{t}_amax_kernel"][r], res[f"{t}_amax"][r]
                for j in range(before.shape[-1]):
                    same = torch.equal(before[..., j], after[..., j])
                    if j >= n or not _waits_for_derive(r, w.L, S, used, j, n):
                        assert same, (w.name, w.used, r, t, j)
                    elif not same:
                        changed_waiting += 1
    assert changed_waiting > 0

def test_scale_sequence_outputs_are_prefix_of_full_width(olib):
    """unpack_for_sage description: scales at scale_sequence are byte-identical to the
    leading slots of the full-width tensors; Q/K/V stay full length."""
    w = small(P=4, L=100, H=4, D=64, used=333, seed=9)
    d = W.generate(w)
    full = pipeline.run_group(d["Q"], d["K"], d["V"], d["mean"], world_size=w.P,
                              used_sequence=333, scale_sequence=None)
    for ns in (1, 64, 65, 333, 400):
        part = pipeline.run_group(d["Q"], d["K"], d["V"], d["mean"], world_size=w.P,
                                  used_sequence=333, scale_sequence=ns)
        Wn = (ns + 63) // 64
        for p in range(w.P):
            f, s = full["outs"][p], part["outs"][p]
            for i in range(3):
                assert torch.equal(f[i], s[i])
            assert torch.equal(s[3], f[3][..., :Wn]) and torch.equal(s[4], f[4][..., :Wn])


def test_group_size_invariance_of_outputs(olib):
    """Scales live on the global grid: the same global tensors give the same live bytes for
    world_size 2 and 4 once the destinations' heads are concatenated."""
    used = 301
    w2 = small(P=2, L=200, H=4, D=64, used=used, scale_sequence=used, seed=21)
    d = W.generate(w2)
    res2 = pipeline.run_group(d["Q"], d["K"], d["V"], d["mean"], world_size=2,
                              used_sequence=used, scale_sequence=used)
    res4 = pipeline.run_group(d["Q"], d["K"], d["V"], d["mean"], world_size=4,
                              used_sequence=used, scale_sequence=used)
    rows = 64 * ((used + 63) // 64)
    for i in range(5):
        a = torch.cat([res2["outs"][p][i] for p in range(2)], dim=2 if i < 3 else 1)
        b = torch.cat([res4["outs"][p][i] for p in range(4)], dim=2 if i < 3 else 1)
        if i < 2:
            a, b = a[:, :rows], b[:, :rows]
        assert torch.equal(a, b), i


# ------------------------------------------------------------------ hand-derived example

def test_hand_worked_example(olib):
    """A case small enough to do by hand.  fp16, B=1, world_size=2, L=96 (S=192: groups
    [0,64), [64,128), [128,192); group 1 crosses the shard boundary at row 96), H=2, D=64,
    used=150 (rows >= 150 zero; partial live group 2), mean 256 everywhere.

    Head 0 deviations from the mean (all others 0):
      group 0: row 10 d3 +63.5 (amax -> scale 63.5/127 = 0.5 exactly), row 20 d4 +0.25 ->
               0.5 -> 0 (tie to even), row 21 d4 +0.75 -> 1.5 -> 2, row 22 d5 -10.25 ->
               -20.5 -> -20.
      group 1: rank 0 rows 70/71/72 d0 +2.5/+3.5/-2.5 and row 80 d63 +100; rank 1 row 100
               d5 -127.  Rank 0's own partial is 100, rank 1's 127; derived: 127 on both,
               scale 1.0, so codes 2, 4, -2, 100, -127.
      group 2: row 130 d1 +31.75 (scale 31.75/127 = 0.25), row 131 d1 -0.125 -> -0.5 -> 0,
               row 132 d1 +0.375 -> 1.5 -> 2; padding rows hold K=0: (0-256)/0.25 clamps to
               -127.  Without the used fix the zero rows would give amax 256.
    Head 1: K = mean on live rows -> amax is the 1e-7 floor, codes 0, padding rows -127.
    Q head 0: row 1 d0 -127, row 2 d0 5.5 -> 6, row 3 d0 4.5 -> 4 (group 0 scale 1.0).
    V head 0 row 0 d0..5: 1.0, -2.0, 448, 500, 2^-9, 0 -> 0x38 0xC0 0x7E 0x7E 0x01 0x00.
    """
    B, P, L, H, D, used = 1, 2, 96, 2, 64, 150
    S = P * L
    f16 = torch.float16
    mean = torch.full((B, H, D), 256.0, dtype=f16)
    dev = torch.zeros(B, S, H, D)
    for (row, d, v) in [(10, 3, 63.5), (20, 4, 0.25), (21, 4, 0.75), (22, 5, -10.25),
                        (70, 0, 2.5), (71, 0, 3.5), (72, 0, -2.5), (80, 63, 100.0),
                        (100, 5, -127.0), (130, 1, 31.75), (131, 1, -0.125),
                        (132, 1, 0.375)]:
        dev[0, row, 0, d] = v
    K = (256.0 + dev).to(f16)
    Q = torch.zeros(B, S, H, D)
    Q[0, 1, 0, 0], Q[0, 2, 0, 0], Q[0, 3, 0, 0] = -127.0, 5.5, 4.5
    Q = Q.to(f16)
    V = torch.zeros(B, S, H, D)
    V[0, 0, 0, :6] = torch.tensor([1.0, -2.0, 448.0, 500.0, 2.0 ** -9, 0.0])
    V = V.to(f16)
    K[:, used:] = 0
    Q[:, used:] = 0
    V[:, used:] = 0

    res = pipeline.run_group(Q, K, V, mean, world_size=P, used_sequence=used)
    f = FLOOR32
    # kernel partials (before derive), head 0; slots(96) = 3, the third is never touched
    assert res["k_amax_kernel"][0][0, 0].tolist() == [63.5, 100.0, f]
    assert res["k_amax_kernel"][1][0, 0].tolist() == [127.0, 31.75, f]
    # after derive
    assert res["k_amax"][0][0, 0].tolist() == [63.5, 127.0, f]
    assert res["k_amax"][1][0, 0].tolist() == [127.0, 31.75, f]
    assert res["k_amax"][0][0, 1].tolist() == [f, f, f]
    # without the used fix the padded group would see |0 - 256|
    unfixed = oracle.k_grouped_amax(pipeline.shards(K, P)[1], mean, rank=1, world_size=P)
    assert unfixed[0, 0].tolist() == [127.0, 256.0, f]

    q8, k8, v8, qs, ks = res["outs"][0]          # destination 0 owns head 0
    assert ks[0, 0].tolist() == [0.5, 1.0, 0.25]
    assert qs[0, 0, 0].item() == 1.0
    expect_k = {(10, 3): 127, (20, 4): 0, (21, 4): 2, (22, 5): -20, (70, 0): 2, (71, 0): 4,
                (72, 0): -2, (80, 63): 100, (100, 5): -127, (130, 1): 127, (131, 1): 0,
                (132, 1): 2}
    for (row, d), code in expect_k.items():
        assert k8[0, row, 0, d].item() == code, (row, d)
    assert (k8[0, used:, 0] == -127).all()
    mask = torch.ones(S, D, dtype=torch.bool)
    for (row, d) in expect_k:
        mask[row, d] = False
    mask[used:] = False
    assert (k8[0, :, 0][mask] == 0).all()
    assert [q8[0, r, 0, 0].item() for r in (1, 2, 3)] == [-127, 6, 4]
    assert v8[0, :6, 0, 0].tolist() == [0x38, 0xC0, 0x7E, 0x7E, 0x01, 0x00]

    q8, k8, v8, qs, ks = res["outs"][1]          # destination 1 owns head 1
    assert ks[0, 0].tolist() == [float(np.float32(f) / np.float32(127))] * 3
    assert (k8[0, :used] == 0).all() and (k8[0, used:] == -127).all()


# ------------------------------------------------------------------ signed zeros in min/max

def _bits(x: float) -> int:
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_boundary_minmax_signed_zeros(olib, dtype):
    """The gathered min/max (derive_k_boundary_amax, gathered_minmax parameter) fixes only a
    shape; the reading taken is that -0 counts as +0 before the min and max, so each entry
    has one bit pattern whatever the row order.  B=1, world_size=2, L=96: rank 0's last
    group is [64,128), its rows 64..95 (the crossing group); rank 1's first group is the
    same group, rows 96..127.  Every other value is 1.0.  Hand-worked expectations, per
    channel of head 0 in that group (rank 0 rows 64..95):
      d0: only -0                    -> min +0, max +0
      d1: -0 and +0 alternating      -> min +0, max +0
      d2: -0 with -3.0 and -0.5      -> min -3.0, max +0
      d3: -0 with +2.0 and +0.25     -> min +0, max +2.0
      d4: -0 only on rank 1's rows   -> rank 1's first entry: min +0, max +0
    used_sequence = 100 also makes rank 1's rows >= 100 zero padding (not min/max rows)."""
    B, P, L, H, D, used = 1, 2, 96, 2, 64, 100
    S = P * L
    X = torch.ones(B, S, H, D)
    X[:, used:] = 0.0
    rows0 = torch.arange(64, 96)
    X[0, rows0, 0, 0] = -0.0
    X[0, rows0, 0, 1] = torch.where(rows0 % 2 == 0, torch.tensor(-0.0), torch.tensor(0.0))
    X[0, rows0, 0, 2] = -0.0
    X[0, 70, 0, 2], X[0, 90, 0, 2] = -3.0, -0.5
    X[0, rows0, 0, 3] = -0.0
    X[0, 71, 0, 3], X[0, 91, 0, 3] = 2.0, 0.25
    X[0, 96:used, 0, 4] = -0.0
    X = X.to(dtype)
    assert torch.signbit(X[0, 64, 0, 0].float()).item()        # the -0 survives the cast
    sh = pipeline.shards(X, P)
    mm0 = oracle.boundary_minmax(sh[0], rank=0, world_size=P, used_sequence=used)
    mm1 = oracle.boundary_minmax(sh[1], rank=1, world_size=P, used_sequence=used)
    POS0, NEG3, TWO = _bits(0.0), _bits(-3.0), _bits(2.0)
    # [b, h, e, s, d]: e = 1 is rank 0's last group, e = 0 is rank 1's first group
    expect0 = {0: (POS0, POS0), 1: (POS0, POS0), 2: (NEG3, POS0), 3: (POS0, TWO)}
    for d, (mn, mx) in expect0.items():
        assert _bits(mm0[0, 0, 1, 0, d].item()) == mn, f"rank 0 min d{d}"
        assert _bits(mm0[0, 0, 1, 1, d].item()) == mx, f"rank 0 max d{d}"
    assert _bits(mm1[0, 0, 0, 0, 4].item()) == POS0
    assert _bits(mm1[0, 0, 0, 1, 4].item()) == POS0
    # no entry anywhere holds the pattern of -0
    for mm in (mm0, mm1):
        assert not (mm.view(torch.int32) == _bits(-0.0) - 2 ** 32).any()


def test_threaded_group_run_equals_sequential(olib):
    """The parity tests run the oracle's independent per-rank and per-destination calls on a
    thread pool; every intermediate and output must be the same bytes as the one-thread
    run (the C calls share no state)."""
    w = small(B=2, P=8, L=100, H=16, D=64, dtype=torch.float16, used=700, scale_sequence=650,
              seed=31)
    d = W.generate(w)
    kw = dict(world_size=w.P, used_sequence=w.used, scale_sequence=w.scale_sequence)
    one = pipeline.run_group(d["Q"], d["K"], d["V"], d["mean"], threads=1, **kw)
    many = pipeline.run_group(d["Q"], d["K"], d["V"], d["mean"], threads=8, **kw)
    for key in ("q_minmax", "k_minmax"):
        assert torch.equal(one[key].view(torch.int32), many[key].view(torch.int32)), key
    for key in ("q_amax_kernel", "k_amax_kernel", "q_amax", "k_amax", "sends"):
        for a, b in zip(one[key], many[key]):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.uint8 else
                               a.view(torch.int32), b.view(torch.uint8) if
                               b.dtype == torch.uint8 else b.view(torch.int32)), key
    for p in range(w.P):
        for a, b in zip(one["outs"][p], many["outs"][p]):
            assert torch.equal(a.view(torch.uint8) if a.element_size() == 1 else
                               a.view(torch.int32), b.view(torch.uint8) if
                               b.element_size() == 1 else b.view(torch.int32)), p
