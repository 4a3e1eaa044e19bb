"""The one-read step (statistics and pack from one read of Q, K and V, then derive together
with the pack of the slots that waited for it) against the CPU oracle, bit for bit (GPU).

The oracle runs the step as the pages lay it out (grouped amax, boundary min/max, derive,
pack); the one-read entry points must reproduce every intermediate (kernel amax, min/max,
derived amax) and every chunk and output byte.  Every output buffer starts poisoned, so an
unwritten byte cannot pass.
"""
from __future__ import annotations

import pytest
import torch

import precision_attention_input_amd as ulp
from precision_attention_input_amd import workloads as W

from gpu_helpers import (DEV, assert_bits_equal, compare_all, run_group, run_group_one_read,
                         run_per_rank_one_read, say, to_dev)
from helpers import sign_pattern_columns, small
from test_gpu_parity import EDGE, RANDOM, oracle_run
from test_gpu_vscale import oracle_run as oracle_run_vs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wname", [W.TINY.name, W.UNALIGNED_PADDED.name,
                                   W.BATCHED_SMALL_HEAD.name])
@pytest.mark.parametrize("mode", ["group", "per_rank"])
def test_workload_one_read_parity(olib, wname, mode):
    w = W.BY_NAME[wname]
    say(f"[one-read] {wname} mode={mode}")
    d = W.generate(w)
    dd = to_dev(d, w.P)
    run = run_group_one_read if mode == "group" else run_per_rank_one_read
    compare_all(run(w, dd, w.aligned), oracle_run(w, d), w, f"{wname}/one-read/{mode}")


@pytest.mark.parametrize("w", EDGE, ids=[f"{w.name}_u{w.used}" for w in EDGE])
def test_edge_shapes_one_read(olib, w):
    say(f"[one-read edge] {w.name} used={w.used} ss={w.scale_sequence}")
    d = W.generate(w)
    dd = to_dev(d, w.P)
    ref = oracle_run(w, d)
    compare_all(run_group_one_read(w, dd), ref, w, "one-read group")
    compare_all(run_per_rank_one_read(w, dd), ref, w, "one-read per_rank")


@pytest.mark.parametrize("w", RANDOM, ids=[f"{w.name}_u{w.used}_s{w.scale_sequence}"
                                            for w in RANDOM])
def test_random_shapes_one_read(olib, w):
    say(f"[one-read random] {w.name} used={w.used} ss={w.scale_sequence}")
    d = W.generate(w)
    dd = to_dev(d, w.P)
    compare_all(run_group_one_read(w, dd), oracle_run(w, d), w, "one-read random")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [64, 128])
def test_sign_and_zero_patterns_one_read(olib, dtype, D):
    """The sign/zero channel patterns of the statistics test: the one-read amax and min/max
    (direct maxima of |x - mean| rather than order statistics) match bit for bit."""
    P, L, H, used = 4, 65, 4, 200
    S = P * L
    w = small(P=P, L=L, H=H, D=D, dtype=dtype, used=used, scale_sequence=used)
    say(f"[one-read sign patterns] {w.name}")
    d = dict(Q=sign_pattern_columns(S, H, D, used, dtype, 1),
             K=sign_pattern_columns(S, H, D, used, dtype, 2),
             V=sign_pattern_columns(S, H, D, used, dtype, 3))
    d["mean"] = W.k_mean_global(d["K"], used, dtype)
    dd = to_dev(d, P)
    ref = oracle_run(w, d)
    compare_all(run_group_one_read(w, dd), ref, w, "one-read group")
    compare_all(run_per_rank_one_read(w, dd), ref, w, "one-read per_rank")


@pytest.mark.parametrize("wname", [W.TINY.name, W.UNALIGNED_PADDED.name,
                                   W.BATCHED_SMALL_HEAD.name])
def test_v_scale_one_read(olib, wname):
    w = W.BY_NAME[wname]
    say(f"[one-read v_scale] {wname}")
    d = W.generate(w)
    vs = W.v_scale(w)
    dd = to_dev(d, w.P)
    vsd = vs.to(DEV)
    ref = oracle_run_vs(w, d, vs)
    compare_all(run_group_one_read(w, dd, w.aligned, v_scale=vsd), ref, w, "one-read v_scale")
    compare_all(run_per_rank_one_read(w, dd, w.aligned, v_scale=vsd), ref, w,
                "one-read per-rank v_scale")



def test_v_scale_one_read_streaming_launch(olib):
    """The long workload (its launch streams from HBM, so V goes through workgroups of its
    own) with the caller's V scale: every byte of the all-to-all buffer equals the separate
    pack's, which the V-scale tests check against the oracle."""
    w = W.LONG_UNALIGNED
    say(f"[one-read v_scale] {w.name}")
    d = W.generate(w)
    vsd = W.v_scale(w).to(DEV)
    dd = to_dev(d, w.P)
    f = run_group_one_read(w, dd, aligned=w.aligned, v_scale=vsd)
    g = run_group(w, dd, aligned=w.aligned, v_scale=vsd)
    assert_bits_equal(f["group"], g["group"], "all-to-all buffer")
    del dd, f, g
    torch.cuda.empty_cache()

def test_one_read_writes_nothing_outside(olib):
    """Outputs inside canary-filled buffers: nothing is written past them."""
    w = small(B=2, P=4, L=100, H=8, D=64, dtype=torch.float16, used=350, seed=8)
    d = W.generate(w)
    dd = to_dev(d, w.P)
    P, L, B, H, D = w.P, w.L, w.B, w.H, w.D
    sl = ulp.slots(L)
    cb = ulp.chunk_bytes(B, L, w.h, D)

    def guarded(shape, dtype):
        n = int(torch.tensor(shape).prod()) * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((n + 8192,), 0xA5, dtype=torch.uint8, device=DEV)
        return buf, buf[4096:4096 + n].view(dtype).view(shape)

    bufs = [guarded((P, B, H, sl), torch.float32), guarded((P, B, H, sl), torch.float32),
            guarded((P, B, H, 2, 2, D), torch.float32),
            guarded((P, B, H, 2, 2, D), torch.float32), guarded((P, P, cb), torch.uint8)]
    (qa, ka, qm, km), grp = ulp.group_stats_pack(
        dd["Q"], dd["K"], dd["V"], dd["mean"], world_size=P, used_sequence=w.used,
        out=tuple(b[1] for b in bufs[:4]), group=bufs[4][1])
    ulp.group_derive_pack(dd["Q"], dd["K"], dd["mean"], qa, ka, qm, km, world_size=P,
                          group=grp, used_sequence=w.used)
    torch.cuda.synchronize()
    for i, (buf, _) in enumerate(bufs):
        m = torch.cat([buf[:4096], buf[-4096:]])
        assert bool((m == 0xA5).all()), f"buffer {i}: write outside the output"
    ref = oracle_run(w, d)
    for r in range(P):
        assert_bits_equal(grp[:, r], ref["sends"][r], f"chunks of rank {r}")
        assert_bits_equal(ka[r], ref["k_amax"][r], f"k_amax r{r}")


def test_one_read_invalid_arguments(olib):
    w = small(P=2, L=100, H=2, D=64)
    d = W.generate(w)
    dd = to_dev(d, w.P)
    with pytest.raises(ValueError, match="used_sequence"):
        ulp.group_stats_pack(dd["Q"], dd["K"], dd["V"], dd["mean"], world_size=2,
                             used_sequence=201)
    with pytest.raises(ValueError, match="rank"):
        ulp.stats_pack(dd["Q"][0], dd["K"][0], dd["V"][0], dd["mean"], rank=2, world_size=2)
