"""The two largest workloads against the CPU oracle, every byte of every head (GPU).

video_dit_aligned (B=1, world_size 8, L=4096, H=32, D=128, bf16) and long_unaligned (B=1,
world_size 8, L=9360, H=40, D=128, bf16, used 74000) are the only workloads large enough to
run the streaming instantiations of every kernel (non-temporal loads and stores, V in
workgroups of its own in the one-read pack, the unpack's streaming wave order).  The oracle
runs the whole group once per workload (its ranks and destinations on a thread pool), and
each entry point sequence is compared with it byte for byte: the boundary min/max, the
kernel and derived amax of every rank, every rank's chunks in the all-to-all buffer, and the
unpacked 5-tuple of every destination (unpack_for_sage Returns; k_grouped_amax Returns).
"""
from __future__ import annotations

import pytest
import torch

from oracle import pipeline
from precision_attention_input_amd import workloads as W

from gpu_helpers import (DEV, compare_all, run_group, run_group_one_read, run_per_rank,
                         run_per_rank_one_read, say, to_dev)
from helpers import oracle_threads

pytestmark = pytest.mark.gpu

MODES = ["group", "per_rank", "one_read_group", "one_read_per_rank", "v_scale_group",
         "v_scale_one_read_group", "v_scale_per_rank"]
RUNNERS = {
    "group": run_group, "per_rank": run_per_rank, "one_read_group": run_group_one_read,
    "one_read_per_rank": run_per_rank_one_read, "v_scale_group": run_group,
    "v_scale_one_read_group": run_group_one_read, "v_scale_per_rank": run_per_rank,
}
# every mode of one workload before the next: one workload's data and references in memory
CASES = [(wn, m) for wn in (W.VIDEO_DIT_ALIGNED.name, W.LONG_UNALIGNED.name) for m in MODES]

_CACHE: dict = {}


def _oracle(w, d, vs=None):
    return pipeline.run_group(d["Q"], d["K"], d["V"], d["mean"], world_size=w.P,
                              used_sequence=w.used, scale_sequence=w.scale_sequence,
                              v_scale=vs, threads=oracle_threads())


def workload(wname: str, v_scale: bool):
    """(w, data, device shards, V scale or None, the oracle's whole-group result), cached
    for one workload at a time."""
    if _CACHE.get("name") != wname:
        _CACHE.clear()
        torch.cuda.empty_cache()
        w = W.BY_NAME[wname]
        say(f"[large] generating {wname}")
        d = W.generate(w)
        say(f"[large] oracle {wname} ({oracle_threads()} threads)")
        _CACHE.update(name=wname, w=w, d=d, dd=to_dev(d, w.P), ref=_oracle(w, d))
    if v_scale and "ref_vs" not in _CACHE:
        w, d = _CACHE["w"], _CACHE["d"]
        vs = W.v_scale(w)
        say(f"[large] oracle {wname} with the caller's V scale")
        _CACHE.update(vs=vs, vs_dev=vs.to(DEV), ref_vs=_oracle(w, d, vs))
    c = _CACHE
    return (c["w"], c["dd"], c.get("vs_dev") if v_scale else None,
            c["ref_vs"] if v_scale else c["ref"])


@pytest.mark.parametrize("wname,mode", CASES, ids=[f"{w}-{m}" for w, m in CASES])
def test_large_workload_every_head(olib, wname, mode):
    vsc = mode.startswith("v_scale")
    w, dd, vs, ref = workload(wname, vsc)
    say(f"[large] {wname} {mode}")
    g = RUNNERS[mode](w, dd, aligned=w.aligned, v_scale=vs)
    compare_all(g, ref, w, f"{wname}/{mode}")
    del g
    torch.cuda.empty_cache()
    if (wname, mode) == CASES[-1]:
        _CACHE.clear()
