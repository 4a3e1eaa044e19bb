"""The streaming instantiations of every kernel on small shapes, against the oracle (GPU).

Each launcher picks between a cached and a streaming (non-temporal) instantiation from the
bytes a launch moves; only launches above the cache budget (the two largest workloads) take
the streaming one in the product build.  libulp_stream.so is the same sources built with a
budget of zero, so every launch of it streams: the statistics and K-mean passes with
non-temporal loads, the pack and the one-read pack with non-temporal stores (the one-read
pack converting V in workgroups of its own), and the unpack with streamed loads, its
second wave order and its other unroll.  Here it runs the edge shapes, the seeded random
geometries, the workloads that fit in seconds, the caller's V scale and the K mean, every
byte against the oracle.
"""
from __future__ import annotations

import os

import pytest
import torch

import precision_attention_input_amd as ulp
from precision_attention_input_amd import _build
from precision_attention_input_amd import workloads as W

from gpu_helpers import (DEV, compare_all, run_group, run_group_one_read, run_per_rank,
                         run_per_rank_one_read, say, to_dev)
from test_gpu_kmean import EDGE as KMEAN_EDGE, _check_with_mean, check as check_k_mean
from test_gpu_parity import EDGE, RANDOM, oracle_run
from test_gpu_vscale import oracle_run as oracle_run_vs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def streaming_library():
    """Route every call of the binding to the streaming build for this module's tests."""
    if not os.path.exists(_build.STREAM_LIB):
        pytest.fail(f"{_build.STREAM_LIB} is missing: build it first")
    ulp.load(_build.STREAM_LIB)
    try:
        yield
    finally:
        ulp.load(ulp.LIB_PATH)


def _all_modes(w, d, label):
    dd = to_dev(d, w.P)
    ref = oracle_run(w, d)
    for name, run in (("group", run_group), ("per_rank", run_per_rank),
                      ("one_read_group", run_group_one_read),
                      ("one_read_per_rank", run_per_rank_one_read)):
        compare_all(run(w, dd, w.aligned), ref, w, f"{label}/{name}")


@pytest.mark.parametrize("w", EDGE, ids=[f"{w.name}_u{w.used}" for w in EDGE])
def test_edge_shapes_streaming(olib, w):
    say(f"[stream edge] {w.name} used={w.used} ss={w.scale_sequence}")
    _all_modes(w, W.generate(w), "streaming edge")


@pytest.mark.parametrize("w", RANDOM[::2], ids=[f"{w.name}_u{w.used}_s{w.scale_sequence}"
                                                 for w in RANDOM[::2]])
def test_random_shapes_streaming(olib, w):
    say(f"[stream random] {w.name} used={w.used} ss={w.scale_sequence}")
    _all_modes(w, W.generate(w), "streaming random")


@pytest.mark.parametrize("wname", [W.TINY.name, W.UNALIGNED_PADDED.name,
                                   W.BATCHED_SMALL_HEAD.name])
def test_workloads_streaming(olib, wname):
    w = W.BY_NAME[wname]
    say(f"[stream] {wname}")
    _all_modes(w, W.generate(w), f"streaming {wname}")


@pytest.mark.parametrize("wname", [W.UNALIGNED_PADDED.name, W.BATCHED_SMALL_HEAD.name])
def test_v_scale_streaming(olib, wname):
    w = W.BY_NAME[wname]
    say(f"[stream v_scale] {wname}")
    d = W.generate(w)
    vs = W.v_scale(w)
    dd = to_dev(d, w.P)
    ref = oracle_run_vs(w, d, vs)
    for name, run in (("group", run_group), ("one_read_group", run_group_one_read),
                      ("per_rank", run_per_rank)):
        compare_all(run(w, dd, w.aligned, v_scale=vs.to(DEV)), ref, w,
                    f"streaming v_scale {wname}/{name}")


@pytest.mark.parametrize("w,used", KMEAN_EDGE, ids=[f"{w.name}_u{u}" for w, u in KMEAN_EDGE])
def test_k_mean_streaming(olib, w, used):
    say(f"[stream k_mean] {w.name} used={used}")
    d = W.generate(w)
    check_k_mean(W.stacked_shards(d["K"], w.P), used, f"streaming {w.name} used={used}")
    w = w.with_(used=used)
    d = W.generate(w)
    _check_with_mean(w, W.stacked_shards(d["K"], w.P).to(DEV),
                     W.stacked_shards(d["Q"], w.P).to(DEV), f"streaming {w.name} used={used}")
