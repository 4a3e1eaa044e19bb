"""The K mean without a workspace argument (ulp_k_mean_noalloc), through the C ABI, against
ulp_k_mean with a caller workspace (GPU).

The no-allocation entry point runs the same kernels over the library's own device scratch
array, so its means must equal ulp_k_mean's bit for bit.  Calls follow one another on the
same GPU, each smaller than the one before it or reusing what an earlier call left in the
shared array, and every output starts poisoned.  Last, the use it exists for: the call
captured into a HIP graph and replayed on new inputs.
"""
from __future__ import annotations

import pytest
import torch

import precision_attention_input_amd as ulp
from precision_attention_input_amd import workloads as W

from gpu_helpers import DEV, assert_bits_equal, say
from helpers import small

pytestmark = pytest.mark.gpu


def _poisoned(B, H, D, dtype):
    return (torch.full((B, H, D), float("nan"), dtype=torch.float32, device=DEV),
            torch.full((B, H, D), float("nan"), dtype=dtype, device=DEV))


def _both(w: W.Workload, label: str):
    d = W.generate(w)
    Ks = W.stacked_shards(d["K"], w.P).to(DEV)
    del d
    P, B, L, H, D = Ks.shape
    got = ulp.k_mean_noalloc(Ks, world_size=P, used_sequence=w.used,
                             out=_poisoned(B, H, D, Ks.dtype))
    # the caller's workspace of the existing entry point starts as NaN patterns too
    need = int(ulp.lib().ulp_k_mean_workspace_bytes(B, L, H, D, P, ulp._none(w.used)))
    ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device=DEV)
    want = ulp.k_mean(Ks, world_size=P, used_sequence=w.used, workspace=ws,
                      out=_poisoned(B, H, D, Ks.dtype))
    torch.cuda.synchronize()
    assert_bits_equal(got[0], want[0], f"{label}: binary32 mean")
    assert_bits_equal(got[1], want[1], f"{label}: dtype mean")
    say(f"[no-alloc] {label}: {need} bytes of scratch, bit-exact")


def test_two_calls_in_a_row_second_smaller(olib):
    _both(W.LONG_UNALIGNED, "long_unaligned (scratch near its largest use here)")
    _both(W.UNALIGNED_PADDED, "unaligned_padded, second call, smaller")
    _both(small(B=1, P=2, L=100, H=4, D=64, used=150, seed=11), "tiny, third call, smaller")


@pytest.mark.parametrize("wname", [W.BATCHED_SMALL_HEAD.name, W.TINY.name,
                                   W.VIDEO_DIT_ALIGNED.name])
def test_workloads(olib, wname):
    _both(W.BY_NAME[wname], wname)


def test_edge_shapes(olib):
    for i, (P, L, H, D, used) in enumerate([(2, 1, 2, 64, None), (8, 3, 16, 64, 17),
                                            (6, 300, 6, 64, 1), (4, 517, 20, 128, 2068)]):
        dtype = (torch.bfloat16, torch.float16)[i % 2]
        _both(small(B=1 + i % 2, P=P, L=L, H=H, D=D, dtype=dtype, used=used, seed=40 + i),
              f"edge P={P} L={L} H={H} D={D} used={used}")


def test_k_mean_noalloc_in_a_graph(olib):
    w = small(B=2, P=4, L=300, H=8, D=128, dtype=torch.bfloat16, used=1100, seed=61)
    P, B, L, H, D = w.P, w.B, w.L, w.H, w.D
    inputs = []
    for seed in (61, 62, 63):
        d = W.generate(w.with_(seed=seed))
        inputs.append(W.stacked_shards(d["K"], P).to(DEV))
    K = torch.empty_like(inputs[0])
    out = (torch.empty(B, H, D, dtype=torch.float32, device=DEV),
           torch.empty(B, H, D, dtype=w.dtype, device=DEV))
    K.copy_(inputs[0])
    ulp.k_mean_noalloc(K, world_size=P, used_sequence=w.used, out=out)   # first call: lookup
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ulp.k_mean_noalloc(K, world_size=P, used_sequence=w.used, out=out)
    for i, src in enumerate(inputs * 2):
        K.copy_(src)
        out[0].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        want = ulp.k_mean(src, world_size=P, used_sequence=w.used)    # eager, own workspace
        torch.cuda.synchronize()
        assert_bits_equal(out[0], want[0], f"replay {i}: binary32 mean")
        assert_bits_equal(out[1], want[1], f"replay {i}: dtype mean")
        say(f"[no-alloc graph] replay {i}: bit-exact")
