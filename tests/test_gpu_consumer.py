"""The consumer check on the HIP path's outputs (GPU): attention read from the unpacked
tensors the way the Sage consumer reads them (oracle/consumer.py, float64 on the CPU),
against float64 attention on the original inputs, at the full workload shapes (sampled
heads and query rows), with and without a caller V scale.  Bounds and their rationale are
those of tests/test_oracle_consumer.py."""
from __future__ import annotations

import pytest
import torch

from precision_attention_input_amd import workloads as W

from gpu_helpers import DEV, run_group, say, to_dev
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
