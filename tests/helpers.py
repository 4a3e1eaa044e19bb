"""Shared test helpers: comparisons against the definition-level oracle."""
from __future__ import annotations

import torch

from precision_attention_input_amd import workloads as W

GROUP = 64


def small(B=1, P=2, L=128, H=None, D=64, dtype=torch.bfloat16, used=None, scale_sequence=None,
          aligned=None, seed=0, **kw) -> W.Workload:
    H = H or P
    name = f"b{B}_p{P}_l{L}_h{H}_d{D}_{'bf16' if dtype == torch.bfloat16 else 'fp16'}"
    return W.Workload(name, B=B, P=P, L=L, H=H, D=D, dtype=dtype, used=used,
                      scale_sequence=scale_sequence, aligned=aligned, seed=seed, **kw)


def first_group(r, L):
    return r * L // GROUP


def last_group(r, L):
    return (r * L + L - 1) // GROUP


def check_outputs_against_definition(outs: dict, df: dict, w: W.Workload):
    """outs[p] = (q8, k8, v8, q_scale, k_scale) of destination p (CPU tensors) against the
    definition: live groups bit-exact, V everywhere, zero V tail, finite extra scales."""
    S = w.S
    spad = (S + GROUP - 1) // GROUP * GROUP
    ns = w.scale_sequence or S
    Wd = (ns + GROUP - 1) // GROUP
    G, rows = df["G"], df["rows"]
    gg = min(G, Wd)
    for p, (q8, k8, v8, qs, ks) in outs.items():
        ref = df["per_dest"](p)
        assert q8.shape == (w.B, S, w.h, w.D) and k8.shape == q8.shape
        assert v8.shape == (w.B, w.D, w.h, spad)
        assert qs.shape == (w.B, w.h, Wd) and ks.shape == qs.shape
        assert torch.equal(qs[:, :, :gg], ref["q_scale"][:, :, :gg]), f"q_scale dest {p}"
        assert torch.equal(ks[:, :, :gg], ref["k_scale"][:, :, :gg]), f"k_scale dest {p}"
        assert torch.isfinite(qs).all() and torch.isfinite(ks).all()
        assert torch.equal(q8[:, :rows], ref["q8"]), f"q8 dest {p}"
        assert torch.equal(k8[:, :rows], ref["k8"]), f"k8 dest {p}"
        assert torch.equal(v8[..., :S], ref["v8"]), f"v8 dest {p}"
        assert (v8[..., S:] == 0).all(), f"v8 tail dest {p}"


def check_amax_against_definition(amax_per_rank, def_amax, w: W.Workload):
    """Every slot of a group with live rows equals the definition's group amax."""
    L = w.L
    for r, a in enumerate(amax_per_rank):
        g0, g1 = first_group(r, L), last_group(r, L)
        for g in range(g0, g1 + 1):
            if g < def_amax.shape[-1]:
                assert torch.equal(a[:, :, g - g0], def_amax[:, :, g]), (r, g)
