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


def sign_pattern_columns(S, H, D, used, dtype, seed):
    """[1, S, H, D] values whose channels (per head) cycle through the sign and zero
    patterns that order statistics on raw 16-bit patterns must get right; rows >= used
    are +0 (the zero tail)."""
    g = torch.Generator().manual_seed(seed)
    fi = torch.finfo(dtype)
    x = torch.empty(S, H, D, dtype=torch.float64)
    rows = torch.arange(S, dtype=torch.float64)[:, None]
    mag = 1.0 + torch.rand(S, H, dtype=torch.float64, generator=g)
    for c in range(D):
        kind = c % 10
        r = mag * (1 + c / D)
        if kind == 0:
            col = torch.full((S, H), -0.0, dtype=torch.float64)
        elif kind == 1:
            col = torch.where(rows % 2 == 0, -0.0, 0.0).expand(S, H).clone()
        elif kind == 2:
            col = -r
        elif kind == 3:
            col = r
        elif kind == 4:
            col = torch.where(rows % 3 == 0, -0.0, -r)
        elif kind == 5:
            col = torch.where(rows % 3 == 0, -0.0, r)
        elif kind == 6:
            col = torch.where(rows % 2 == 0, -fi.max, fi.max).expand(S, H).clone()
        elif kind == 7:
            col = -fi.smallest_normal * (rows % 7 + 1).expand(S, H) / 8
        elif kind == 8:
            col = torch.where(rows % 4 == 0, -0.0, fi.smallest_normal * (rows % 5) / 8).expand(S, H).clone()
        else:
            col = torch.randn(S, H, dtype=torch.float64, generator=g)
        x[:, :, c] = col
    x[used:] = 0.0
    return x.to(dtype).unsqueeze(0).contiguous()


def oracle_threads() -> int:
    """Threads for running the oracle's independent per-rank calls side by side: the cores
    this process may use, at most 16."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))
