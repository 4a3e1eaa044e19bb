"""GPU-side runners for the parity tests: the whole Ulysses group through libulp, by the
per-rank entry points and by the whole-group entry points, returned as CPU tensors laid out
like ``oracle.pipeline.run_group``'s result."""
from __future__ import annotations

import sys

import torch

import precision_attention_input_amd as ulp
from precision_attention_input_amd import workloads as W

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> torch.Tensor:
    """A byte view, so that comparisons are bit-exact (-0 != +0, NaN == NaN)."""
    t = t.contiguous()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    return t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int32 if t.element_size() == 4 else torch.int16)


def assert_bits_equal(a: torch.Tensor, b: torch.Tensor, what: str):
    a, b = a.cpu(), b.cpu()
    assert a.shape == b.shape, f"{what}: shape {tuple(a.shape)} vs {tuple(b.shape)}"
    ba, bb = bits(a), bits(b)
    if not torch.equal(ba, bb):
        bad = (ba != bb).nonzero()
        first = tuple(bad[0].tolist())
        raise AssertionError(f"{what}: {bad.shape[0]} mismatches, first at {first}: "
                             f"gpu={a[first].item()} oracle={b[first].item()}")


def to_dev(d: dict, P: int) -> dict:
    """Global host tensors -> stacked device shards [P,B,L,H,D] and the mean."""
    out = {n: W.stacked_shards(d[n], P).to(DEV) for n in ("Q", "K", "V")}
    out["mean"] = d["mean"].to(DEV)
    return out


def _poisoned_group(w: W.Workload) -> torch.Tensor:
    """An all-to-all buffer whose every byte starts as 0x5A, so that a byte the kernels
    leave unwritten cannot match the oracle by chance (torch.empty may hand back memory
    that still holds an earlier run's identical bytes)."""
    cb = ulp.chunk_bytes(w.B, w.L, w.h, w.D)
    return torch.full((w.P, w.P, cb), 0x5A, dtype=torch.uint8, device=DEV)


def _poisoned_stats(lead: tuple, w: W.Workload) -> tuple:
    f = dict(dtype=torch.float32, device=DEV)
    sl = ulp.slots(w.L)
    return (torch.full((*lead, w.B, w.H, sl), float("nan"), **f),
            torch.full((*lead, w.B, w.H, sl), float("nan"), **f),
            torch.full((*lead, w.B, w.H, 2, 2, w.D), float("nan"), **f),
            torch.full((*lead, w.B, w.H, 2, 2, w.D), float("nan"), **f))


def _poisoned_unpack(w: W.Workload, lead: tuple = ()) -> tuple:
    """Unpack outputs (q8, k8, v8, q_scale, k_scale) filled with 0x5A bytes / NaN."""
    qk, vs, sc = ulp.unpack_shapes(w.B, w.L, w.h, w.D, w.P, w.scale_sequence)
    i8 = dict(dtype=torch.int8, device=DEV)
    f = dict(dtype=torch.float32, device=DEV)
    return (torch.full((*lead, *qk), 0x5A, **i8), torch.full((*lead, *qk), 0x5A, **i8),
            torch.full((*lead, *vs), 0x5A, dtype=torch.uint8, device=DEV).view(
                torch.float8_e4m3fn),
            torch.full((*lead, *sc), float("nan"), **f), torch.full((*lead, *sc), float("nan"), **f))


def run_per_rank(w: W.Workload, dd: dict, aligned=None, v_scale=None) -> dict:
    """Every rank through the per-rank entry points; the all-to-all is the [P,P,cb] buffer.
    v_scale: optional [B,H,D] float32 device tensor (the caller's V divisor)."""
    P, L = w.P, w.L
    kw = dict(world_size=P, used_sequence=w.used)
    qs = [dd["Q"][r] for r in range(P)]
    ks = [dd["K"][r] for r in range(P)]
    vs = [dd["V"][r] for r in range(P)]
    # per-rank outputs of their own (a rank's slice of a stacked tensor need not be
    # 16-byte aligned), poisoned
    po = [_poisoned_stats((), w) for _ in range(P)]
    q_mm = torch.stack([ulp.boundary_minmax(qs[r], rank=r, out=po[r][2], **kw)
                        for r in range(P)])
    k_mm = torch.stack([ulp.boundary_minmax(ks[r], rank=r, out=po[r][3], **kw)
                        for r in range(P)])
    qa = [ulp.k_grouped_amax(qs[r], None, rank=r, out=po[r][0], **kw) for r in range(P)]
    ka = [ulp.k_grouped_amax(ks[r], dd["mean"], rank=r, out=po[r][1], **kw)
          for r in range(P)]
    qa_kernel = [a.clone() for a in qa]
    ka_kernel = [a.clone() for a in ka]
    for r in range(P):
        ulp.derive_k_boundary_amax(qa[r], q_mm, None, rank=r, local_sequence=L, world_size=P)
        ulp.derive_k_boundary_amax(ka[r], k_mm, dd["mean"], rank=r, local_sequence=L,
                                   world_size=P)
    grp = _poisoned_group(w)
    cb = grp.shape[-1]
    for r in range(P):
        ulp.pack(qs[r], ks[r], vs[r], dd["mean"], qa[r], ka[r], rank=r, world_size=P,
                 v_scale=v_scale, send=grp[0, r], dest_stride=P * cb)
    outs = {}
    for p in range(P):
        outs[p] = ulp.unpack_for_sage(grp[p], batch_size=w.B, local_sequence=L,
                                      local_heads=w.h, head_dim=w.D, world_size=P,
                                      aligned=aligned, scale_sequence=w.scale_sequence,
                                      out=_poisoned_unpack(w))
    torch.cuda.synchronize()
    return dict(q_minmax=q_mm, k_minmax=k_mm, q_amax_kernel=qa_kernel, k_amax_kernel=ka_kernel,
                q_amax=qa, k_amax=ka, group=grp,
                sends=[grp[:, r] for r in range(P)], outs=outs)


def run_group(w: W.Workload, dd: dict, aligned=None, v_scale=None) -> dict:
    """The whole group through the group entry points (the benchmark's launch sequence)."""
    P, L = w.P, w.L
    qa, ka, qm, km = ulp.group_stats(dd["Q"], dd["K"], dd["mean"], world_size=P,
                                     used_sequence=w.used, out=_poisoned_stats((P,), w))
    qa_kernel, ka_kernel = qa.clone(), ka.clone()
    ulp.group_derive(qa, ka, qm, km, dd["mean"], local_sequence=L, world_size=P)
    grp = ulp.group_pack(dd["Q"], dd["K"], dd["V"], dd["mean"], qa, ka, world_size=P,
                         v_scale=v_scale, group=_poisoned_group(w))
    o = ulp.group_unpack(grp, batch_size=w.B, local_sequence=L, local_heads=w.h, head_dim=w.D,
                         world_size=P, aligned=aligned, scale_sequence=w.scale_sequence,
                         out=_poisoned_unpack(w, (P,)))
    torch.cuda.synchronize()
    return dict(q_minmax=qm, k_minmax=km, q_amax_kernel=list(qa_kernel),
                k_amax_kernel=list(ka_kernel), q_amax=list(qa), k_amax=list(ka), group=grp,
                sends=[grp[:, r] for r in range(P)],
                outs={p: tuple(t[p] for t in o) for p in range(P)})


def compare_all(g: dict, ref: dict, w: W.Workload, label: str):
    """Bit-exact comparison of every intermediate and output with the oracle's."""
    P = w.P
    assert_bits_equal(g["q_minmax"], ref["q_minmax"], f"{label} q_minmax")
    assert_bits_equal(g["k_minmax"], ref["k_minmax"], f"{label} k_minmax")
    for r in range(P):
        assert_bits_equal(g["q_amax_kernel"][r], ref["q_amax_kernel"][r], f"{label} q_amax r{r}")
        assert_bits_equal(g["k_amax_kernel"][r], ref["k_amax_kernel"][r], f"{label} k_amax r{r}")
        assert_bits_equal(g["q_amax"][r], ref["q_amax"][r], f"{label} q_amax derived r{r}")
        assert_bits_equal(g["k_amax"][r], ref["k_amax"][r], f"{label} k_amax derived r{r}")
        if "sends" in ref:
            assert_bits_equal(g["sends"][r], ref["sends"][r], f"{label} chunks of rank {r}")
    for p in ref["outs"]:
        for i, name in enumerate(("q8", "k8", "v8", "q_scale", "k_scale")):
            assert_bits_equal(g["outs"][p][i], ref["outs"][p][i], f"{label} {name} dest {p}")


def run_group_one_read(w: W.Workload, dd: dict, aligned=None, v_scale=None) -> dict:
    """The whole group through the one-read entry points: group_stats_pack,
    group_derive_pack, group_unpack (outputs start poisoned)."""
    P, L = w.P, w.L
    (qa, ka, qm, km), grp = ulp.group_stats_pack(
        dd["Q"], dd["K"], dd["V"], dd["mean"], world_size=P, used_sequence=w.used,
        v_scale=v_scale, out=_poisoned_stats((P,), w), group=_poisoned_group(w))
    qa_kernel, ka_kernel = qa.clone(), ka.clone()
    ulp.group_derive_pack(dd["Q"], dd["K"], dd["mean"], qa, ka, qm, km, world_size=P,
                          group=grp, used_sequence=w.used)
    o = ulp.group_unpack(grp, batch_size=w.B, local_sequence=L, local_heads=w.h, head_dim=w.D,
                         world_size=P, aligned=aligned, scale_sequence=w.scale_sequence,
                         out=_poisoned_unpack(w, (P,)))
    torch.cuda.synchronize()
    return dict(q_minmax=qm, k_minmax=km, q_amax_kernel=list(qa_kernel),
                k_amax_kernel=list(ka_kernel), q_amax=list(qa), k_amax=list(ka), group=grp,
                sends=[grp[:, r] for r in range(P)],
                outs={p: tuple(t[p] for t in o) for p in range(P)})


def run_per_rank_one_read(w: W.Workload, dd: dict, aligned=None, v_scale=None) -> dict:
    """Every rank through stats_pack, then (after the min/max are gathered) derive_pack."""
    P, L = w.P, w.L
    kw = dict(world_size=P, used_sequence=w.used)
    grp = _poisoned_group(w)
    cb = grp.shape[-1]
    stats = []
    for r in range(P):
        st, _ = ulp.stats_pack(dd["Q"][r], dd["K"][r], dd["V"][r], dd["mean"], rank=r,
                               v_scale=v_scale, out=_poisoned_stats((), w), send=grp[0, r],
                               dest_stride=P * cb, **kw)
        stats.append(st)
    q_mm = torch.stack([s[2] for s in stats])
    k_mm = torch.stack([s[3] for s in stats])
    qa = [s[0] for s in stats]
    ka = [s[1] for s in stats]
    qa_kernel = [a.clone() for a in qa]
    ka_kernel = [a.clone() for a in ka]
    for r in range(P):
        ulp.derive_pack(dd["Q"][r], dd["K"][r], dd["mean"], qa[r], ka[r], q_mm, k_mm, rank=r,
                        send=grp[0, r], dest_stride=P * cb, **kw)
    outs = {}
    for p in range(P):
        outs[p] = ulp.unpack_for_sage(grp[p], batch_size=w.B, local_sequence=L,
                                      local_heads=w.h, head_dim=w.D, world_size=P,
                                      aligned=aligned, scale_sequence=w.scale_sequence,
                                      out=_poisoned_unpack(w))
    torch.cuda.synchronize()
    return dict(q_minmax=q_mm, k_minmax=k_mm, q_amax_kernel=qa_kernel, k_amax_kernel=ka_kernel,
                q_amax=qa, k_amax=ka, group=grp,
                sends=[grp[:, r] for r in range(P)], outs=outs)
