"""64-bit addressing at a size past 2^31 elements per tensor (GPU).

Every input tensor here holds just over 2^31 elements (4 GiB of bf16 or fp16), the
all-to-all buffer 6.4 GB, so element offsets pass 2^31 and byte offsets pass 2^32 in the
statistics, derive, pack, unpack and K-mean kernels (their streaming instantiations, at
this size), at head_dim 64 and 128.  The oracle cannot
follow at this size, so the inputs are periodic: Q, K and V depend only on the global row
modulo 128, i.e. every even 64-row group holds the same values and so does every odd one.
A group's outputs (its scale and its codes) depend only on its own values and on the K
mean (k_grouped_amax and derive_k_boundary_amax pages, description; the boundary groups'
derived amax is the same maximum by the derive page's identity), so the unpacked outputs
must be the oracle's outputs for a small instance with the same period, tiled."""
from __future__ import annotations

import pytest
import torch

from oracle import pipeline
import precision_attention_input_amd as ulp

from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu

P, B, H = 2, 1, 2
PERIOD = 128
# (dtype, head_dim, local_sequence): P L H D = 2^31 + 8192 or + 16384 elements per tensor;
# S = P L is a multiple of 64 and the shards end mid-group
CASES = [(torch.bfloat16, 64, (1 << 23) + 32), (torch.float16, 128, (1 << 22) + 32)]


def _period(seed: int, DT, D):
    """One period of 128 rows of Q, K, V (two 64-row groups with different value ranges)
    and a K mean."""
    g = torch.Generator().manual_seed(seed)
    spread = torch.tensor([0.25] * 64 + [3.0] * 64).view(PERIOD, 1, 1)
    q = (torch.randn(PERIOD, H, D, generator=g) * spread).to(DT)
    mu = torch.randn(1, H, D, generator=g) * 4.0
    k = (mu + torch.randn(PERIOD, H, D, generator=g) * spread).to(DT)
    v = (torch.randn(PERIOD, H, D, generator=g) * spread * 2.0).to(DT)
    mean = mu.to(DT).view(B, H, D)
    return q, k, v, mean


def _expected(q, k, v, mean):
    """The oracle on a small instance with the same period (L = 160: shards end mid-group
    as in the large instance); its first 128 rows and two scale groups are one period."""
    Ls = 160
    rows = torch.arange(P * Ls) % PERIOD
    ref = pipeline.run_group(q[rows].unsqueeze(0), k[rows].unsqueeze(0),
                             v[rows].unsqueeze(0), mean, world_size=P)
    return {p: tuple(t for t in ref["outs"][p]) for p in range(P)}


def _check_tiled(outs, exp, label, S, D):
    """outs[p] = (q8, k8, v8, q_scale, k_scale) of the large instance on the GPU."""
    n = S // PERIOD
    for p in range(P):
        q8, k8, v8, qs, ks = outs[p]
        eq8, ek8, ev8, eqs, eks = (t.to(DEV) for t in exp[p])
        for name, big, small in (("q8", q8, eq8), ("k8", k8, ek8)):
            h = big.shape[2]
            full = big[:, :n * PERIOD].reshape(B, n, PERIOD, h, D)
            assert torch.equal(full.view(torch.uint8),
                               small[:, :PERIOD].unsqueeze(1).expand_as(full).view(torch.uint8)), \
                (label, name, p)
            rest = S - n * PERIOD
            assert torch.equal(big[:, n * PERIOD:].view(torch.uint8),
                               small[:, :rest].view(torch.uint8)), (label, name, p, "tail")
        h = v8.shape[2]
        fv = v8[..., :n * PERIOD].reshape(B, D, h, n, PERIOD)
        assert torch.equal(fv.view(torch.uint8),
                           ev8[..., :PERIOD].unsqueeze(3).expand_as(fv).view(torch.uint8)), \
            (label, "v8", p)
        assert torch.equal(v8[..., n * PERIOD:].view(torch.uint8),
                           ev8[..., :S - n * PERIOD].view(torch.uint8)), (label, "v8 tail", p)
        W = qs.shape[-1]
        assert W == S // 64
        idx = torch.arange(W, device=DEV) % 2
        for name, big, small in (("q_scale", qs, eqs), ("k_scale", ks, eks)):
            assert torch.equal(big.view(torch.int32), small[..., idx].view(torch.int32)), \
                (label, name, p)


@pytest.mark.parametrize("DT,D,L", CASES)
def test_offsets_past_4gib(olib, DT, D, L):
    S = P * L
    q, k, v, mean = _period(2024, DT, D)
    exp = _expected(q, k, v, mean)
    say(f"[large offsets] P={P} B={B} L={L} H={H} D={D}: "
        f"{P * B * L * H * D} elements per tensor")
    rows = torch.arange(S, device=DEV) % PERIOD
    Q = q.to(DEV)[rows].view(P, B, L, H, D)
    K = k.to(DEV)[rows].view(P, B, L, H, D)
    V = v.to(DEV)[rows].view(P, B, L, H, D)
    del rows
    md = mean.to(DEV)
    assert Q.numel() > 2 ** 31 and Q.numel() * Q.element_size() > 2 ** 32

    # the statistics, derive, pack and unpack one after another
    qa, ka, qm, km = ulp.group_stats(Q, K, md, world_size=P)
    ulp.group_derive(qa, ka, qm, km, md, local_sequence=L, world_size=P)
    grp = ulp.group_pack(Q, K, V, md, qa, ka, world_size=P)
    assert grp.numel() > 2 ** 32
    o = ulp.group_unpack(grp, batch_size=B, local_sequence=L, local_heads=H // P,
                         head_dim=D, world_size=P)
    torch.cuda.synchronize()
    _check_tiled({p: tuple(t[p] for t in o) for p in range(P)}, exp, "separate", S, D)

    # the one-read entry points into the same buffers, cleared first
    grp.fill_(0xA5)
    for t in o:
        t.view(torch.uint8).fill_(0xA5)
    (qa, ka, qm, km), grp = ulp.group_stats_pack(Q, K, V, md, world_size=P, group=grp)
    ulp.group_derive_pack(Q, K, md, qa, ka, qm, km, world_size=P, group=grp)
    o = ulp.group_unpack(grp, batch_size=B, local_sequence=L, local_heads=H // P,
                         head_dim=D, world_size=P, out=o)
    torch.cuda.synchronize()
    _check_tiled({p: tuple(t[p] for t in o) for p in range(P)}, exp, "one-read", S, D)

    # the K mean over every row: n whole periods and the first S - n 128 rows
    del grp, o
    n, rest = divmod(S, PERIOD)
    k64 = k.double()
    ref = (n * k64.sum(0) + k64[:rest].sum(0)) / S
    mf, _ = ulp.k_mean(K, world_size=P)
    torch.cuda.synchronize()
    got = mf.double().cpu().view(H, D)
    assert ((got - ref).abs() <= 1e-6 * ref.abs().clamp_min(1e-30)).all(), \
        float(((got - ref).abs() / ref.abs()).max())
