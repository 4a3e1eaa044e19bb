"""Seeded synthetic inputs for the smooth-K low-precision Ulysses pack/unpack.

This module only draws input tensors; it holds none of the method's arithmetic.  Both the
GPU path's tests/benchmark and the CPU oracle consume the tensors it returns.

Recipe (per workload): a ``torch.Generator`` seeded with the workload's seed draws, in this
order and all in float32,

  1. Q [B,S,H,D]  (normal, or 0.5 * Student-t with 3 degrees of freedom built as
     Z / sqrt((Z1^2 + Z2^2 + Z3^2) / 3) from four standard normal tensors);
  2. mu [H,D]     the per-(head, channel) K mean, normal with std ``mu_std``;
  3. (outlier workloads only) ``randperm(H*D)[:n]`` picks n = round(frac*H*D) (head,
     channel) pairs, then n normals with std ``outlier_std`` replace their means;
  4. eps [B,S,H,D] the K deviation, normal with std ``eps_std``;
  5. V [B,S,H,D]  (same law as Q).

K = mu + eps in float32.  Each tensor is cast to the workload dtype by round-to-nearest-even
(``Tensor.to``).  Rows t >= used of Q, K and V are then set to zero (the caller contract of
zero-filled tail padding on the k_grouped_amax page, used_sequence parameter).

k_mean_global, which the pages take as an input already rounded to the dtype
(k_grouped_amax Parameters), is the float64 mean of the dtype-valued K over live rows
[0, used) per (b, h, d), rounded to float32 and then to the dtype.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    P: int              # Ulysses group size (world_size)
    L: int              # rows per source shard (local_sequence)
    H: int              # global heads
    D: int              # head_dim
    dtype: torch.dtype
    used: int | None    # used_sequence (None = all rows live)
    scale_sequence: int | None
    aligned: bool | None
    seed: int
    qv_law: str = "normal"          # "normal" | "student_t3_half"
    mu_std: float = 8.0
    eps_std: float = 0.1
    outlier_frac: float = 0.0
    outlier_std: float = 0.0

    @property
    def S(self) -> int:
        return self.P * self.L

    @property
    def h(self) -> int:
        return self.H // self.P

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the benchmark and the parity tests use.
TINY = Workload("tiny_b1_p2_l128_h4_d64_bf16", B=1, P=2, L=128, H=4, D=64,
                dtype=torch.bfloat16, used=None, scale_sequence=None, aligned=None, seed=0)
UNALIGNED_PADDED = Workload("unaligned_padded_b2_p4_l1000_h16_d128_fp16", B=2, P=4, L=1000,
                            H=16, D=128, dtype=torch.float16, used=3700, scale_sequence=3700,
                            aligned=None, seed=1)
VIDEO_DIT_ALIGNED = Workload("video_dit_aligned_b1_p8_l4096_h32_d128_bf16", B=1, P=8, L=4096,
                             H=32, D=128, dtype=torch.bfloat16, used=None, scale_sequence=None,
                             aligned=True, seed=2, mu_std=16.0, eps_std=0.05)
LONG_UNALIGNED = Workload("long_unaligned_b1_p8_l9360_h40_d128_bf16", B=1, P=8, L=9360, H=40,
                          D=128, dtype=torch.bfloat16, used=74000, scale_sequence=None,
                          aligned=None, seed=3)
BATCHED_SMALL_HEAD = Workload("batched_small_head_b4_p2_l2048_h24_d64_fp16", B=4, P=2, L=2048,
                              H=24, D=64, dtype=torch.float16, used=3500, scale_sequence=3500,
                              aligned=None, seed=4, qv_law="student_t3_half",
                              outlier_frac=0.01, outlier_std=64.0)

WORKLOADS = [TINY, UNALIGNED_PADDED, VIDEO_DIT_ALIGNED, LONG_UNALIGNED, BATCHED_SMALL_HEAD]
BY_NAME = {w.name: w for w in WORKLOADS}


def _qv(g: torch.Generator, shape, law: str) -> torch.Tensor:
    if law == "normal":
        return torch.randn(shape, generator=g)
    if law == "student_t3_half":
        z = torch.randn(shape, generator=g)
        chi = torch.zeros(shape)
        for _ in range(3):
            chi += torch.randn(shape, generator=g).square_()
        return z.div_(chi.div_(3.0).sqrt_()).mul_(0.5)
    raise ValueError(law)


def k_mean_global(K: torch.Tensor, used: int, dtype: torch.dtype) -> torch.Tensor:
    """float64 mean over rows [0, used) -> float32 -> dtype.  K: [B,S,H,D]."""
    B, S, H, D = K.shape
    acc = torch.zeros(B, H, D, dtype=torch.float64)
    step = 4096
    for t0 in range(0, used, step):
        acc += K[:, t0:min(used, t0 + step)].double().sum(dim=1)
    return (acc / used).float().to(dtype).contiguous()


def generate(w: Workload) -> dict:
    """-> dict(Q, K, V, mean): global CPU tensors [B,S,H,D] (dtype) and mean [B,H,D]."""
    g = torch.Generator().manual_seed(w.seed)
    shape = (w.B, w.S, w.H, w.D)
    used = w.used or w.S
    Q = _qv(g, shape, w.qv_law).to(w.dtype)
    mu = torch.randn(w.H, w.D, generator=g) * w.mu_std
    if w.outlier_frac > 0:
        n = round(w.outlier_frac * w.H * w.D)
        idx = torch.randperm(w.H * w.D, generator=g)[:n]
        mu.view(-1)[idx] = torch.randn(n, generator=g) * w.outlier_std
    K = torch.randn(shape, generator=g).mul_(w.eps_std).add_(mu).to(w.dtype)
    V = _qv(g, shape, w.qv_law).to(w.dtype)
    if used < w.S:
        Q[:, used:] = 0
        K[:, used:] = 0
        V[:, used:] = 0
    return dict(Q=Q, K=K, V=V, mean=k_mean_global(K, used, w.dtype))


def stacked_shards(X: torch.Tensor, P: int) -> torch.Tensor:
    """Global [B,S,H,D] -> [P,B,L,H,D] contiguous: shard r holds rows [r*L, (r+1)*L)."""
    B, S, H, D = X.shape
    return X.view(B, P, S // P, H, D).permute(1, 0, 2, 3, 4).contiguous()


def sample_heads(w: Workload, per_dest: int = 1, seed: int = 12345) -> list[int]:
    """A seeded choice of ``per_dest`` global heads inside each destination's head range,
    sorted; the sub-problem on these heads has H' = P * per_dest and h' = per_dest."""
    g = torch.Generator().manual_seed(seed)
    heads = []
    for p in range(w.P):
        pick = torch.randperm(w.h, generator=g)[:per_dest].sort().values
        heads += [p * w.h + int(j) for j in pick]
    return heads


def v_scale(w: Workload, seed: int | None = None) -> torch.Tensor:
    """A caller-held V scale [B,H,D] float32 (the pages leave its origin to the caller):
    2^u with u uniform in [-7, 2) drawn in float32 by a generator seeded with the workload's
    seed + 1000, so that mantissas are arbitrary and V / scale spans E4M3's subnormals,
    normals and saturation."""
    g = torch.Generator().manual_seed(w.seed + 1000 if seed is None else seed)
    u = torch.empty(w.B, w.H, w.D).uniform_(-7.0, 2.0, generator=g)
    return torch.exp2(u).contiguous()
