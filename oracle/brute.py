"""Definition-level oracle on the unsharded global tensors.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Shares no code with ``oracle.c``
or with the GPU path.

What the method computes, stated without ranks, slots or chunks (FlashInfer pages
flashinfer.comm._ulysses_lowp.k_grouped_amax, derive_k_boundary_amax and unpack_for_sage):

* the global sequence of S rows is cut into 64-row groups;
* for every group with at least one live row (row < used), the Q amax is the max of |Q|
  and the K amax the max of |RN(K - mean)| over the live rows of the group and all
  channels, floored at 1e-7 (k_grouped_amax description; derive_k_boundary_amax
  description shows the cross-shard result equals this direct amax);
* scale = amax / 127, and every row of the group is quantized to
  clamp(rint(x / scale), -127, 127);
* V is converted to FP8 E4M3 on every row (unpack_for_sage Returns);
* destination p receives heads [p*h, (p+1)*h).

Every binary32 operation (subtraction, division) is evaluated here in binary64 and rounded
once to binary32.  For +, -, x, / of binary32 operands this gives exactly the correctly
rounded binary32 result, because binary64 carries more than 2*24+2 significand bits
(Figueroa, "When is double rounding innocuous?", SIGNUM 1995), so the result does not
depend on how torch vectorizes float32 arithmetic.
"""
from __future__ import annotations

import torch

GROUP = 64
FLOOR = torch.tensor(1e-7, dtype=torch.float32)   # binary32 nearest to 1e-7


def rn32_sub(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """Correctly rounded binary32 a - b (a, b hold binary32 values)."""
    return (a.double() - b.double()).float()


def rn32_div(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """Correctly rounded binary32 a / b."""
    return (a.double() / b.double()).float()


def group_amax(x: torch.Tensor, used: int) -> torch.Tensor:
    """x: [B,S,H,D] float32 magnitudes source.  -> [B,H,G] with G = ceil(used/64):
    max of |x| over the live rows of each group and all channels, floored at 1e-7."""
    B, S, H, D = x.shape
    G = (used + GROUP - 1) // GROUP
    a = x[:, :used].abs()
    pad = G * GROUP - used
    if pad:
        a = torch.cat([a, torch.full((B, pad, H, D), float("-inf"))], dim=1)
    a = a.reshape(B, G, GROUP, H, D).amax(dim=(2, 4))          # [B,G,H]
    return torch.maximum(a, FLOOR).permute(0, 2, 1).contiguous()  # [B,H,G]


def quantize_rows(x: torch.Tensor, scale: torch.Tensor, rows: int) -> torch.Tensor:
    """x: [B,S,H,D] float32; scale: [B,H,G]; quantize rows [0, rows) with the scale of their
    group.  -> int8 [B,rows,H,D]."""
    g = torch.arange(rows) // GROUP
    s = scale[:, :, g].permute(0, 2, 1).unsqueeze(-1)           # [B,rows,H,1]
    qf = rn32_div(x[:, :rows], s.expand(-1, -1, -1, x.shape[-1]))
    return qf.round().clamp(-127, 127).to(torch.int8)           # round: half to even


def e4m3_bytes(v: torch.Tensor) -> torch.Tensor:
    """float32 -> OCP E4M3FN bytes, round to nearest even, saturating at +-448."""
    return v.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def define(Q, K, V, mean, *, world_size, used_sequence=None, v_scale=None):
    """Q, K, V: global [B,S,H,D] bf16/fp16; mean: [B,H,D] same dtype; v_scale: optional
    [B,H,D] float32 divisor of V (the caller's V scale, unpack_for_sage Returns).

    Returns a dict with, for the live groups g < ceil(used/64):
      q_amax, k_amax   [B,H,G] fp32
      q_scale, k_scale [B,H,G] fp32
      q8, k8           [B,64*G capped at S,H,D] int8
      v8               [B,S,H,D] uint8 (E4M3) for all rows
    and ``per_dest(p)`` giving destination p's head slice of each in the unpack layouts.
    """
    B, S, H, D = Q.shape
    used = used_sequence or S
    G = (used + GROUP - 1) // GROUP
    rows = min(S, G * GROUP)
    xq = Q.float()
    xk = rn32_sub(K.float(), mean.float()[:, None])
    q_amax = group_amax(xq, used)
    k_amax = group_amax(xk, used)
    q_scale = rn32_div(q_amax, torch.full_like(q_amax, 127.0))
    k_scale = rn32_div(k_amax, torch.full_like(k_amax, 127.0))
    res = dict(
        G=G, rows=rows, used=used,
        q_amax=q_amax, k_amax=k_amax, q_scale=q_scale, k_scale=k_scale,
        q8=quantize_rows(xq, q_scale, rows), k8=quantize_rows(xk, k_scale, rows),
        v8=e4m3_bytes(V.float() if v_scale is None
                      else rn32_div(V.float(), v_scale.float()[:, None].expand_as(V))),
    )
    h = H // world_size

    def per_dest(p):
        sl = slice(p * h, (p + 1) * h)
        return dict(
            q8=res["q8"][:, :, sl], k8=res["k8"][:, :, sl],
            v8=res["v8"][:, :, sl].permute(0, 3, 2, 1),          # [B,D,h,S]
            q_scale=q_scale[:, sl], k_scale=k_scale[:, sl],
        )

    res["per_dest"] = per_dest
    return res
