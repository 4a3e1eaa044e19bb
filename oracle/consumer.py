"""A consumer of the unpacked tensors: attention over INT8 Q/K and FP8 E4M3 V, in float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The unpack_for_sage page names the consumer (the Sage attention kernel) and the layouts
it is handed: q8, k8 INT8 [B, S, h, D] with one FP32 scale per 64-row group in
q_scale, k_scale [B, h, W]; v8 FP8 E4M3 [B, D, h, ceil(S/64)*64]; the V scale stays with
the caller.  This module reads them the way such a consumer would -- a score is the
integer dot product of a Q row and a K row times the two rows' group scales, the softmax
runs over the live keys only, and the output weights the decoded E4M3 values (times the
caller's V scale, if any) -- but in float64 and without tiling, so that the result
depends only on the stored bytes and their layouts.  Smooth K needs no correction: a
per-channel mean removed from every key shifts every score of a query row by the same
amount, which the softmax cancels.

``reference_attention`` is the same attention on the original bf16/fp16 Q, K, V.
"""
from __future__ import annotations

import math

import torch

GROUP = 64


def e4m3_values(v8: torch.Tensor) -> torch.Tensor:
    """E4M3FN bytes -> float64 values (library decode)."""
    return v8.contiguous().view(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)


def _probabilities(q8, k8, q_scale, k_scale, b, j, queries, used):
    """Unnormalized softmax weights exp(score - row max) [nq, used] and their row sums,
    float64 (scores as defined in the module docstring)."""
    qi = torch.as_tensor(queries, dtype=torch.int64)
    D = q8.shape[-1]
    q = q8[b, qi, j].to(torch.float64)                       # [nq, D] integers
    k = k8[b, :used, j].to(torch.float64)                    # [nk, D]
    dots = q @ k.T                                           # exact: |sum| < 2^21
    keys = torch.arange(used)
    scores = dots * q_scale[b, j, qi // GROUP].double()[:, None] \
        * k_scale[b, j, keys // GROUP].double()[None, :] / math.sqrt(D)
    p = torch.exp(scores - scores.max(dim=-1, keepdim=True).values)
    return p, p.sum(dim=-1, keepdim=True)


def _values(v8, b, j, used, v_scale_row):
    v = e4m3_values(v8[b, :, j, :used]).T                    # [nk, D]
    if v_scale_row is not None:
        v = v * v_scale_row.double()[None, :]
    return v


def quantized_attention(q8, k8, v8, q_scale, k_scale, *, b: int, j: int, queries, used: int,
                        v_scale_row=None) -> torch.Tensor:
    """Output rows [len(queries), D] of local head j of batch entry b, from one
    destination's unpacked tensors (CPU).  Keys t < used; v_scale_row: optional [D]."""
    p, l = _probabilities(q8, k8, q_scale, k_scale, b, j, queries, used)
    return (p @ _values(v8, b, j, used, v_scale_row)) / l


def fp8_probability_bound(q8, k8, v8, q_scale, k_scale, *, b: int, j: int, queries,
                          used: int, v_scale_row=None, exponent_error: float = 0.0):
    """(out, bound) [len(queries), D]: the attention above and a per-element bound on how far
    a consumer may land from it that rounds each probability to E4M3 (after scaling it by
    448, with any running maximum m_run <= the row maximum), normalizes each row by the sum
    of its rounded probabilities, and computes each exponent argument (log2 units) to
    within `exponent_error` of score * log2(e) - m_run.

    In units of the row maximum, the exponent moves a probability p by a factor within
    2^(+-exponent_error); rounding to E4M3 then moves it by at most 2^-4 of itself in the
    normal range and by at most 2^-10 (half the smallest subnormal step) below it, i.e. by
    at most max(2^-4 p, 2^-10 / 448) <= max(2^-4 p, 2^-18); scaling by
    exp2(m_run - max) <= 1 only shrinks that.  So a rounded probability q_t lies within
        E_t = 2^x max(2^-4 p_t, 2^-18) + (2^x - 1) p_t        (x = exponent_error)
    of p_t.  As sum_t p_t (v_t - out) = 0, the consumer's sum_t q_t v_t / sum_t q_t differs
    from out by sum_t (q_t - p_t)(v_t - out) / sum_t q_t, hence
        |out_fp8 - out| <= sum_t E_t |v_t - out| / (sum_t p_t - sum_t E_t)
    (sum_t p_t >= 1, the maximum's term; the bound is infinite where the denominator is not
    positive), plus binary32 arithmetic (FP32 accumulation of up to `used` terms, the
    rescales, the final division), held to 1e-3 of sum_t p_t |v_t| / sum_t p_t."""
    p, l = _probabilities(q8, k8, q_scale, k_scale, b, j, queries, used)
    v = _values(v8, b, j, used, v_scale_row)
    out = (p @ v) / l
    grow = 2.0 ** exponent_error
    e = grow * torch.maximum(p * 2.0 ** -4, torch.full_like(p, 2.0 ** -18)) + (grow - 1.0) * p
    den = l - e.sum(dim=-1, keepdim=True)
    num = torch.stack([e[i] @ (v - out[i]).abs() for i in range(len(out))])   # [nq, D]
    bound = torch.where(den > 0, num / den.clamp_min(1e-300), torch.full_like(num, float("inf")))
    return out, bound + 1e-3 * (p @ v.abs()) / l


def reference_attention(Q, K, V, *, b: int, head: int, queries, used: int) -> torch.Tensor:
    """The same rows from the original global Q, K, V [B, S, H, D] (bf16/fp16 values) in
    float64."""
    qi = torch.as_tensor(queries, dtype=torch.int64)
    D = Q.shape[-1]
    q = Q[b, qi, head].double()
    k = K[b, :used, head].double()
    v = V[b, :used, head].double()
    p = torch.softmax((q @ k.T) / math.sqrt(D), dim=-1)
    return p @ v


def compare(out: torch.Tensor, ref: torch.Tensor) -> dict:
    """Cosine similarity and relative L2 / max errors of out against ref."""
    o, r = out.flatten().double(), ref.flatten().double()
    cos = float((o @ r) / (o.norm() * r.norm()).clamp_min(1e-300))
    rel_l2 = float((o - r).norm() / r.norm().clamp_min(1e-300))
    rel_max = float((o - r).abs().max() / r.abs().max().clamp_min(1e-300))
    return dict(cos=cos, rel_l2=rel_l2, rel_max=rel_max)
