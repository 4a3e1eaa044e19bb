"""Smooth-K low-precision Ulysses pack/unpack for SageAttention inputs on MI355X (gfx950).

A thin Python binding over the C ABI of ``libulp.so`` (declared in ``include/ulp.h``):
argument marshalling only.  Every step runs in the library's HIP kernels; torch provides
device memory and the current stream.  There is no fallback: when the library is missing,
every call raises.

Per-rank functions mirror the FlashInfer pages ``flashinfer.comm._ulysses_lowp``:
``k_grouped_amax``, ``derive_k_boundary_amax`` and ``unpack_for_sage`` (the pages'
``enable_pdl`` has no counterpart: launches are ordered on the current stream), plus
``boundary_minmax`` (the stats all-gather payload) and ``pack``.  The ``group_*`` functions
run a whole Ulysses group held by one GPU with one launch per step.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "ULP_NONE", "GROUP_ROWS", "UlpError", "lib", "slots", "chunk_bytes", "scale_widths",
    "k_grouped_amax", "boundary_minmax", "derive_k_boundary_amax", "pack", "unpack_for_sage",
    "group_stats", "group_derive", "group_pack", "group_unpack", "group_buffer", "k_mean",
    "k_mean_noalloc",
    "group_stats_with_mean", "consumer_attention", "stats_pack", "derive_pack",
    "group_stats_pack", "group_derive_pack",
    "unpack_shapes",
]

ULP_NONE = -1
GROUP_ROWS = 64
_OK, _EINVAL, _EUNSUPPORTED, _EALIGN, _ELAUNCH = 0, 1, 2, 3, 4
_DTYPES = {torch.bfloat16: 0, torch.float16: 1}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libulp.so")
_lib = None


class UlpError(RuntimeError):
    """A kernel launch failed (ULP_ELAUNCH)."""


def lib():
    """The loaded libulp.so; raises if it has not been built."""
    if _lib is None:
        load(LIB_PATH)
    return _lib


def load(path: str = LIB_PATH):
    """Load the library at ``path`` (a build of the same sources) and route every call of
    this module to it from now on; returns it.  Raises if the file does not exist."""
    global _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it first (python -c "
            "'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    sig = {
        "ulp_slots": ([i64], i64),
        "ulp_scale_widths": ([i64, vp, vp], i32),
        "ulp_chunk_bytes": ([i64, i64, i64, i64], i64),
        "ulp_last_error": ([], ctypes.c_char_p),
        "ulp_k_grouped_amax": ([vp, vp, i32, i64, i64, i64, i64, i32, i32, i64, vp, vp], i32),
        "ulp_boundary_minmax": ([vp, i32, i64, i64, i64, i64, i32, i32, i64, vp, vp], i32),
        "ulp_derive_k_boundary_amax": ([vp, vp, vp, i32, i64, i64, i64, i32, i64, i32, vp],
                                       i32),
        "ulp_pack": ([vp, vp, vp, vp, i32, vp, vp, vp, i64, i64, i64, i64, i32, i32, vp, i64,
                      vp], i32),
        "ulp_unpack_for_sage": ([vp, i64, i64, i64, i64, i32, i32, i64, vp, vp, vp, vp, vp,
                                 vp], i32),
        "ulp_group_stats": ([vp, vp, vp, i32, i64, i64, i64, i64, i32, i64, vp, vp, vp, vp,
                             vp], i32),
        "ulp_group_derive": ([vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, i32, vp], i32),
        "ulp_group_pack": ([vp, vp, vp, vp, i32, vp, vp, vp, i64, i64, i64, i64, i32, vp,
                            vp], i32),
        "ulp_group_unpack": ([vp, i64, i64, i64, i64, i32, i32, i64, vp, vp, vp, vp, vp, vp],
                             i32),
        "ulp_k_mean_workspace_bytes": ([i64, i64, i64, i64, i32, i64], i64),
        "ulp_k_mean": ([vp, i32, i64, i64, i64, i64, i32, i64, vp, i64, vp, vp, vp], i32),
        "ulp_k_mean_noalloc": ([vp, i32, i64, i64, i64, i64, i32, i64, vp, vp, vp], i32),
        "ulp_group_stats_with_mean_workspace_bytes": ([i64, i64, i64, i64, i32], i64),
        "ulp_group_stats_with_mean": ([vp, vp, i32, i64, i64, i64, i64, i32, i64, vp, i64,
                                       vp, vp, vp, vp, vp, vp, vp], i32),
        "ulp_stats_pack": ([vp, vp, vp, vp, i32, vp, i64, i64, i64, i64, i32, i32, i64, vp,
                            vp, vp, vp, vp, i64, vp], i32),
        "ulp_derive_pack": ([vp, vp, vp, i32, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32,
                             i64, vp, i64, vp], i32),
        "ulp_group_stats_pack": ([vp, vp, vp, vp, i32, vp, i64, i64, i64, i64, i32, i64, vp,
                                  vp, vp, vp, vp, vp], i32),
        "ulp_group_derive_pack": ([vp, vp, vp, i32, vp, vp, vp, vp, i64, i64, i64, i64, i32,
                                   i64, vp, vp], i32),
        "ulp_consumer_attention": ([vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                    vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc == _OK:
        return
    msg = lib().ulp_last_error().decode()
    if rc == _ELAUNCH:
        raise UlpError(msg)
    raise ValueError(msg)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


_F32 = (torch.float32,)
_X16 = (torch.bfloat16, torch.float16)
_I8 = (torch.int8,)
_B8 = (torch.uint8, torch.float8_e4m3fn)


def _need(t, shape, dtypes, name):
    """The library reads and writes every tensor by the sizes it is given, not by the
    tensor's own: ``t`` (None passes) must hold exactly prod(shape) elements of one of
    ``dtypes``, or the call is refused before anything runs."""
    if t is None:
        return
    n = math.prod(shape)
    if t.dtype not in dtypes or t.numel() != n:
        raise ValueError(f"{name} must hold {n} elements {tuple(shape)} of "
                         f"{'/'.join(str(d) for d in dtypes)}, got {t.dtype} {tuple(t.shape)}")


def _need_bytes(t, nbytes, name):
    """A byte buffer addressed by offsets the library computes (a destination stride may
    reach past a view into the rest of its buffer): at least ``nbytes`` of the tensor's
    storage from its first byte on."""
    room = t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()
    if room < nbytes:
        raise ValueError(f"{name} must reach at least {nbytes} bytes, its storage holds "
                         f"{room} from its start")


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise ValueError(f"expected bfloat16 or float16, got {t.dtype}")
    return _DTYPES[t.dtype]


def _none(v):
    return ULP_NONE if v is None else int(v)


def slots(local_sequence: int) -> int:
    """slots(L, 64): the most 64-row global groups an L-row shard can touch."""
    return int(lib().ulp_slots(local_sequence))


def chunk_bytes(batch_size: int, local_sequence: int, local_heads: int, head_dim: int) -> int:
    return int(lib().ulp_chunk_bytes(batch_size, local_sequence, local_heads, head_dim))


def scale_widths(n: int) -> tuple[int, int]:
    """(q_width, k_width) of the scale tensors for a live prefix of n rows."""
    q, k = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ulp_scale_widths(n, ctypes.byref(q), ctypes.byref(k)))
    return q.value, k.value


def _need_unpack_out(out, shapes, lead=()):
    qk, vs, sc = shapes
    for t, shape, dts, name in zip(out, (qk, qk, vs, sc, sc), (_I8, _I8, _B8, _F32, _F32),
                                   ("q8", "k8", "v8", "q_scale", "k_scale")):
        _need(t, (*lead, *shape), dts, name)


def unpack_shapes(batch_size, local_sequence, local_heads, head_dim, world_size,
                  scale_sequence=None):
    S = world_size * local_sequence
    spad = (S + GROUP_ROWS - 1) // GROUP_ROWS * GROUP_ROWS
    W = scale_widths(scale_sequence or S)[0]
    B, h, D = batch_size, local_heads, head_dim
    return (B, S, h, D), (B, D, h, spad), (B, h, W)


# ------------------------------------------------------------------------- per rank

def k_grouped_amax(k, k_mean_global, *, rank, world_size, used_sequence=None, out=None,
                   enable_pdl=None):
    """[B, H, slots(L)] fp32 partial amax of |K - k_mean_global| (k_mean_global None: raw
    values, the Q amax).  flashinfer.comm._ulysses_lowp.k_grouped_amax.  ``enable_pdl`` is
    accepted and ignored: launches on one stream run in order on gfx950."""
    _dev(k, k_mean_global, out)
    B, L, H, D = k.shape
    if out is None:
        out = torch.empty(B, H, slots(L), dtype=torch.float32, device=k.device)
    _need(k_mean_global, (B, H, D), (k.dtype,), "k_mean_global")
    _need(out, (B, H, slots(L)), _F32, "out")
    _check(lib().ulp_k_grouped_amax(_p(k), _p(k_mean_global), _dt(k), B, L, H, D, rank,
                                    world_size, _none(used_sequence), _p(out), _stream(k)))
    return out


def boundary_minmax(x, *, rank, world_size, used_sequence=None, out=None):
    """[B, H, 2, 2, D] fp32 raw min/max of the live rows of the rank's first/last group."""
    _dev(x, out)
    B, L, H, D = x.shape
    if out is None:
        out = torch.empty(B, H, 2, 2, D, dtype=torch.float32, device=x.device)
    _need(out, (B, H, 2, 2, D), _F32, "out")
    _check(lib().ulp_boundary_minmax(_p(x), _dt(x), B, L, H, D, rank, world_size,
                                     _none(used_sequence), _p(out), _stream(x)))
    return out


def derive_k_boundary_amax(grouped_amax, gathered_minmax, k_mean_global, *, rank,
                           local_sequence, world_size):
    """Overwrites this rank's boundary slots in place and returns ``grouped_amax``.
    flashinfer.comm._ulysses_lowp.derive_k_boundary_amax.  k_mean_global None: mean +0."""
    _dev(grouped_amax, gathered_minmax, k_mean_global)
    P, B, H, _, _, D = gathered_minmax.shape
    _need(gathered_minmax, (world_size, B, H, 2, 2, D), _F32, "gathered_minmax")
    _need(grouped_amax, (B, H, slots(local_sequence)), _F32, "grouped_amax")
    _need(k_mean_global, (B, H, D), _X16, "k_mean_global")
    dt = _dt(k_mean_global) if k_mean_global is not None else 0
    _check(lib().ulp_derive_k_boundary_amax(_p(grouped_amax), _p(gathered_minmax),
                                            _p(k_mean_global), dt, B, H, D, rank,
                                            local_sequence, world_size,
                                            _stream(grouped_amax)))
    return grouped_amax


def _need_shard_inputs(q, k, v, k_mean_global, B, L, H, D, lead=()):
    """k and v like q (shape and dtype), the mean [B,H,D] in the same dtype."""
    for t, name in ((k, "k"), (v, "v")):
        _need(t, (*lead, B, L, H, D), (q.dtype,), name)
    _need(k_mean_global, (B, H, D), (q.dtype,), "k_mean_global")


def _v_scale(v_scale, B, H, D):
    if v_scale is not None and (v_scale.dtype != torch.float32 or
                                tuple(v_scale.shape) != (B, H, D)):
        raise ValueError(f"v_scale must be float32 [{B}, {H}, {D}], got {v_scale.dtype} "
                         f"{tuple(v_scale.shape)}")


def pack(q, k, v, k_mean_global, q_amax, k_amax, *, rank, world_size, v_scale=None, send=None,
         dest_stride=None):
    """Quantize one rank's shard; returns the send buffer [world_size, chunk_bytes] uint8
    (or writes chunk p at ``send`` + p * dest_stride bytes when ``send`` is given).
    v_scale: the caller's optional [B,H,D] float32 V divisor, applied before E4M3."""
    _dev(q, k, v, k_mean_global, q_amax, k_amax, v_scale)
    B, L, H, D = q.shape
    _v_scale(v_scale, B, H, D)
    cb = chunk_bytes(B, L, H // world_size, D)
    if send is None:
        send = torch.empty(world_size, cb, dtype=torch.uint8, device=q.device)
        dest_stride = cb
    _need_shard_inputs(q, k, v, k_mean_global, B, L, H, D)
    _need(q_amax, (B, H, slots(L)), _F32, "q_amax")
    _need(k_amax, (B, H, slots(L)), _F32, "k_amax")
    _need_bytes(send, (world_size - 1) * (dest_stride or cb) + cb, "send")
    _check(lib().ulp_pack(_p(q), _p(k), _p(v), _p(k_mean_global), _dt(q), _p(q_amax),
                          _p(k_amax), _p(v_scale), B, L, H, D, rank, world_size, _p(send),
                          dest_stride or cb, _stream(q)))
    return send


def _alloc_unpack(device, shapes, lead=()):
    qk, vs, sc = shapes
    return (torch.empty(*lead, *qk, dtype=torch.int8, device=device),
            torch.empty(*lead, *qk, dtype=torch.int8, device=device),
            torch.empty(*lead, *vs, dtype=torch.float8_e4m3fn, device=device),
            torch.empty(*lead, *sc, dtype=torch.float32, device=device),
            torch.empty(*lead, *sc, dtype=torch.float32, device=device))


def unpack_for_sage(recv_u8, *, batch_size, local_sequence, local_heads, head_dim, world_size,
                    aligned=None, scale_sequence=None, out=None, enable_pdl=None):
    """(q8, k8, v8, q_scale, k_scale): INT8 [B,S,h,D] x2, FP8 E4M3 [B,D,h,ceil(S/64)*64],
    FP32 [B,h,W] x2.  flashinfer.comm._ulysses_lowp.unpack_for_sage.  ``enable_pdl`` is
    accepted and ignored: launches on one stream run in order on gfx950."""
    if out is None:
        out = _alloc_unpack(recv_u8.device, unpack_shapes(batch_size, local_sequence,
                                                          local_heads, head_dim, world_size,
                                                          scale_sequence))
    _dev(recv_u8, *out)
    _need_bytes(recv_u8, world_size * chunk_bytes(batch_size, local_sequence, local_heads,
                                                  head_dim), "recv_u8")
    _need_unpack_out(out, unpack_shapes(batch_size, local_sequence, local_heads, head_dim,
                                        world_size, scale_sequence))
    q8, k8, v8, qs, ks = out
    _check(lib().ulp_unpack_for_sage(_p(recv_u8), batch_size, local_sequence, local_heads,
                                     head_dim, world_size, _none(aligned),
                                     _none(scale_sequence), _p(q8), _p(k8), _p(v8), _p(qs),
                                     _p(ks), _stream(recv_u8)))
    return tuple(out)


# ------------------------------------------------------------------------- whole group

def _need_group_stats(q, k, k_mean_global, out, world_size):
    """Stacked shards [world_size,B,L,H,D]; statistics outputs of those sizes."""
    P, B, L, H, D = q.shape
    if P != world_size:
        raise ValueError(f"stacked shards hold {P} ranks, world_size is {world_size}")
    _need(k, q.shape, (q.dtype,), "k")
    _need(k_mean_global, (B, H, D), (q.dtype,), "k_mean_global")
    for t, shape, name in zip(out, ((P, B, H, slots(L)),) * 2 + ((P, B, H, 2, 2, D),) * 2,
                              ("q_amax", "k_amax", "q_minmax", "k_minmax")):
        _need(t, shape, _F32, name)


def group_stats(q, k, k_mean_global, *, world_size, used_sequence=None, out=None):
    """Stacked shards [P,B,L,H,D] -> (q_amax, k_amax [P,B,H,slots], q_minmax, k_minmax
    [P,B,H,2,2,D]) in one launch."""
    P, B, L, H, D = q.shape
    if out is None:
        f = dict(dtype=torch.float32, device=q.device)
        out = (torch.empty(P, B, H, slots(L), **f), torch.empty(P, B, H, slots(L), **f),
               torch.empty(P, B, H, 2, 2, D, **f), torch.empty(P, B, H, 2, 2, D, **f))
    _dev(q, k, k_mean_global, *out)
    _need_group_stats(q, k, k_mean_global, out, world_size)
    qa, ka, qm, km = out
    _check(lib().ulp_group_stats(_p(q), _p(k), _p(k_mean_global), _dt(q), B, L, H, D,
                                 world_size, _none(used_sequence), _p(qa), _p(ka), _p(qm),
                                 _p(km), _stream(q)))
    return tuple(out)


def group_derive(q_amax, k_amax, q_minmax, k_minmax, k_mean_global, *, local_sequence,
                 world_size):
    """Boundary derive of every rank for Q and K, in place; returns (q_amax, k_amax)."""
    _dev(q_amax, k_amax, q_minmax, k_minmax, k_mean_global)
    P, B, H, _, _, D = k_minmax.shape
    for t, name in ((q_minmax, "q_minmax"), (k_minmax, "k_minmax")):
        _need(t, (world_size, B, H, 2, 2, D), _F32, name)
    for t, name in ((q_amax, "q_amax"), (k_amax, "k_amax")):
        _need(t, (world_size, B, H, slots(local_sequence)), _F32, name)
    _need(k_mean_global, (B, H, D), _X16, "k_mean_global")
    _check(lib().ulp_group_derive(_p(q_amax), _p(k_amax), _p(q_minmax), _p(k_minmax),
                                  _p(k_mean_global), _dt(k_mean_global), B, H, D,
                                  local_sequence, world_size, _stream(q_amax)))
    return q_amax, k_amax


def group_buffer(batch_size, local_sequence, heads, head_dim, world_size, device):
    """An all-to-all buffer [P_dst, P_src, chunk_bytes] uint8."""
    cb = chunk_bytes(batch_size, local_sequence, heads // world_size, head_dim)
    return torch.empty(world_size, world_size, cb, dtype=torch.uint8, device=device)


def group_pack(q, k, v, k_mean_global, q_amax, k_amax, *, world_size, v_scale=None,
               group=None):
    """Every rank's pack into the all-to-all buffer [P_dst, P_src, chunk_bytes]."""
    P, B, L, H, D = q.shape
    if group is None:
        group = group_buffer(B, L, H, D, world_size, q.device)
    _dev(q, k, v, k_mean_global, q_amax, k_amax, v_scale, group)
    _v_scale(v_scale, B, H, D)
    if P != world_size:
        raise ValueError(f"stacked shards hold {P} ranks, world_size is {world_size}")
    _need_shard_inputs(q, k, v, k_mean_global, B, L, H, D, lead=(P,))
    _need(q_amax, (P, B, H, slots(L)), _F32, "q_amax")
    _need(k_amax, (P, B, H, slots(L)), _F32, "k_amax")
    _need_bytes(group, P * P * chunk_bytes(B, L, H // world_size, D), "group")
    _check(lib().ulp_group_pack(_p(q), _p(k), _p(v), _p(k_mean_global), _dt(q), _p(q_amax),
                                _p(k_amax), _p(v_scale), B, L, H, D, world_size, _p(group),
                                _stream(q)))
    return group


def group_unpack(group, *, batch_size, local_sequence, local_heads, head_dim, world_size,
                 aligned=None, scale_sequence=None, out=None):
    """Every destination's unpack; outputs stacked over destinations."""
    if out is None:
        out = _alloc_unpack(group.device, unpack_shapes(batch_size, local_sequence,
                                                        local_heads, head_dim, world_size,
                                                        scale_sequence), lead=(world_size,))
    _dev(group, *out)
    _need_bytes(group, world_size * world_size * chunk_bytes(batch_size, local_sequence,
                                                              local_heads, head_dim), "group")
    _need_unpack_out(out, unpack_shapes(batch_size, local_sequence, local_heads, head_dim,
                                        world_size, scale_sequence), lead=(world_size,))
    q8, k8, v8, qs, ks = out
    _check(lib().ulp_group_unpack(_p(group), batch_size, local_sequence, local_heads,
                                  head_dim, world_size, _none(aligned), _none(scale_sequence),
                                  _p(q8), _p(k8), _p(v8), _p(qs), _p(ks), _stream(group)))
    return tuple(out)


# ------------------------------------------------------------------------- one-read step

def _stats_out(lead, B, L, H, D, device):
    f = dict(dtype=torch.float32, device=device)
    return (torch.empty(*lead, B, H, slots(L), **f), torch.empty(*lead, B, H, slots(L), **f),
            torch.empty(*lead, B, H, 2, 2, D, **f), torch.empty(*lead, B, H, 2, 2, D, **f))


def stats_pack(q, k, v, k_mean_global, *, rank, world_size, used_sequence=None, v_scale=None,
               out=None, send=None, dest_stride=None):
    """One rank's grouped amax (Q raw, K centered), boundary min/max and the pack of every
    slot that derive cannot change, from one read of q, k, v [B,L,H,D].  Returns
    ((q_amax, k_amax, q_minmax, k_minmax), send); after the all-gather of the min/max,
    finish with derive_pack."""
    B, L, H, D = q.shape
    if out is None:
        out = _stats_out((), B, L, H, D, q.device)
    cb = chunk_bytes(B, L, H // world_size, D)
    if send is None:
        send = torch.empty(world_size, cb, dtype=torch.uint8, device=q.device)
        dest_stride = cb
    _dev(q, k, v, k_mean_global, v_scale, *out)
    _v_scale(v_scale, B, H, D)
    _need_shard_inputs(q, k, v, k_mean_global, B, L, H, D)
    for t, shape, name in zip(out, ((B, H, slots(L)),) * 2 + ((B, H, 2, 2, D),) * 2,
                              ("q_amax", "k_amax", "q_minmax", "k_minmax")):
        _need(t, shape, _F32, name)
    _need_bytes(send, (world_size - 1) * (dest_stride or cb) + cb, "send")
    qa, ka, qm, km = out
    _check(lib().ulp_stats_pack(_p(q), _p(k), _p(v), _p(k_mean_global), _dt(q), _p(v_scale),
                                B, L, H, D, rank, world_size, _none(used_sequence), _p(qa),
                                _p(ka), _p(qm), _p(km), _p(send), dest_stride or cb,
                                _stream(q)))
    return tuple(out), send


def derive_pack(q, k, k_mean_global, q_amax, k_amax, q_minmax, k_minmax, *, rank, world_size,
                send, used_sequence=None, dest_stride=None):
    """derive_k_boundary_amax on both amax in place (gathered min/max [P,B,H,2,2,D]), then
    the pack of the slots that waited for it.  Returns (q_amax, k_amax)."""
    _dev(q, k, k_mean_global, q_amax, k_amax, q_minmax, k_minmax, send)
    B, L, H, D = q.shape
    cb = chunk_bytes(B, L, H // world_size, D)
    _need(k, (B, L, H, D), (q.dtype,), "k")
    _need(k_mean_global, (B, H, D), (q.dtype,), "k_mean_global")
    for t, name in ((q_amax, "q_amax"), (k_amax, "k_amax")):
        _need(t, (B, H, slots(L)), _F32, name)
    for t, name in ((q_minmax, "q_minmax"), (k_minmax, "k_minmax")):
        _need(t, (world_size, B, H, 2, 2, D), _F32, name)
    _need_bytes(send, (world_size - 1) * (dest_stride or cb) + cb, "send")
    _check(lib().ulp_derive_pack(_p(q), _p(k), _p(k_mean_global), _dt(q), _p(q_amax),
                                 _p(k_amax), _p(q_minmax), _p(k_minmax), B, L, H, D, rank,
                                 world_size, _none(used_sequence), _p(send), dest_stride or cb,
                                 _stream(q)))
    return q_amax, k_amax


def group_stats_pack(q, k, v, k_mean_global, *, world_size, used_sequence=None, v_scale=None,
                     out=None, group=None):
    """stats_pack for every rank of stacked shards [P,B,L,H,D]; returns ((q_amax, k_amax
    [P,B,H,slots], q_minmax, k_minmax [P,B,H,2,2,D]), group).  Then group_derive_pack."""
    P, B, L, H, D = q.shape
    if out is None:
        out = _stats_out((P,), B, L, H, D, q.device)
    if group is None:
        group = group_buffer(B, L, H, D, world_size, q.device)
    _dev(q, k, v, k_mean_global, v_scale, group, *out)
    _v_scale(v_scale, B, H, D)
    _need_group_stats(q, k, k_mean_global, out, world_size)
    _need(v, q.shape, (q.dtype,), "v")
    _need_bytes(group, P * P * chunk_bytes(B, L, H // world_size, D), "group")
    qa, ka, qm, km = out
    _check(lib().ulp_group_stats_pack(_p(q), _p(k), _p(v), _p(k_mean_global), _dt(q),
                                      _p(v_scale), B, L, H, D, world_size,
                                      _none(used_sequence), _p(qa), _p(ka), _p(qm), _p(km),
                                      _p(group), _stream(q)))
    return tuple(out), group


def group_derive_pack(q, k, k_mean_global, q_amax, k_amax, q_minmax, k_minmax, *,
                      world_size, group, used_sequence=None):
    """derive_pack for every rank (after group_stats_pack); returns (q_amax, k_amax)."""
    _dev(q, k, k_mean_global, q_amax, k_amax, q_minmax, k_minmax, group)
    P, B, L, H, D = q.shape
    _need_group_stats(q, k, k_mean_global, (q_amax, k_amax, q_minmax, k_minmax), world_size)
    _need_bytes(group, P * P * chunk_bytes(B, L, H // world_size, D), "group")
    _check(lib().ulp_group_derive_pack(_p(q), _p(k), _p(k_mean_global), _dt(q), _p(q_amax),
                                       _p(k_amax), _p(q_minmax), _p(k_minmax), B, L, H, D,
                                       world_size, _none(used_sequence), _p(group),
                                       _stream(q)))
    return q_amax, k_amax


# ------------------------------------------------------------------------- global K mean

def k_mean(k, *, world_size, used_sequence=None, workspace=None, out=None):
    """Stacked K shards [P,B,L,H,D] -> (mean fp32 [B,H,D], mean in the dtype [B,H,D]): the
    k_mean_global input of the pages, over the live rows [0, used)."""
    P, B, L, H, D = k.shape
    need = int(lib().ulp_k_mean_workspace_bytes(B, L, H, D, world_size, _none(used_sequence)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=k.device)
    if out is None:
        out = (torch.empty(B, H, D, dtype=torch.float32, device=k.device),
               torch.empty(B, H, D, dtype=k.dtype, device=k.device))
    _dev(k, workspace, *out)
    mf, md = out
    if P != world_size:
        raise ValueError(f"stacked shards hold {P} ranks, world_size is {world_size}")
    _need(mf, (B, H, D), _F32, "mean_f32")
    _need(md, (B, H, D), (k.dtype,), "mean_dtype")
    _check(lib().ulp_k_mean(_p(k), _dt(k), B, L, H, D, world_size, _none(used_sequence),
                            _p(workspace), workspace.numel() * workspace.element_size(),
                            _p(mf), _p(md), _stream(k)))
    return mf, md


def k_mean_noalloc(k, *, world_size, out, used_sequence=None):
    """``k_mean`` without a workspace argument: the library's own device scratch array
    serves as workspace (nothing is allocated, here or in the library).  ``out`` = (mean
    fp32 [B,H,D], mean in the dtype [B,H,D] or None) must be given."""
    P, B, L, H, D = k.shape
    mf, md = out
    _dev(k, mf, md)
    if P != world_size:
        raise ValueError(f"stacked shards hold {P} ranks, world_size is {world_size}")
    _need(mf, (B, H, D), _F32, "mean_f32")
    _need(md, (B, H, D), (k.dtype,), "mean_dtype")
    _check(lib().ulp_k_mean_noalloc(_p(k), _dt(k), B, L, H, D, world_size,
                                    _none(used_sequence), _p(mf), _p(md), _stream(k)))
    return mf, md


def group_stats_with_mean(q, k, *, world_size, used_sequence=None, workspace=None, out=None):
    """Stacked shards [P,B,L,H,D] -> (q_amax, k_amax, q_minmax, k_minmax, k_mean_f32,
    k_mean_dtype), reading Q and K once each: the statistics of ``group_stats`` with the
    global K mean formed in the same pass over K."""
    P, B, L, H, D = q.shape
    need = int(lib().ulp_group_stats_with_mean_workspace_bytes(B, L, H, D, world_size))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        f = dict(dtype=torch.float32, device=q.device)
        out = (torch.empty(P, B, H, slots(L), **f), torch.empty(P, B, H, slots(L), **f),
               torch.empty(P, B, H, 2, 2, D, **f), torch.empty(P, B, H, 2, 2, D, **f),
               torch.empty(B, H, D, **f), torch.empty(B, H, D, dtype=q.dtype, device=q.device))
    _dev(q, k, workspace, *out)
    _need_group_stats(q, k, None, out[:4], world_size)
    _need(out[4], (B, H, D), _F32, "mean_f32")
    _need(out[5], (B, H, D), (q.dtype,), "mean_dtype")
    qa, ka, qm, km, mf, md = out
    _check(lib().ulp_group_stats_with_mean(
        _p(q), _p(k), _dt(q), B, L, H, D, world_size, _none(used_sequence), _p(workspace),
        workspace.numel() * workspace.element_size(), _p(qa), _p(ka), _p(qm), _p(km), _p(mf),
        _p(md), _stream(q)))
    return tuple(out)


# ------------------------------------------------------------------------- consumer check

def consumer_attention(q8, k8, v8, q_scale, k_scale, *, used, v_scale=None, out=None):
    """Attention over one destination's unpacked tensors as the Sage consumer reads them
    (INT8 Q.K, FP8 P.V on MFMA): q8, k8 [B,S,h,D] int8, v8 [B,D,h,Spad] E4M3, scales
    [B,h,W], v_scale [B,h,D] or None -> out [B,used,h,D] float32."""
    B, S, h, D = q8.shape
    W = q_scale.shape[-1]
    if v_scale is not None and (v_scale.dtype != torch.float32 or
                                tuple(v_scale.shape) != (B, h, D)):
        raise ValueError("v_scale must be float32 [B, h, D]")
    if out is None:
        out = torch.empty(B, used, h, D, dtype=torch.float32, device=q8.device)
    _dev(q8, k8, v8, q_scale, k_scale, v_scale, out)
    _need(q8, (B, S, h, D), _I8, "q8")
    _need(k8, (B, S, h, D), _I8, "k8")
    _need(v8, (B, D, h, (S + GROUP_ROWS - 1) // GROUP_ROWS * GROUP_ROWS), _B8, "v8")
    _need(q_scale, (B, h, W), _F32, "q_scale")
    _need(k_scale, (B, h, W), _F32, "k_scale")
    if not 1 <= used <= S:
        raise ValueError(f"used must be in [1, {S}], got {used}")
    _need(out, (B, used, h, D), _F32, "out")
    _check(lib().ulp_consumer_attention(_p(q8), _p(k8), _p(v8), _p(q_scale), _p(k_scale),
                                        _p(v_scale), B, S, h, D, W, used, _p(out),
                                        _stream(q8)))
    return out
