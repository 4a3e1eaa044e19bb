"""CPU oracle of the smooth-K low-precision Ulysses pack/unpack.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg import this package.  The product (``libulp.so`` and
``precision_attention_input_amd``) never imports it, and the two share no code.

Two independent oracles live here:

* ``oracle.c`` (wrapped below) -- the per-rank pipeline, step by step, in plain C loops:
  the bit-exact target for every byte the GPU path writes.
* ``brute.py`` -- the plain definition on the unsharded global tensors (no ranks, no
  slots, no chunks), written with torch CPU float32 operations.  It pins ``oracle.c``.

All tensors passed here are torch CPU tensors; ``bf16``/``fp16`` inputs are read as their
16-bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

# IEEE-faithful build: no FMA contraction, no fast-math, SSE float arithmetic.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

BF16, FP16 = 0, 1
GROUP = 64
FLOOR = 1e-7  # rounded to binary32 where used


def build(out: str = LIB_PATH, src: str = SRC_PATH, extra: list[str] | None = None) -> str:
    """Compile oracle.c with gcc into a shared library and return its path."""
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = ["gcc", *CFLAGS, *(extra or []), src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)    # atomic: concurrent builders never expose a partial file
    return out


_lib = None


def _load(path: str = LIB_PATH):
    lib = ctypes.CDLL(path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.ora_slots.argtypes = [i64]
    lib.ora_slots.restype = i64
    lib.ora_chunk_bytes.argtypes = [i64, i64, i64, i64]
    lib.ora_chunk_bytes.restype = i64
    lib.ora_e4m3.argtypes = [ctypes.c_float]
    lib.ora_e4m3.restype = ctypes.c_uint8
    lib.ora_quant_i8.argtypes = [ctypes.c_float, ctypes.c_float]
    lib.ora_quant_i8.restype = ctypes.c_int8
    lib.ora_k_grouped_amax.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, i64, i64, vp]
    lib.ora_k_grouped_amax.restype = None
    lib.ora_boundary_minmax.argtypes = [vp, i32, i64, i64, i64, i64, i64, i64, i64, vp]
    lib.ora_boundary_minmax.restype = None
    lib.ora_derive_k_boundary_amax.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, i64]
    lib.ora_derive_k_boundary_amax.restype = None
    lib.ora_pack.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp,
                             i64]
    lib.ora_pack.restype = None
    lib.ora_unpack_for_sage.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.ora_unpack_for_sage.restype = None
    lib.ora_bf16_bits.argtypes = [ctypes.c_float]
    lib.ora_bf16_bits.restype = ctypes.c_uint16
    lib.ora_fp16_bits.argtypes = [ctypes.c_float]
    lib.ora_fp16_bits.restype = ctypes.c_uint16
    lib.ora_k_mean.argtypes = [vp, i32, i64, i64, i64, i64, i64, i64, vp, vp]
    lib.ora_k_mean.restype = None
    return lib


def lib(path: str | None = None):
    """The loaded oracle library (built on first use if missing)."""
    global _lib
    if path is not None:
        return _load(path)
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        _lib = _load(LIB_PATH)
    return _lib


def _dt(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return BF16
    if x.dtype == torch.float16:
        return FP16
    raise TypeError(f"oracle inputs must be bf16 or fp16, got {x.dtype}")


def _p(x):
    if x is None:
        return None
    assert x.device.type == "cpu" and x.is_contiguous()
    return ctypes.c_void_p(x.data_ptr())


def slots(L: int) -> int:
    return int(lib().ora_slots(L))


def chunk_bytes(B: int, L: int, h: int, D: int) -> int:
    return int(lib().ora_chunk_bytes(B, L, h, D))


def e4m3(x: float) -> int:
    return int(lib().ora_e4m3(x))


def quant_i8(x: float, scale: float) -> int:
    return int(lib().ora_quant_i8(x, scale))


def k_grouped_amax(x, mean, *, rank, world_size, used_sequence=None, L=None, _lib=None):
    """x: [B,L,H,D] shard; mean: [B,H,D] or None (raw values).  -> [B,H,slots] fp32."""
    lb = _lib or lib()
    B, L, H, D = x.shape
    out = torch.empty(B, H, slots(L), dtype=torch.float32)
    lb.ora_k_grouped_amax(_p(x), _p(mean), _dt(x), B, L, H, D, rank, world_size,
                          used_sequence or 0, _p(out))
    return out


def boundary_minmax(x, *, rank, world_size, used_sequence=None, _lib=None):
    """x: [B,L,H,D] shard -> [B,H,2,2,D] fp32 raw min/max of the first/last touched group."""
    lb = _lib or lib()
    B, L, H, D = x.shape
    out = torch.empty(B, H, 2, 2, D, dtype=torch.float32)
    lb.ora_boundary_minmax(_p(x), _dt(x), B, L, H, D, rank, world_size, used_sequence or 0,
                           _p(out))
    return out


def derive_k_boundary_amax(grouped, gathered, mean, *, rank, local_sequence, world_size,
                           dtype=None, _lib=None):
    """Overwrites the boundary slots of ``grouped`` [B,H,slots] in place and returns it."""
    lb = _lib or lib()
    P, B, H, _, _, D = gathered.shape
    dt = _dt(mean) if mean is not None else (BF16 if dtype in (None, torch.bfloat16) else FP16)
    lb.ora_derive_k_boundary_amax(_p(grouped), _p(gathered.contiguous()), _p(mean), dt, B, H, D,
                                  rank, local_sequence, world_size)
    return grouped


def pack(q, k, v, mean, q_amax, k_amax, *, rank, world_size, v_scale=None, _lib=None):
    """-> send buffer [world_size, chunk_bytes] uint8 (chunk p for destination p).
    v_scale: optional [B,H,D] float32 divisor of V before E4M3."""
    lb = _lib or lib()
    B, L, H, D = q.shape
    h = H // world_size
    cb = chunk_bytes(B, L, h, D)
    send = torch.empty(world_size, cb, dtype=torch.uint8)
    if v_scale is not None:
        v_scale = v_scale.to(torch.float32).contiguous()
        assert v_scale.shape == (B, H, D)
    lb.ora_pack(_p(q), _p(k), _p(v), _p(mean), _dt(q), _p(q_amax.contiguous()),
                _p(k_amax.contiguous()), _p(v_scale), B, L, H, D, rank, world_size, _p(send),
                cb)
    return send


def unpack_for_sage(recv, *, batch_size, local_sequence, local_heads, head_dim, world_size,
                    scale_sequence=None, _lib=None):
    """recv: [world_size, chunk_bytes] uint8 -> (q8, k8, v8, q_scale, k_scale)."""
    lb = _lib or lib()
    B, L, h, D, P = batch_size, local_sequence, local_heads, head_dim, world_size
    S = P * L
    spad = (S + GROUP - 1) // GROUP * GROUP
    ns = scale_sequence or S
    W = (ns + GROUP - 1) // GROUP
    q8 = torch.empty(B, S, h, D, dtype=torch.int8)
    k8 = torch.empty(B, S, h, D, dtype=torch.int8)
    v8 = torch.empty(B, D, h, spad, dtype=torch.uint8)
    qs = torch.empty(B, h, W, dtype=torch.float32)
    ks = torch.empty(B, h, W, dtype=torch.float32)
    lb.ora_unpack_for_sage(_p(recv.contiguous()), B, L, h, D, P, scale_sequence or 0,
                           _p(q8), _p(k8), _p(v8), _p(qs), _p(ks))
    return q8, k8, v8, qs, ks


def dtype_bits(x: float, dtype) -> int:
    """binary32 value -> 16-bit pattern of bf16/fp16, round to nearest even."""
    f = lib().ora_bf16_bits if dtype == torch.bfloat16 else lib().ora_fp16_bits
    return int(f(x))


def k_mean(k_stack, *, used_sequence=None, _lib=None):
    """k_stack: stacked shards [P,B,L,H,D] -> (mean fp32 [B,H,D], mean in the dtype)."""
    lb = _lib or lib()
    P, B, L, H, D = k_stack.shape
    mf = torch.empty(B, H, D, dtype=torch.float32)
    md = torch.empty(B, H, D, dtype=k_stack.dtype)
    lb.ora_k_mean(_p(k_stack.contiguous()), _dt(k_stack), B, L, H, D, P, used_sequence or 0,
                  _p(mf), _p(md))
    return mf, md
