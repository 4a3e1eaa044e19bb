"""The whole Ulysses group run through the C oracle, rank by rank.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The stats all-gather is the stack of every rank's boundary min/max, and the all-to-all is
the regrouping of the per-rank send buffers by destination (unpack_for_sage Parameters:
the receive buffer is source-major [world_size, chunk_bytes]).

The ranks' calls are independent of one another (each reads only its own shard, or, for
the unpack, its own receive buffer), so ``threads > 1`` runs them on a thread pool: the C
functions are called through ctypes, which releases the interpreter lock for the duration
of each call.  The arithmetic and every result are the same for any number of threads.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import torch

from . import (boundary_minmax, derive_k_boundary_amax, k_grouped_amax, pack,
               unpack_for_sage)


def shards(X: torch.Tensor, world_size: int):
    """Global [B,S,H,D] -> list of contiguous rank shards [B,L,H,D]."""
    B, S, H, D = X.shape
    L = S // world_size
    return [X[:, r * L:(r + 1) * L].contiguous() for r in range(world_size)]


def _map(fn, items, threads: int):
    items = list(items)
    if threads <= 1 or len(items) <= 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(max_workers=min(threads, len(items))) as ex:
        return list(ex.map(fn, items))


def run_stats(qs, ks, mean, *, world_size, used_sequence=None, threads=1, _lib=None):
    """Every rank's boundary min/max and grouped amax (Q raw, K centered), before derive.
    -> (q_mm [P,B,H,2,2,D], k_mm, q_amax_kernel list, k_amax_kernel list)."""
    P = world_size
    kw = dict(world_size=P, used_sequence=used_sequence, _lib=_lib)

    def one(r):
        return (boundary_minmax(qs[r], rank=r, **kw), boundary_minmax(ks[r], rank=r, **kw),
                k_grouped_amax(qs[r], None, rank=r, **kw),
                k_grouped_amax(ks[r], mean, rank=r, **kw))

    res = _map(one, range(P), threads)
    return (torch.stack([x[0] for x in res]), torch.stack([x[1] for x in res]),
            [x[2] for x in res], [x[3] for x in res])


def run_group(Q, K, V, mean, *, world_size, used_sequence=None, scale_sequence=None,
              destinations=None, v_scale=None, threads=1, _lib=None):
    """Q, K, V: global [B,S,H,D]; mean [B,H,D].  Returns every intermediate:
    q_minmax/k_minmax [P,B,H,2,2,D], q_amax_kernel/k_amax_kernel (before derive) and
    q_amax/k_amax (after derive) per rank, send buffers per rank, and the unpack 5-tuple
    per destination (all destinations unless ``destinations`` lists a subset).  v_scale:
    the caller's optional [B,H,D] V divisor.  threads: ranks (and destinations) run
    concurrently on that many threads."""
    P = world_size
    B, S, H, D = Q.shape
    L = S // P
    kw = dict(world_size=P, _lib=_lib)
    qs, ks, vs = shards(Q, P), shards(K, P), shards(V, P)
    q_mm, k_mm, q_amax_kernel, k_amax_kernel = run_stats(
        qs, ks, mean, world_size=P, used_sequence=used_sequence, threads=threads, _lib=_lib)
    q_amax = [a.clone() for a in q_amax_kernel]
    k_amax = [a.clone() for a in k_amax_kernel]
    for r in range(P):
        derive_k_boundary_amax(q_amax[r], q_mm, None, rank=r, local_sequence=L,
                               dtype=Q.dtype, **kw)
        derive_k_boundary_amax(k_amax[r], k_mm, mean, rank=r, local_sequence=L, **kw)
    sends = _map(lambda r: pack(qs[r], ks[r], vs[r], mean, q_amax[r], k_amax[r], rank=r,
                                v_scale=v_scale, **kw), range(P), threads)
    del qs, ks, vs
    dests = list(range(P) if destinations is None else destinations)

    def unpack_dest(p):
        recv = torch.stack([sends[r][p] for r in range(P)])
        return unpack_for_sage(recv, batch_size=B, local_sequence=L, local_heads=H // P,
                               head_dim=D, world_size=P, scale_sequence=scale_sequence,
                               _lib=_lib)

    outs = dict(zip(dests, _map(unpack_dest, dests, threads)))
    return dict(q_minmax=q_mm, k_minmax=k_mm, q_amax_kernel=q_amax_kernel,
                k_amax_kernel=k_amax_kernel, q_amax=q_amax, k_amax=k_amax, sends=sends,
                outs=outs)
