"""The C ABI of libulp.so without a GPU: every symbol declared in include/ulp.h is exported,
the geometry helpers agree with the oracle, and every validation error is reported with
its code before anything is launched (CPU only: no call here reaches a kernel)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import oracle
import precision_attention_input_amd as ulp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ulp.h")

OK, EINVAL, EUNSUPPORTED, EALIGN = 0, 1, 2, 3
NONE = -1
A = 0x10000          # a fake, 16-byte aligned address: validation rejects before any use


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ulp.LIB_PATH):
        from precision_attention_input_amd import _build
        _build.build()
    return ulp.lib()


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ulp_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared()
    assert "ulp_pack" in names and "ulp_unpack_for_sage" in names and len(names) >= 13
    for n in names:
        assert hasattr(L, n), n




def test_library_exports_nothing_undeclared(L):
    """The C-ABI surface is exactly ulp.h: no ulp_* symbol is exported that the header does
    not declare (read with nm from the library built here)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", ulp.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {f[2] for f in (line.split() for line in out.splitlines())
                if len(f) == 3 and f[1] == "T" and f[2].startswith("ulp_")}
    assert exported == set(declared())

def test_binding_signatures_match_header(L):
    """Every declaration in include/ulp.h has a binding with the same number of arguments,
    pointers where the header has pointers, int64_t and int where it has those (a drifted
    signature would otherwise pass garbage to a kernel)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    decls = re.findall(r"\b(?:int64_t|int|const char\*)\s+(ulp_\w+)\s*\(([^)]*)\)\s*;", text)
    assert len(decls) == len(declared())
    for name, params in decls:
        want = []
        for prm in (x.strip() for x in params.split(",")):
            if not prm or prm == "void":
                continue
            want.append(ctypes.c_void_p if "*" in prm else
                        ctypes.c_int64 if prm.startswith("int64_t") else ctypes.c_int)
        got = list(getattr(L, name).argtypes or [])
        assert got == want, f"{name}: binding {got} vs header {want}"

def test_geometry_helpers_match_oracle(L, olib):
    for Lseq in [1, 2, 31, 63, 64, 65, 96, 100, 127, 128, 129, 200, 1000, 2048, 4096, 9360]:
        assert ulp.slots(Lseq) == oracle.slots(Lseq)
        for (B, h, D) in [(1, 1, 64), (2, 4, 128), (4, 12, 64), (1, 5, 128)]:
            assert ulp.chunk_bytes(B, Lseq, h, D) == oracle.chunk_bytes(B, Lseq, h, D)
            assert ulp.chunk_bytes(B, Lseq, h, D) % 256 == 0
    assert ulp.scale_widths(3700) == (58, 58)
    assert ulp.scale_widths(1) == (1, 1)
    assert ulp.scale_widths(64) == (1, 1) and ulp.scale_widths(65) == (2, 2)
    assert L.ulp_slots(0) == 0 and L.ulp_chunk_bytes(0, 1, 1, 64) == 0


def test_scale_widths_rejects_empty_prefix(L):
    q, k = ctypes.c_int64(), ctypes.c_int64()
    assert L.ulp_scale_widths(0, ctypes.byref(q), ctypes.byref(k)) == EINVAL
    assert b"n must be" in L.ulp_last_error()


def amax_call(L, dtype=0, B=1, Lq=128, H=4, D=64, rank=0, P=2, used=NONE, x=A, mean=A, out=A):
    return L.ulp_k_grouped_amax(x, mean, dtype, B, Lq, H, D, rank, P, used, out, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dtype=2), EINVAL, b"dtype"),
    (dict(D=96), EUNSUPPORTED, b"head_dim"),
    (dict(P=3, H=6), EUNSUPPORTED, b"world_size"),
    (dict(P=16, H=16), EUNSUPPORTED, b"world_size"),
    (dict(rank=2), EINVAL, b"rank"),
    (dict(rank=-1), EINVAL, b"rank"),
    (dict(H=3), EINVAL, b"divisible"),
    (dict(B=0), EINVAL, b">= 1"),
    (dict(Lq=0), EINVAL, b">= 1"),
    (dict(used=0), EINVAL, b"used_sequence"),
    (dict(used=257), EINVAL, b"used_sequence"),
    (dict(used=-5), EINVAL, b"used_sequence"),
    (dict(x=0), EINVAL, b"NULL"),
    (dict(out=0), EINVAL, b"NULL"),
    (dict(x=A + 2), EALIGN, b"aligned"),
    (dict(mean=A + 8), EALIGN, b"aligned"),
    (dict(B=1 << 30, Lq=1 << 20), EINVAL, b"too large"),
])
def test_amax_validation(L, kw, code, msg):
    assert amax_call(L, **kw) == code
    assert msg in L.ulp_last_error()


def test_minmax_and_derive_validation(L):
    assert L.ulp_boundary_minmax(A, 0, 1, 128, 4, 128, 5, 4, NONE, A, None) == EINVAL
    assert L.ulp_boundary_minmax(A, 1, 1, 128, 4, 128, 0, 4, 513, A, None) == EINVAL
    assert L.ulp_boundary_minmax(A, 1, 1, 128, 4, 32, 0, 4, NONE, A, None) == EUNSUPPORTED
    assert L.ulp_derive_k_boundary_amax(0, A, A, 0, 1, 4, 64, 0, 128, 2, None) == EINVAL
    assert L.ulp_derive_k_boundary_amax(A, A + 4, A, 0, 1, 4, 64, 0, 128, 2, None) == EALIGN
    assert L.ulp_derive_k_boundary_amax(A, A, A, 0, 1, 5, 64, 0, 128, 2, None) == EINVAL


def test_pack_validation(L):
    cb = ulp.chunk_bytes(1, 128, 2, 64)
    args = [A, A, A, A, 0, A, A, None, 1, 128, 4, 64, 0, 2, A]
    assert L.ulp_pack(*args, cb + 16, None) == EALIGN
    assert b"multiple of 256" in L.ulp_last_error()
    assert L.ulp_pack(*args, cb - 256, None) == EINVAL
    assert b"smaller than the chunk" in L.ulp_last_error()
    bad = list(args)
    bad[3] = 0                      # k_mean is required by pack
    assert L.ulp_pack(*bad, cb, None) == EINVAL
    bad = list(args)
    bad[7] = A + 4                  # an optional V scale must be aligned like every tensor
    assert L.ulp_pack(*bad, cb, None) == EALIGN and b"v_scale" in L.ulp_last_error()


def test_unpack_validation(L):
    def call(B=1, Lq=100, h=2, D=64, P=2, aligned=NONE, ss=NONE):
        return L.ulp_unpack_for_sage(A, B, Lq, h, D, P, aligned, ss, A, A, A, A, A, None)
    assert call(aligned=1) == EINVAL and b"aligned=True" in L.ulp_last_error()
    assert call(aligned=2) == EINVAL
    assert call(ss=201) == EINVAL and b"scale_sequence" in L.ulp_last_error()
    assert call(ss=0) == EINVAL
    assert call(h=0) == EINVAL
    assert call(D=256) == EUNSUPPORTED
    assert call(P=5) == EUNSUPPORTED
    assert L.ulp_unpack_for_sage(A, 1, 128, 2, 64, 2, 1, NONE, A, A, A + 1, A, A, None) == EALIGN


def test_group_validation(L):
    assert L.ulp_group_stats(A, A, 0, 0, 1, 128, 4, 64, 2, NONE, A, A, A, A, None) == EINVAL
    assert L.ulp_group_derive(A, A, A, A, A, 0, 1, 4, 64, 128, 3, None) == EUNSUPPORTED
    assert L.ulp_group_pack(A, A, A, A, 0, A, A, None, 1, 128, 3, 64, 2, A, None) == EINVAL
    assert L.ulp_group_pack(A, A, A, A, 0, A, A, A + 8, 1, 128, 4, 64, 2, A, None) == EALIGN
    assert L.ulp_group_unpack(A, 1, 100, 2, 64, 2, 1, NONE, A, A, A, A, A, None) == EINVAL



def test_one_read_validation(L):
    cb = ulp.chunk_bytes(1, 128, 2, 64)
    # ulp_stats_pack(q, k, v, mean, dtype, v_scale, B, L, H, D, rank, P, used, qa, ka, qm, km,
    #                send, dest_stride, stream)
    sp = [A, A, A, A, 0, None, 1, 128, 4, 64, 0, 2, NONE, A, A, A, A, A]
    assert L.ulp_stats_pack(*sp, cb + 16, None) == EALIGN
    assert L.ulp_stats_pack(*sp, cb - 256, None) == EINVAL
    bad = list(sp); bad[10] = 2                       # rank outside [0, P)
    assert L.ulp_stats_pack(*bad, cb, None) == EINVAL and b"rank" in L.ulp_last_error()
    bad = list(sp); bad[12] = 257                     # used_sequence > S
    assert L.ulp_stats_pack(*bad, cb, None) == EINVAL and b"used_sequence" in L.ulp_last_error()
    bad = list(sp); bad[2] = 0                        # v is required
    assert L.ulp_stats_pack(*bad, cb, None) == EINVAL and b"v is NULL" in L.ulp_last_error()
    bad = list(sp); bad[15] = A + 4                   # a min/max output misaligned
    assert L.ulp_stats_pack(*bad, cb, None) == EALIGN
    bad = list(sp); bad[5] = A + 8                    # optional V scale misaligned
    assert L.ulp_stats_pack(*bad, cb, None) == EALIGN and b"v_scale" in L.ulp_last_error()
    bad = list(sp); bad[9] = 96
    assert L.ulp_stats_pack(*bad, cb, None) == EUNSUPPORTED
    # ulp_derive_pack(q, k, mean, dtype, qa, ka, qm, km, B, L, H, D, rank, P, used, send,
    #                 stride, stream)
    pd = [A, A, A, 0, A, A, A, A, 1, 128, 4, 64, 0, 2, NONE, A]
    assert L.ulp_derive_pack(*pd, cb + 256 + 16, None) == EALIGN
    bad = list(pd); bad[2] = 0                        # k_mean is required
    assert L.ulp_derive_pack(*bad, cb, None) == EINVAL and b"k_mean" in L.ulp_last_error()
    bad = list(pd); bad[7] = 0                        # the gathered K min/max is required
    assert L.ulp_derive_pack(*bad, cb, None) == EINVAL and b"k_minmax" in L.ulp_last_error()
    bad = list(pd); bad[13] = 3
    assert L.ulp_derive_pack(*bad, cb, None) == EUNSUPPORTED
    # group forms
    assert L.ulp_group_stats_pack(A, A, A, A, 0, None, 1, 128, 3, 64, 2, NONE, A, A, A, A, A,
                                  None) == EINVAL          # heads not divisible by P
    assert L.ulp_group_stats_pack(A, A, A, A, 2, None, 1, 128, 4, 64, 2, NONE, A, A, A, A, A,
                                  None) == EINVAL          # dtype
    assert L.ulp_group_stats_pack(A, A, A, A, 0, None, 1, 128, 4, 64, 2, 0, A, A, A, A, A,
                                  None) == EINVAL          # used 0
    assert L.ulp_group_derive_pack(A, A, A, 0, A, 0, A, A, 1, 128, 4, 64, 2, NONE, A,
                                   None) == EINVAL         # k_amax NULL
    assert L.ulp_group_derive_pack(A, A, A, 0, A, A, A, A, 1, 128, 4, 64, 2, NONE, A + 8,
                                   None) == EALIGN         # group misaligned


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """The binding has no fallback: without libulp.so every call raises."""
    monkeypatch.setattr(ulp, "_lib", None)
    monkeypatch.setattr(ulp, "LIB_PATH", str(tmp_path / "libulp.so"))
    with pytest.raises(RuntimeError, match="missing"):
        ulp.slots(100)


def test_k_mean_validation(L):
    # workspace size: 8 * B * H * D * ceil(used / R); small shapes take R = 32 rows
    assert L.ulp_k_mean_workspace_bytes(2, 100, 4, 64, 2, NONE) == 8 * 2 * 4 * 64 * 7
    assert L.ulp_k_mean_workspace_bytes(1, 1000, 4, 128, 4, NONE) == 8 * 4 * 128 * 125
    assert L.ulp_k_mean_workspace_bytes(1, 1000, 4, 128, 4, 257) == 8 * 4 * 128 * 9
    # a long sequence over many heads takes taller chunks, never more than 512 rows
    big = L.ulp_k_mean_workspace_bytes(1, 9360, 40, 128, 8, 74000)
    assert 8 * 40 * 128 * -(-74000 // 512) <= big <= 8 * 40 * 128 * -(-74000 // 32)
    assert L.ulp_k_mean_workspace_bytes(1, 100, 4, 64, 2, 201) == 0
    assert L.ulp_k_mean_workspace_bytes(0, 100, 4, 64, 2, NONE) == 0

    need = L.ulp_k_mean_workspace_bytes(1, 128, 4, 64, 2, NONE)

    def call(dtype=0, B=1, Lq=128, H=4, D=64, P=2, used=NONE, k=A, ws=A, wsb=need, mf=A,
             md=A):
        return L.ulp_k_mean(k, dtype, B, Lq, H, D, P, used, ws, wsb, mf, md, None)
    assert call(wsb=need - 8) == EINVAL and b"workspace" in L.ulp_last_error()
    assert call(used=257) == EINVAL and b"used_sequence" in L.ulp_last_error()
    assert call(D=32) == EUNSUPPORTED
    assert call(H=3) == EINVAL
    assert call(k=0) == EINVAL
    assert call(mf=A + 4) == EALIGN
    assert call(md=A + 2) == EALIGN
    assert call(ws=0) == EINVAL
    assert call(B=70000, wsb=1 << 40) == EINVAL and b"too large" in L.ulp_last_error()


def test_k_mean_noalloc_rejects_shapes_beyond_its_scratch(L):
    """The entry point without a workspace argument takes at most 16 MiB of the library's
    own scratch; a larger need is an argument error, found before any device call."""
    # B=1, H=64, D=128, used = 2 * 131072: at most 512 rows per partial sum, so 512 partial
    # rows of 8 * 64 * 128 bytes = 32 MiB
    need = L.ulp_k_mean_workspace_bytes(1, 131072, 64, 128, 2, NONE)
    assert need > 16 * 2 ** 20
    f = ctypes.c_void_p(A)
    assert L.ulp_k_mean_noalloc(f, 0, 1, 131072, 64, 128, 2, NONE, f, f, None) == EINVAL
    assert b"scratch" in L.ulp_last_error()
    assert L.ulp_k_mean_noalloc(f, 0, 1, 100, 4, 96, 2, NONE, f, f, None) == EUNSUPPORTED
    assert L.ulp_k_mean_noalloc(f, 0, 1, 100, 4, 64, 2, 201, f, f, None) == EINVAL


def test_consumer_validation(L):
    def call(B=1, S=128, h=2, D=64, W=2, used=128, v=None):
        return L.ulp_consumer_attention(A, A, A, A, A, v, B, S, h, D, W, used, A, None)
    assert call(D=96) == EUNSUPPORTED
    assert call(used=0) == EINVAL and b"used" in L.ulp_last_error()
    assert call(used=129) == EINVAL
    assert call(W=1) == EINVAL and b"scale width" in L.ulp_last_error()
    assert call(h=0) == EINVAL
    assert call(v=A + 4) == EALIGN
    assert L.ulp_consumer_attention(A, 0, A, A, A, None, 1, 128, 2, 64, 2, 128, A, None) == EINVAL
    # one batch entry of k8 / v8 must stay below 2 GiB (32-bit offsets inside the kernel):
    # S * h * D = 2^31 exactly is refused
    S = 2 ** 31 // (64 * 128)
    assert call(S=S, h=64, D=128, W=S // 64, used=S) == EINVAL
    assert b"2 GiB" in L.ulp_last_error()


def test_stats_with_mean_validation(L):
    need = L.ulp_group_stats_with_mean_workspace_bytes(1, 128, 4, 64, 2)
    assert need == 2 * 1 * 4 * 2 * 64 * 12          # P*B*H*slots*D*(8 + 2*2)

    def call(dtype=0, B=1, Lq=128, H=4, D=64, P=2, used=NONE, ws=A, wsb=need, md=A):
        return L.ulp_group_stats_with_mean(A, A, dtype, B, Lq, H, D, P, used, ws, wsb, A, A,
                                           A, A, A, md, None)
    assert call(wsb=need - 1) == EINVAL and b"workspace" in L.ulp_last_error()
    assert call(md=0) == EINVAL
    assert call(D=96) == EUNSUPPORTED
    assert call(used=300) == EINVAL
    assert call(ws=A + 8) == EALIGN


def test_page_signatures_are_accepted():
    """The Python functions take the keyword arguments the three API pages list (plus an
    optional ``out``), so calls written against the pages run unchanged."""
    import inspect
    pages = {
        "k_grouped_amax": (["k", "k_mean_global"],
                           ["rank", "world_size", "used_sequence", "enable_pdl"]),
        "derive_k_boundary_amax": (["grouped_amax", "gathered_minmax", "k_mean_global"],
                                   ["rank", "local_sequence", "world_size"]),
        "unpack_for_sage": (["recv_u8"],
                            ["batch_size", "local_sequence", "local_heads", "head_dim",
                             "world_size", "aligned", "scale_sequence", "out", "enable_pdl"]),
    }
    for name, (positional, keywords) in pages.items():
        sig = inspect.signature(getattr(ulp, name))
        params = sig.parameters
        got_pos = [n for n, p in params.items()
                   if p.kind == inspect.Parameter.POSITIONAL_OR_KEYWORD]
        assert got_pos == positional, name
        for kw in keywords:
            assert kw in params and params[kw].kind == inspect.Parameter.KEYWORD_ONLY, (name, kw)
        for n, p in params.items():        # everything beyond the pages is optional
            if n not in positional and n not in keywords:
                assert p.default is not inspect.Parameter.empty, (name, n)
