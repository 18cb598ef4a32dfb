"""C ABI of libmaxsim.so on a host without a GPU.

Checks that the library loads, exports every function include/maxsim.h
declares with the argument count the binding uses, and that host-side
validation returns the documented status codes.  Only invalid or empty
arguments are passed: validation rejects them before any HIP call, so no
device work is attempted.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "maxsim.h")
LIB = os.path.join(ROOT, "late_interaction_retrieval_amd", "libmaxsim.so")


def _ensure_built():
    if not os.path.exists(LIB):
        from late_interaction_retrieval_amd import build
        build.build()


_ensure_built()
from late_interaction_retrieval_amd import binding as bd  # noqa: E402

L = bd.lib()
A = ctypes.c_void_p(0x10000)  # aligned non-null fake pointers: never dereferenced
M = ctypes.c_void_p(0x10001)  # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(maxsim_\w+)\s*\(([^)]*)\)\s*;", text, flags=re.M):
        params = [p for p in m.group(2).split(",") if p.strip() and p.strip() != "void"]
        out[m.group(1)] = len(params)
    return out


def test_every_declared_symbol_is_exported_with_binding_arity():
    decl = declared_functions()
    assert set(decl) == {"maxsim_fwd", "maxsim_fwd_varlen", "maxsim_fwd_i8", "maxsim_bwd_workspace_bytes",
                         "maxsim_bwd", "maxsim_status_string", "maxsim_fwd_pairs", "maxsim_topk",
                         "maxsim_two_stage_workspace_bytes", "maxsim_two_stage_topk",
                         "maxsim_bwd_varlen_workspace_bytes", "maxsim_bwd_varlen", "maxsim_bwd_scatter",
                         "maxsim_bwd_prefer_scatter", "maxsim_bwd_scatter_workspace_bytes",
                         "maxsim_fwd_host_stream_staging_bytes", "maxsim_fwd_host_stream",
                         "maxsim_chamfer_fwd_workspace_bytes", "maxsim_chamfer_fwd",
                         "maxsim_chamfer_bwd_workspace_bytes", "maxsim_chamfer_bwd",
                         "maxsim_bwd_noalloc_scratch_bytes", "maxsim_bwd_noalloc"}
    raw = ctypes.CDLL(LIB)
    for name, nargs in decl.items():
        assert hasattr(raw, name), name
        assert len(bd.SIGNATURES[name][1]) == nargs, name


def fwd(**kw):
    a = dict(Q=A, D=A, d_lens=None, Nq=2, Lq=32, B=3, Ld=10, d=128, dt=0, scores=A, argmax=A, stream=None)
    a.update(kw)
    return L.maxsim_fwd(a["Q"], a["D"], a["d_lens"], a["Nq"], a["Lq"], a["B"], a["Ld"], a["d"], a["dt"],
                        a["scores"], a["argmax"], a["stream"])


def fwd_varlen(**kw):
    a = dict(Q=A, D=A, cu=A, Nq=2, Lq=32, B=3, T=100, maxld=50, d=128, dt=1, scores=A, argmax=None,
             stream=None)
    a.update(kw)
    return L.maxsim_fwd_varlen(a["Q"], a["D"], a["cu"], a["Nq"], a["Lq"], a["B"], a["T"], a["maxld"], a["d"],
                               a["dt"], a["scores"], a["argmax"], a["stream"])


def fwd_i8(**kw):
    a = dict(Q=A, qs=A, D=A, ds=A, cu=A, Nq=2, Lq=32, B=3, T=100, maxld=50, d=128, scores=A, argmax=A,
             stream=None)
    a.update(kw)
    return L.maxsim_fwd_i8(a["Q"], a["qs"], a["D"], a["ds"], a["cu"], a["Nq"], a["Lq"], a["B"], a["T"],
                           a["maxld"], a["d"], a["scores"], a["argmax"], a["stream"])


def bwd(**kw):
    a = dict(Q=A, D=A, dt=0, A=A, g=A, Nq=4, Lq=32, B=5, Ld=64, d=128, dQ=A, dD=A, rp=A, ci=A, ws=A,
             wsb=1 << 30, stream=None)
    a.update(kw)
    return L.maxsim_bwd(a["Q"], a["D"], a["dt"], a["A"], a["g"], a["Nq"], a["Lq"], a["B"], a["Ld"], a["d"],
                        a["dQ"], a["dD"], a["rp"], a["ci"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), bd.MAXSIM_ERR_NULL), (dict(D=None), bd.MAXSIM_ERR_NULL),
    (dict(scores=None), bd.MAXSIM_ERR_NULL),
    (dict(Lq=0), bd.MAXSIM_ERR_SHAPE), (dict(Nq=-1), bd.MAXSIM_ERR_SHAPE), (dict(B=-2), bd.MAXSIM_ERR_SHAPE),
    (dict(Ld=0), bd.MAXSIM_ERR_SHAPE),
    (dict(d=64), bd.MAXSIM_ERR_UNSUPPORTED), (dict(Lq=1025), bd.MAXSIM_ERR_UNSUPPORTED),
    (dict(dt=7), bd.MAXSIM_ERR_UNSUPPORTED),
    (dict(Q=M), bd.MAXSIM_ERR_ALIGN), (dict(D=M), bd.MAXSIM_ERR_ALIGN), (dict(scores=M), bd.MAXSIM_ERR_ALIGN),
    (dict(argmax=M), bd.MAXSIM_ERR_ALIGN), (dict(d_lens=M), bd.MAXSIM_ERR_ALIGN),
    (dict(Nq=0, Q=None), bd.MAXSIM_OK), (dict(B=0, D=None), bd.MAXSIM_OK),
])
def test_fwd_validation(kw, code):
    assert fwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), bd.MAXSIM_ERR_NULL), (dict(D=None), bd.MAXSIM_ERR_NULL),
    (dict(D=None, T=0), bd.MAXSIM_ERR_ALIGN),  # D may be NULL when T == 0; argmax/cu still checked
    (dict(T=-1), bd.MAXSIM_ERR_SHAPE), (dict(maxld=0), bd.MAXSIM_ERR_SHAPE),
    (dict(dt=2), bd.MAXSIM_ERR_UNSUPPORTED), (dict(d=256), bd.MAXSIM_ERR_UNSUPPORTED),
    (dict(cu=M), bd.MAXSIM_ERR_ALIGN), (dict(Q=M), bd.MAXSIM_ERR_ALIGN),
    (dict(B=0), bd.MAXSIM_OK),
])
def test_fwd_varlen_validation(kw, code):
    if kw.get("T") == 0:
        kw = dict(kw, cu=M)
    assert fwd_varlen(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(qs=None), bd.MAXSIM_ERR_NULL), (dict(ds=None), bd.MAXSIM_ERR_NULL), (dict(cu=None), bd.MAXSIM_ERR_NULL),
    (dict(Lq=-3), bd.MAXSIM_ERR_SHAPE), (dict(T=-5), bd.MAXSIM_ERR_SHAPE),
    (dict(d=127), bd.MAXSIM_ERR_UNSUPPORTED), (dict(Lq=4096), bd.MAXSIM_ERR_UNSUPPORTED),
    (dict(Q=M), bd.MAXSIM_ERR_ALIGN), (dict(ds=M), bd.MAXSIM_ERR_ALIGN), (dict(qs=M), bd.MAXSIM_ERR_ALIGN),
    (dict(Nq=0), bd.MAXSIM_OK),
])
def test_fwd_i8_validation(kw, code):
    assert fwd_i8(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), bd.MAXSIM_ERR_NULL), (dict(ws=None), bd.MAXSIM_ERR_NULL), (dict(ci=None), bd.MAXSIM_ERR_NULL),
    (dict(Nq=0), bd.MAXSIM_ERR_SHAPE), (dict(Ld=0), bd.MAXSIM_ERR_SHAPE),
    (dict(Nq=1 << 15, B=1 << 10, Lq=1 << 6), bd.MAXSIM_ERR_SHAPE),  # Nq*B*Lq >= 2^31
    (dict(Ld=5000), bd.MAXSIM_ERR_UNSUPPORTED), (dict(d=96), bd.MAXSIM_ERR_UNSUPPORTED),
    (dict(dt=3), bd.MAXSIM_ERR_UNSUPPORTED),
    (dict(dQ=M), bd.MAXSIM_ERR_ALIGN), (dict(ws=M), bd.MAXSIM_ERR_ALIGN), (dict(g=M), bd.MAXSIM_ERR_ALIGN),
    (dict(wsb=0), bd.MAXSIM_ERR_WORKSPACE),
])
def test_bwd_validation(kw, code):
    assert bwd(**kw) == code


def test_workspace_bytes():
    # one int32 count per (document, group of queries, row); one total per (document, group);
    # the documents' first slots (B + 1); the heavy-row list: a count and room for every row
    # that can hold more than 512 of the 64*64*1024 sources; each part at a 256-byte boundary
    n = L.maxsim_bwd_workspace_bytes(64, 64, 1024, 1024)
    heavy = (1 + 64 * 64 * 1024 // 513) * 4
    up = lambda x: (x + 255) // 256 * 256
    # Ld = 1024 -> groups of 16 queries (16 * 1024 slots), 4 groups per document
    assert n == 64 * 4 * 1024 * 4 + up(64 * 4 * 4) + up(65 * 4) + up(heavy)
    assert L.maxsim_bwd_workspace_bytes(0, 1, 1, 1) == 0
    assert L.maxsim_bwd_workspace_bytes(1, 1, 1, 5000) == 0
    assert bwd(wsb=n - 1, Nq=64, B=64, Lq=1024, Ld=1024) == bd.MAXSIM_ERR_WORKSPACE


def test_status_strings():
    for code in range(8):
        s = L.maxsim_status_string(code).decode()
        assert s.startswith("MAXSIM_")
    assert "unknown" in L.maxsim_status_string(99).decode()


def test_pairs_topk_two_stage_validation():
    ok, NULL, SHAPE, UNSUP, ALIGN, WS = (bd.MAXSIM_OK, bd.MAXSIM_ERR_NULL, bd.MAXSIM_ERR_SHAPE,
                                         bd.MAXSIM_ERR_UNSUPPORTED, bd.MAXSIM_ERR_ALIGN, bd.MAXSIM_ERR_WORKSPACE)
    # pairs: Q, D, cu, dtype, pq, pb, P, Nq, Lq, B, T, d, scores, argmax, stream
    assert L.maxsim_fwd_pairs(A, A, A, 0, A, A, 0, 2, 32, 3, 10, 128, A, None, None) == ok  # P = 0: nothing
    assert L.maxsim_fwd_pairs(A, A, A, 0, A, A, -1, 2, 32, 3, 10, 128, A, None, None) == SHAPE
    assert L.maxsim_fwd_pairs(A, A, A, 0, A, A, 4, 2, 1025, 3, 10, 128, A, None, None) == UNSUP
    assert L.maxsim_fwd_pairs(A, A, A, 0, A, A, 4, 2, 32, 3, 10, 64, A, None, None) == UNSUP
    assert L.maxsim_fwd_pairs(A, A, A, 2, A, A, 4, 2, 32, 3, 10, 128, A, None, None) == UNSUP
    assert L.maxsim_fwd_pairs(A, A, A, 0, None, A, 4, 2, 32, 3, 10, 128, A, None, None) == NULL
    assert L.maxsim_fwd_pairs(M, A, A, 0, A, A, 4, 2, 32, 3, 10, 128, A, None, None) == ALIGN
    # topk: scores, ids, Nq, B, K, idx, val, stream
    assert L.maxsim_topk(A, None, 2, 10, 11, A, A, None) == SHAPE
    assert L.maxsim_topk(A, None, 2, 10, 0, A, A, None) == SHAPE
    assert L.maxsim_topk(A, None, 2, 5000, 1025, A, A, None) == UNSUP
    assert L.maxsim_topk(A, None, 0, 10, 3, A, A, None) == ok
    assert L.maxsim_topk(None, None, 2, 10, 3, A, A, None) == NULL
    assert L.maxsim_topk(A, M, 2, 10, 3, A, A, None) == ALIGN
    # two-stage: workspace size and argument checks happen before any launch
    need = L.maxsim_two_stage_workspace_bytes(2, 10, 4)
    assert need == 256 + 256 + 2 * 4 * 4
    assert L.maxsim_two_stage_workspace_bytes(0, 10, 4) == 0
    args = lambda K1, K2, ws, nbytes: L.maxsim_two_stage_topk(A, A, A, A, A, A, A, 0, 2, 32, 10, 100, 20, 128,
                                                              K1, K2, A, A, A, A, ws, nbytes, None)
    assert args(4, 5, A, need) == SHAPE
    assert args(11, 2, A, need) == SHAPE
    assert args(4, 2, A, need - 1) == WS
    assert args(4, 2, ctypes.c_void_p(0x10010), need) == ALIGN
    assert args(4, 2, None, need) == NULL


def bwd_varlen(**kw):
    a = dict(Q=A, D=A, cu=A, dt=1, A=A, g=A, Nq=4, Lq=32, B=5, T=300, maxld=64, d=128, dQ=A, dD=A, rp=A, ci=A,
             ws=A, wsb=1 << 30, stream=None)
    a.update(kw)
    return L.maxsim_bwd_varlen(a["Q"], a["D"], a["cu"], a["dt"], a["A"], a["g"], a["Nq"], a["Lq"], a["B"],
                               a["T"], a["maxld"], a["d"], a["dQ"], a["dD"], a["rp"], a["ci"], a["ws"], a["wsb"],
                               a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), bd.MAXSIM_ERR_NULL), (dict(cu=None), bd.MAXSIM_ERR_NULL), (dict(A=None), bd.MAXSIM_ERR_NULL),
    (dict(D=None), bd.MAXSIM_ERR_NULL), (dict(dD=None), bd.MAXSIM_ERR_NULL), (dict(ws=None), bd.MAXSIM_ERR_NULL),
    (dict(Nq=0), bd.MAXSIM_ERR_SHAPE), (dict(B=0), bd.MAXSIM_ERR_SHAPE), (dict(T=-1), bd.MAXSIM_ERR_SHAPE),
    (dict(maxld=0), bd.MAXSIM_ERR_SHAPE), (dict(T=1 << 31), bd.MAXSIM_ERR_SHAPE),
    (dict(Nq=1 << 16, B=1 << 10, Lq=32), bd.MAXSIM_ERR_SHAPE),
    (dict(maxld=4097), bd.MAXSIM_ERR_UNSUPPORTED), (dict(d=64), bd.MAXSIM_ERR_UNSUPPORTED),
    (dict(Lq=1025), bd.MAXSIM_ERR_UNSUPPORTED), (dict(dt=2), bd.MAXSIM_ERR_UNSUPPORTED),
    (dict(Q=M), bd.MAXSIM_ERR_ALIGN), (dict(dD=M), bd.MAXSIM_ERR_ALIGN),
    (dict(ws=ctypes.c_void_p(0x10010)), bd.MAXSIM_ERR_ALIGN),
    (dict(wsb=0), bd.MAXSIM_ERR_WORKSPACE),
])
def test_bwd_varlen_validation(kw, code):
    assert bwd_varlen(**kw) == code


def test_bwd_varlen_workspace_bytes():
    # the counts for max_Ld, the per-document first slots, the heavy-row list (1 + 32000 // 513
    # entries), then the dQ chunk sums, each at a 256-byte boundary.  320 query rows fill 10
    # gather workgroups, so the 100 documents are split into min(ceil(512 / 10), 100 // 8) = 12
    # chunks for dQ.
    counts = 100 * 2 * 100 * 4  # 10 short queries form two groups of 8 at Ld = 100
    part = 12 * 320 * 128 * 4
    # counts, group totals (200), document first slots (101), heavy list, dQ chunks
    assert L.maxsim_bwd_workspace_bytes(10, 100, 32, 100) == 80128 + 1024 + 512 + 256 + part
    assert L.maxsim_bwd_varlen_workspace_bytes(10, 100, 32, 100) == 80128 + 1024 + 512 + 256 + part
    assert counts <= 80128 < counts + 256
    assert L.maxsim_bwd_scatter_workspace_bytes(10, 100, 32) == part
    assert L.maxsim_bwd_scatter_workspace_bytes(10, 7, 32) == 256  # too few documents to split
    assert L.maxsim_bwd_scatter_workspace_bytes(64, 64, 1024) == 256  # 65536 rows fill the chip: no split
    assert L.maxsim_bwd_varlen_workspace_bytes(0, 7, 32, 100) == 0
    assert L.maxsim_bwd_varlen_workspace_bytes(1, 1, 1, 5000) == 0
    n = L.maxsim_bwd_varlen_workspace_bytes(10, 7, 32, 100)
    assert bwd_varlen(wsb=n - 1, Nq=10, B=7, Lq=32, maxld=100) == bd.MAXSIM_ERR_WORKSPACE


def bwd_scatter(**kw):
    a = dict(Q=A, D=A, cu=None, dt=0, A=A, g=A, Nq=4, Lq=32, B=5, Ld=64, T=0, d=128, dQ=A, dD=A, ws=A,
             wsb=1 << 30, stream=None)
    a.update(kw)
    return L.maxsim_bwd_scatter(a["Q"], a["D"], a["cu"], a["dt"], a["A"], a["g"], a["Nq"], a["Lq"], a["B"],
                                a["Ld"], a["T"], a["d"], a["dQ"], a["dD"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), bd.MAXSIM_ERR_NULL), (dict(D=None), bd.MAXSIM_ERR_NULL), (dict(dD=None), bd.MAXSIM_ERR_NULL),
    (dict(A=None), bd.MAXSIM_ERR_NULL), (dict(g=None), bd.MAXSIM_ERR_NULL), (dict(dQ=None), bd.MAXSIM_ERR_NULL),
    (dict(Nq=0), bd.MAXSIM_ERR_SHAPE), (dict(Ld=0), bd.MAXSIM_ERR_SHAPE), (dict(cu=A, T=-1), bd.MAXSIM_ERR_SHAPE),
    (dict(cu=A, T=1 << 31), bd.MAXSIM_ERR_SHAPE), (dict(Nq=1 << 16, B=1 << 10, Lq=32), bd.MAXSIM_ERR_SHAPE),
    (dict(Ld=4097), bd.MAXSIM_ERR_UNSUPPORTED), (dict(d=64), bd.MAXSIM_ERR_UNSUPPORTED),
    (dict(dt=5), bd.MAXSIM_ERR_UNSUPPORTED), (dict(Lq=2000), bd.MAXSIM_ERR_UNSUPPORTED),
    (dict(D=M), bd.MAXSIM_ERR_ALIGN), (dict(cu=M, T=10), bd.MAXSIM_ERR_ALIGN), (dict(g=M), bd.MAXSIM_ERR_ALIGN),
    (dict(ws=None), bd.MAXSIM_ERR_NULL), (dict(ws=ctypes.c_void_p(0x10010)), bd.MAXSIM_ERR_ALIGN),
    (dict(wsb=255), bd.MAXSIM_ERR_WORKSPACE),
])
def test_bwd_scatter_validation(kw, code):
    assert bwd_scatter(**kw) == code


def test_bwd_dispatch_rule():
    """Scatter below the measured sources-per-row threshold, CSR above it."""
    assert L.maxsim_bwd_prefer_scatter(1, 32, 1000, 1000 * 180) == 1      # 0.18 sources per row
    assert L.maxsim_bwd_prefer_scatter(2, 32, 1000, 1000 * 180) == 1      # 0.36: scatter measured faster
    assert L.maxsim_bwd_prefer_scatter(4, 32, 1000, 1000 * 180) == 0      # 0.71: CSR measured faster
    assert L.maxsim_bwd_prefer_scatter(64, 1024, 64, 64 * 1024) == 0      # 64 per row (training)
    assert L.maxsim_bwd_prefer_scatter(0, 32, 10, 100) == 0
    assert L.maxsim_bwd_prefer_scatter(1, 32, 10, 0) == 0


def host_stream(**kw):
    a = dict(Q=A, D=A, cuh=None, cu=None, lens=None, Nq=2, Lq=32, B=10, Ld=64, d=128, dt=0, blk=4, st=A,
             stb=1 << 40, scores=A, argmax=None, stream=None)
    a.update(kw)
    return L.maxsim_fwd_host_stream(a["Q"], a["D"], a["cuh"], a["cu"], a["lens"], a["Nq"], a["Lq"], a["B"],
                                    a["Ld"], a["d"], a["dt"], a["blk"], a["st"], a["stb"], a["scores"],
                                    a["argmax"], a["stream"])


def test_host_stream_staging_bytes():
    # two D blocks, the block's scores, its cu_seqlens [+ its argmax], each at a 256-byte boundary
    n = L.maxsim_fwd_host_stream_staging_bytes(2, 32, 64, 4, 0)
    assert n == 2 * (4 * 64 * 256) + 256 + 256
    assert L.maxsim_fwd_host_stream_staging_bytes(2, 32, 64, 4, 1) == n + 1024
    assert L.maxsim_fwd_host_stream_staging_bytes(0, 32, 64, 4, 0) == 0
    assert L.maxsim_fwd_host_stream_staging_bytes(2, 32, 64, 0, 0) == 0
    assert L.maxsim_fwd_host_stream_staging_bytes(2, 1025, 64, 4, 0) == 0


def test_host_stream_validation():
    """Every rejection happens on the host before any HIP call (the host
    cu_seqlens is read here, so it is a real array)."""
    cu_ok = (ctypes.c_int32 * 4)(0, 10, 10, 70)
    cu_long = (ctypes.c_int32 * 4)(0, 10, 75, 80)   # a document longer than Ld = 64
    cu_off = (ctypes.c_int32 * 4)(5, 10, 20, 30)    # does not start at 0
    cu_empty = (ctypes.c_int32 * 4)(0, 0, 0, 0)
    assert host_stream(Q=None) == bd.MAXSIM_ERR_NULL
    assert host_stream(D=None) == bd.MAXSIM_ERR_NULL
    assert host_stream(st=None) == bd.MAXSIM_ERR_NULL
    assert host_stream(cuh=cu_ok, B=3) == bd.MAXSIM_ERR_NULL  # device cu_seqlens missing
    assert host_stream(blk=0) == bd.MAXSIM_ERR_SHAPE
    assert host_stream(Ld=0) == bd.MAXSIM_ERR_SHAPE
    assert host_stream(cuh=cu_long, cu=A, B=3) == bd.MAXSIM_ERR_SHAPE
    assert host_stream(cuh=cu_off, cu=A, B=3) == bd.MAXSIM_ERR_SHAPE
    assert host_stream(cuh=cu_ok, cu=A, B=3, lens=A) == bd.MAXSIM_ERR_SHAPE
    assert host_stream(cuh=cu_ok, cu=A, B=3, D=None) == bd.MAXSIM_ERR_NULL
    assert host_stream(d=64) == bd.MAXSIM_ERR_UNSUPPORTED
    assert host_stream(dt=2) == bd.MAXSIM_ERR_UNSUPPORTED
    assert host_stream(st=ctypes.c_void_p(0x10010)) == bd.MAXSIM_ERR_ALIGN
    assert host_stream(D=M) == bd.MAXSIM_ERR_ALIGN
    assert host_stream(stb=1000) == bd.MAXSIM_ERR_WORKSPACE
    assert host_stream(Nq=0) == bd.MAXSIM_OK
    assert host_stream(B=0) == bd.MAXSIM_OK
    # an empty packed corpus may pass no host rows; this still needs staging
    assert host_stream(cuh=cu_empty, cu=A, B=3, D=None, stb=0) == bd.MAXSIM_ERR_WORKSPACE


def test_chamfer_validation():
    big = 1 << 40
    fwd = lambda **kw: L.maxsim_chamfer_fwd(*[kw.get(k, v) for k, v in (
        ("P", A), ("Q", A), ("Bt", 2), ("N", 10), ("M", 20), ("dp", A), ("ip", A), ("dq", A), ("iq", A),
        ("ws", A), ("wsb", big), ("stream", None))])
    assert fwd(Bt=-1) == bd.MAXSIM_ERR_SHAPE
    assert fwd(Bt=1 << 16, N=1 << 15) == bd.MAXSIM_ERR_SHAPE
    assert fwd(P=None) == bd.MAXSIM_ERR_NULL
    assert fwd(iq=None) == bd.MAXSIM_ERR_NULL
    assert fwd(ws=None) == bd.MAXSIM_ERR_NULL
    assert fwd(P=M) == bd.MAXSIM_ERR_ALIGN
    assert fwd(ws=ctypes.c_void_p(0x10010)) == bd.MAXSIM_ERR_ALIGN
    assert fwd(wsb=0, N=100000, M=100000, Bt=1) == bd.MAXSIM_ERR_WORKSPACE
    assert fwd(Bt=0) == bd.MAXSIM_OK
    assert fwd(N=0, M=0) == bd.MAXSIM_OK
    bwd_ = lambda **kw: L.maxsim_chamfer_bwd(*[kw.get(k, v) for k, v in (
        ("P", A), ("Q", A), ("ip", A), ("iq", A), ("gp", A), ("gq", A), ("Bt", 2), ("N", 10), ("M", 20),
        ("dP", A), ("dQ", A), ("rpp", A), ("cip", A), ("rpq", A), ("ciq", A), ("ws", A), ("wsb", big),
        ("stream", None))])
    assert bwd_(N=-1) == bd.MAXSIM_ERR_SHAPE
    # both directions are sorted together: Bt*(N+M) must stay below 2^31
    # even when Bt*N and Bt*M each do (the forward accepts these sizes)
    assert bwd_(Bt=1, N=(1 << 31) - 10, M=20) == bd.MAXSIM_ERR_SHAPE
    assert bwd_(Bt=2, N=(1 << 30) - 1, M=2) == bd.MAXSIM_ERR_SHAPE
    assert L.maxsim_chamfer_bwd_workspace_bytes(1, (1 << 31) - 10, 20) == 0
    assert fwd(Bt=1, N=(1 << 31) - 10, M=20, wsb=big) != bd.MAXSIM_ERR_SHAPE
    assert bwd_(gq=None) == bd.MAXSIM_ERR_NULL
    assert bwd_(rpq=None) == bd.MAXSIM_ERR_NULL
    assert bwd_(cip=None) == bd.MAXSIM_ERR_NULL
    assert bwd_(dP=M) == bd.MAXSIM_ERR_ALIGN
    assert bwd_(wsb=0) == bd.MAXSIM_ERR_WORKSPACE
    assert bwd_(Bt=0) == bd.MAXSIM_OK


def test_chamfer_workspace_bytes():
    # forward: chunk minima (fp32 + int32) of both directions side by side when the targets are
    # split; 100K x 100K splits each direction into 83 chunks
    assert L.maxsim_chamfer_fwd_workspace_bytes(1, 100000, 100000) == 2 * 83 * 100000 * 8
    assert L.maxsim_chamfer_fwd_workspace_bytes(1, 10, 20) == 256  # one chunk: no partials
    assert L.maxsim_chamfer_fwd_workspace_bytes(-1, 10, 20) == 0
    # backward: one sort of both clouds' points (keys and values twice plus 256 counters per
    # 2048-element tile), then the heavy-row list (a count and n // 257 rows)
    n = 10 + 3000
    assert L.maxsim_chamfer_bwd_workspace_bytes(1, 10, 3000) == 4 * ((n * 4 + 255) // 256 * 256) + 2 * 256 * 4 + 256


def test_bwd_noalloc_validation():
    """The allocation-free backward validates like maxsim_bwd (no workspace
    arguments) and refuses, before any HIP call, a shape whose workspace
    exceeds its fixed scratch."""
    cap = L.maxsim_bwd_noalloc_scratch_bytes()
    assert cap == 64 << 20

    def call(**kw):
        a = dict(Q=A, D=A, dt=1, am=A, g=A, Nq=4, Lq=32, B=3, Ld=50, d=128, dQ=A, dD=A, rp=A, ci=A, stream=None)
        a.update(kw)
        return L.maxsim_bwd_noalloc(a["Q"], a["D"], a["dt"], a["am"], a["g"], a["Nq"], a["Lq"], a["B"], a["Ld"],
                                    a["d"], a["dQ"], a["dD"], a["rp"], a["ci"], a["stream"])

    assert call(Nq=0) == bd.MAXSIM_ERR_SHAPE
    assert call(Nq=1 << 12, B=1 << 10, Lq=1 << 10) == bd.MAXSIM_ERR_SHAPE
    assert call(d=64) == bd.MAXSIM_ERR_UNSUPPORTED
    assert call(Ld=5000) == bd.MAXSIM_ERR_UNSUPPORTED
    assert call(dt=5) == bd.MAXSIM_ERR_UNSUPPORTED
    assert call(am=None) == bd.MAXSIM_ERR_NULL
    assert call(ci=None) == bd.MAXSIM_ERR_NULL
    assert call(Q=M) == bd.MAXSIM_ERR_ALIGN
    assert call(rp=M) == bd.MAXSIM_ERR_ALIGN
    # 100,000 documents of 180 rows: the workspace exceeds the scratch array
    assert L.maxsim_bwd_workspace_bytes(1, 100000, 32, 180) > cap
    assert call(Nq=1, B=100000, Ld=180) == bd.MAXSIM_ERR_SCRATCH
    assert L.maxsim_bwd_workspace_bytes(64, 64, 1024, 1024) <= cap  # the training step fits
    assert b"SCRATCH" in L.maxsim_status_string(bd.MAXSIM_ERR_SCRATCH)
