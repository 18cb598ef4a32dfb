"""ctypes wrapper over ``maxsim_oracle.c`` (test infrastructure only).

Arrays cross as numpy arrays; fp16 / bf16 tensors cross as their raw uint16
bit patterns so the C side decodes them exactly.  Every function mirrors one
C entry point; the passages of the paper each follows are cited in the C file.
"""
import ctypes
import os
import subprocess

import numpy as np

F16 = 0
BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "maxsim_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# Tests that plant mistakes in a copy of the oracle point this at the mutant.
_LIB_OVERRIDE = os.environ.get("MAXSIM_ORACLE_LIB")
_lib = None


def lib_path():
    return _LIB


def build(force=True):
    """Compile the oracle with gcc: -O2, OpenMP, no FMA contraction, no fast-math."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build()
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_fwd_padded.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P]
        lib.oracle_fwd_varlen.argtypes = [P, P, P, I, I, I, I, I, P, P, P]
        lib.oracle_fwd_i8.argtypes = [P, P, P, P, P, I, I, I, I, P, P]
        lib.oracle_sim_at.argtypes = [P, P, P, I, I, I, I, I, P, P]
        lib.oracle_csr_build.argtypes = [P, I, I, I, I, P, P]
        lib.oracle_bwd.argtypes = [P, P, I, P, P, I, I, I, I, I, P, P]
        lib.oracle_fwd_pairs.argtypes = [P, P, P, I, P, P, I, I, I, I, I, P, P]
        lib.oracle_topk.argtypes = [P, I, I, I, P, P]
        lib.oracle_csr_build_varlen.argtypes = [P, I, I, I, P, P, P]
        lib.oracle_bwd_varlen.argtypes = [P, P, P, I, P, P, I, I, I, I, P, P]
        lib.oracle_chamfer_nn.argtypes = [P, P, I, I, I, P, P]
        lib.oracle_chamfer_csr.argtypes = [P, I, I, I, P, P]
        lib.oracle_chamfer_bwd.argtypes = [P, P, I, I, I, P, P, P, P, P, P]
        for name in ("oracle_fwd_padded", "oracle_fwd_varlen", "oracle_fwd_i8", "oracle_sim_at",
                     "oracle_csr_build", "oracle_bwd", "oracle_num_threads", "oracle_fwd_pairs",
                     "oracle_topk", "oracle_csr_build_varlen", "oracle_bwd_varlen", "oracle_chamfer_nn",
                     "oracle_chamfer_csr", "oracle_chamfer_bwd"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _bits16(a):
    """fp16 arrays -> their uint16 bits; uint16 arrays (bf16 bits) pass through."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected float16 or uint16 (bf16 bits), got %s" % a.dtype)
    return a


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments (rc=%d)" % (what, rc))


def f16_to_f64(bits):
    lib = _load()
    return np.array([lib.oracle_f16_to_f64(int(b)) for b in np.asarray(bits).ravel()])


def bf16_to_f64(bits):
    lib = _load()
    return np.array([lib.oracle_bf16_to_f64(int(b)) for b in np.asarray(bits).ravel()])


def fwd_padded(Q, D, dtype, d_lens=None, want_rowmax=False):
    """Q [Nq, Lq, d], D [B, Ld, d] -> (scores fp64 [Nq, B], argmax int32 [Nq, B, Lq][, rowmax])."""
    Qb, Db = _bits16(Q), _bits16(D)
    Nq, Lq, d = Qb.shape
    B, Ld, d2 = Db.shape
    assert d == d2
    lens = None if d_lens is None else np.ascontiguousarray(d_lens, dtype=np.int32)
    scores = np.empty((Nq, B), np.float64)
    amax = np.empty((Nq, B, Lq), np.int32)
    rowmax = np.empty((Nq, B, Lq), np.float64) if want_rowmax else None
    rc = _load().oracle_fwd_padded(_p(Qb), _p(Db), _p(lens), dtype, Nq, Lq, B, Ld, d,
                                   _p(scores), _p(amax), _p(rowmax))
    _check(rc, "fwd_padded")
    return (scores, amax, rowmax) if want_rowmax else (scores, amax)


def fwd_varlen(Q, D_packed, cu_seqlens, dtype, want_rowmax=False):
    """Q [Nq, Lq, d], D_packed [T, d], cu_seqlens [B+1] -> (scores, argmax[, rowmax])."""
    Qb, Db = _bits16(Q), _bits16(D_packed)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    Nq, Lq, d = Qb.shape
    B = cu.shape[0] - 1
    assert Db.shape[1] == d and Db.shape[0] >= cu[-1]
    scores = np.empty((Nq, B), np.float64)
    amax = np.empty((Nq, B, Lq), np.int32)
    rowmax = np.empty((Nq, B, Lq), np.float64) if want_rowmax else None
    rc = _load().oracle_fwd_varlen(_p(Qb), _p(Db), _p(cu), dtype, Nq, Lq, B, d,
                                   _p(scores), _p(amax), _p(rowmax))
    _check(rc, "fwd_varlen")
    return (scores, amax, rowmax) if want_rowmax else (scores, amax)


def fwd_i8(Q, q_scale, D_packed, d_scale, cu_seqlens):
    """INT8 x INT8 forward -> (scores fp32 [Nq, B], argmax int32 [Nq, B, Lq])."""
    Q = np.ascontiguousarray(Q, dtype=np.int8)
    D_packed = np.ascontiguousarray(D_packed, dtype=np.int8)
    qs = np.ascontiguousarray(q_scale, dtype=np.float32)
    ds = np.ascontiguousarray(d_scale, dtype=np.float32)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    Nq, Lq, d = Q.shape
    B = cu.shape[0] - 1
    assert qs.shape == (Nq, Lq) and ds.shape[0] >= cu[-1] and D_packed.shape[1] == d
    scores = np.empty((Nq, B), np.float32)
    amax = np.empty((Nq, B, Lq), np.int32)
    rc = _load().oracle_fwd_i8(_p(Q), _p(qs), _p(D_packed), _p(ds), _p(cu), Nq, Lq, B, d,
                               _p(scores), _p(amax))
    _check(rc, "fwd_i8")
    return scores, amax


def sim_at(Q, D_packed, cu_seqlens, dtype, sel):
    """fp64 <Q[q,i], D[b, sel[q,b,i]]> for every (q, b, i); -inf where sel is out of range."""
    Qb, Db = _bits16(Q), _bits16(D_packed)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    Nq, Lq, d = Qb.shape
    B = cu.shape[0] - 1
    assert sel.shape == (Nq, B, Lq)
    out = np.empty((Nq, B, Lq), np.float64)
    _check(_load().oracle_sim_at(_p(Qb), _p(Db), _p(cu), dtype, Nq, Lq, B, d, _p(sel), _p(out)),
           "sim_at")
    return out


def csr_build(argmax, Ld):
    """argmax [Nq, B, Lq] -> (row_ptr int32 [B*Ld+1], col_idx int32 [row_ptr[-1]]).

    Negative entries (an empty document) select no row, so col_idx holds
    Nq*B*Lq entries only when every argmax is >= 0."""
    A = np.ascontiguousarray(argmax, dtype=np.int32)
    Nq, B, Lq = A.shape
    row_ptr = np.empty(B * Ld + 1, np.int32)
    col_idx = np.empty(Nq * B * Lq, np.int32)
    _check(_load().oracle_csr_build(_p(A), Nq, B, Lq, Ld, _p(row_ptr), _p(col_idx)), "csr_build")
    return row_ptr, col_idx[:row_ptr[-1]]


def bwd(Q, D, dtype, argmax, g):
    """Closed-form gradients -> (dQ fp64 [Nq, Lq, d], dD fp64 [B, Ld, d])."""
    Qb, Db = _bits16(Q), _bits16(D)
    A = np.ascontiguousarray(argmax, dtype=np.int32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    Nq, Lq, d = Qb.shape
    B, Ld, _ = Db.shape
    assert A.shape == (Nq, B, Lq) and g.shape == (Nq, B)
    dQ = np.empty((Nq, Lq, d), np.float64)
    dD = np.empty((B, Ld, d), np.float64)
    _check(_load().oracle_bwd(_p(Qb), _p(Db), dtype, _p(A), _p(g), Nq, Lq, B, Ld, d, _p(dQ), _p(dD)),
           "bwd")
    return dQ, dD


def num_threads():
    return int(_load().oracle_num_threads())


def fwd_pairs(Q, D_packed, cu_seqlens, dtype, pairs_q, pairs_b, want_argmax=True):
    """Scores (fp64) [and argmax [P, Lq]] of the listed (query, document) pairs."""
    Qb, Db = _bits16(Q), _bits16(D_packed)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    pq = np.ascontiguousarray(pairs_q, dtype=np.int32)
    pb = np.ascontiguousarray(pairs_b, dtype=np.int32)
    Nq, Lq, d = Qb.shape
    B = cu.shape[0] - 1
    P = pq.shape[0]
    assert pb.shape == (P,) and Db.shape[1] == d
    s = np.zeros(P, np.float64)
    a = np.zeros((P, Lq), np.int32) if want_argmax else None
    rc = _load().oracle_fwd_pairs(_p(Qb), _p(Db), _p(cu), dtype, _p(pq), _p(pb), P, Nq, Lq, B, d, _p(s), _p(a))
    _check(rc, "fwd_pairs")
    return (s, a) if want_argmax else s


def topk(scores, K):
    """Per query row of float32 scores: (indices [Nq, K], values [Nq, K]),
    best first, equal scores by ascending index."""
    sc = np.ascontiguousarray(scores, dtype=np.float32)
    Nq, B = sc.shape
    idx = np.zeros((Nq, K), np.int32)
    val = np.zeros((Nq, K), np.float32)
    rc = _load().oracle_topk(_p(sc), Nq, B, K, _p(idx), _p(val))
    _check(rc, "topk")
    return idx, val


def two_stage_topk(Q8, q_scale, D8, d_scale, Q16, D16, cu_seqlens, dtype, K1, K2):
    """The two-stage scan as a composition of the plain definitions: INT8 scores
    of every pair, each query's top-K1 candidates (oracle_topk), fp16/bf16
    scores of those candidates in fp64, their K2 best (a stable sort by
    descending score).  Returns (candidates [Nq, K1], their int8 scores,
    final documents [Nq, K2], final fp64 scores [Nq, K2])."""
    s8, _ = fwd_i8(Q8, q_scale, D8, d_scale, cu_seqlens)
    cand, cval = topk(s8, K1)
    Nq = cand.shape[0]
    pq = np.repeat(np.arange(Nq, dtype=np.int32), K1)
    s16 = fwd_pairs(Q16, D16, cu_seqlens, dtype, pq, cand.reshape(-1), want_argmax=False).reshape(Nq, K1)
    final = np.empty((Nq, K2), np.int32)
    fval = np.empty((Nq, K2), np.float64)
    for q in range(Nq):
        order = np.lexsort((cand[q], -s16[q]))[:K2]  # score descending, then document index
        final[q] = cand[q][order]
        fval[q] = s16[q][order]
    return cand, cval, final, fval


def csr_build_varlen(argmax, cu_seqlens):
    """argmax [Nq, B, Lq] over a packed corpus -> (row_ptr [T+1], col_idx [row_ptr[T]])."""
    A = np.ascontiguousarray(argmax, dtype=np.int32)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    Nq, B, Lq = A.shape
    T = int(cu[-1])
    row_ptr = np.empty(T + 1, np.int32)
    col_idx = np.empty(Nq * B * Lq, np.int32)
    _check(_load().oracle_csr_build_varlen(_p(A), Nq, B, Lq, _p(cu), _p(row_ptr), _p(col_idx)), "csr_build_varlen")
    return row_ptr, col_idx[:row_ptr[-1]]


def bwd_varlen(Q, D_packed, cu_seqlens, dtype, argmax, g):
    """Packed-corpus backward -> (dQ [Nq, Lq, d], dD [T, d]) in fp64."""
    Qb, Db = _bits16(Q), _bits16(D_packed)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    A = np.ascontiguousarray(argmax, dtype=np.int32)
    gg = np.ascontiguousarray(g, dtype=np.float32)
    Nq, Lq, d = Qb.shape
    B = cu.shape[0] - 1
    T = int(cu[-1])
    dQ = np.empty((Nq, Lq, d), np.float64)
    dD = np.empty((T, d), np.float64)
    _check(_load().oracle_bwd_varlen(_p(Qb), _p(Db), _p(cu), dtype, _p(A), _p(gg), Nq, Lq, B, d, _p(dQ), _p(dD)),
           "bwd_varlen")
    return dQ, dD


def _points(X):
    X = np.ascontiguousarray(X, dtype=np.float32)
    if X.ndim == 2:
        X = X[None]
    assert X.ndim == 3 and X.shape[2] == 3
    return X


def chamfer_nn(A, B):
    """For every point of A [Bt, Na, 3]: (squared distance to the nearest point of
    B [Bt, Nb, 3] in fp64 [Bt, Na], its first index int32 [Bt, Na]); batch items pair up."""
    A, B = _points(A), _points(B)
    Bt, Na, _ = A.shape
    assert B.shape[0] == Bt
    Nb = B.shape[1]
    dist = np.empty((Bt, Na), np.float64)
    idx = np.empty((Bt, Na), np.int32)
    _check(_load().oracle_chamfer_nn(_p(A), _p(B), Bt, Na, Nb, _p(dist), _p(idx)), "chamfer_nn")
    return dist, idx


def chamfer(P, Q):
    """Both directions: (dist_p, idx_p, dist_q, idx_q)."""
    dp, ip = chamfer_nn(P, Q)
    dq, iq = chamfer_nn(Q, P)
    return dp, ip, dq, iq


def chamfer_loss(P, Q):
    """The page's Chamfer distance per batch item: mean_p min_q |p-q|^2 + mean_q min_p |q-p|^2."""
    dp, _, dq, _ = chamfer(P, Q)
    return dp.mean(axis=1) + dq.mean(axis=1)


def chamfer_csr(idx, Nb):
    """Inverse map of a selection idx [Bt, Na] into Nb destinations per item:
    (row_ptr [Bt*Nb + 1], col_idx [row_ptr[-1]]) with global source ids b*Na + i."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    if idx.ndim == 1:
        idx = idx[None]
    Bt, Na = idx.shape
    row_ptr = np.empty(Bt * Nb + 1, np.int32)
    col_idx = np.empty(max(1, Bt * Na), np.int32)
    _check(_load().oracle_chamfer_csr(_p(idx), Bt, Na, Nb, _p(row_ptr), _p(col_idx)), "chamfer_csr")
    return row_ptr, col_idx[:row_ptr[-1]]


def chamfer_bwd(P, Q, idx_p, idx_q, gp, gq):
    """Gradients (dP [Bt, N, 3], dQ [Bt, M, 3], fp64) of sum gp*dist_p + sum gq*dist_q
    with the selections fixed."""
    P, Q = _points(P), _points(Q)
    Bt, N, _ = P.shape
    M = Q.shape[1]
    ip = np.ascontiguousarray(idx_p, dtype=np.int32).reshape(Bt, N)
    iq = np.ascontiguousarray(idx_q, dtype=np.int32).reshape(Bt, M)
    gp = np.ascontiguousarray(gp, dtype=np.float32).reshape(Bt, N)
    gq = np.ascontiguousarray(gq, dtype=np.float32).reshape(Bt, M)
    dP = np.empty((Bt, N, 3), np.float64)
    dQ = np.empty((Bt, M, 3), np.float64)
    _check(_load().oracle_chamfer_bwd(_p(P), _p(Q), Bt, N, M, _p(ip), _p(iq), _p(gp), _p(gq), _p(dP), _p(dQ)),
           "chamfer_bwd")
    return dP, dQ
