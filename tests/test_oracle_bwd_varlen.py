"""Pins for the oracle's packed-corpus (cu_seqlens) CSR build and backward
(test infrastructure; no GPU).

With every document the same length the packed layout is the padded one, so
both must equal the already-pinned padded oracle exactly.  Empty documents
must behave as if removed.  Independently: numpy scatter-add on tiny inputs,
Euler homogeneity <dQ, Q> = sum g * score = <dD, D> with the oracle forward's
own argmax, and the CSR invariants.
"""
import numpy as np
import pytest

import oracle
from late_interaction_retrieval_amd import inputs


def _rows(seed, n, dtn=inputs.F16):
    return inputs.random_rows(seed, n, 128, dtn)


def _dec(a, dtn):
    return a.astype(np.float64) if dtn == inputs.F16 else oracle.bf16_to_f64(a).reshape(a.shape)


@pytest.mark.parametrize("dtn", [inputs.F16, inputs.BF16])
def test_equal_lengths_reduce_to_padded(dtn):
    Nq, Lq, B, Ld = 3, 9, 5, 11
    Q = _rows(1, Nq * Lq, dtn).reshape(Nq, Lq, 128)
    D = _rows(2, B * Ld, dtn)
    cu = inputs.cu_seqlens(np.full(B, Ld, np.int32))
    A = np.random.default_rng(3).integers(0, Ld, size=(Nq, B, Lq)).astype(np.int32)
    g = np.random.default_rng(4).standard_normal((Nq, B)).astype(np.float32)
    rp, ci = oracle.csr_build_varlen(A, cu)
    rp2, ci2 = oracle.csr_build(A, Ld)
    assert np.array_equal(rp, rp2) and np.array_equal(ci, ci2)
    dQ, dD = oracle.bwd_varlen(Q, D, cu, oracle.F16 if dtn == inputs.F16 else oracle.BF16, A, g)
    dQ2, dD2 = oracle.bwd(Q, D.reshape(B, Ld, 128), oracle.F16 if dtn == inputs.F16 else oracle.BF16, A, g)
    assert np.array_equal(dQ, dQ2) and np.array_equal(dD, dD2.reshape(B * Ld, 128))


def test_scatter_add_brute_force_and_csr_invariants():
    rng = np.random.default_rng(9)
    Nq, Lq, B = 4, 6, 7
    lens = np.array([3, 1, 5, 2, 8, 4, 1], np.int32)
    cu = inputs.cu_seqlens(lens)
    T = int(cu[-1])
    Q = _rows(5, Nq * Lq).reshape(Nq, Lq, 128)
    D = _rows(6, T)
    A = np.stack([rng.integers(0, lens[b], size=(Nq, Lq)) for b in range(B)], axis=1).astype(np.int32)
    g = rng.standard_normal((Nq, B)).astype(np.float32)
    dQ, dD = oracle.bwd_varlen(Q, D, cu, oracle.F16, A, g)
    rdQ = np.zeros((Nq, Lq, 128))
    rdD = np.zeros((T, 128))
    qd, dd = Q.astype(np.float64), D.astype(np.float64)
    for q in range(Nq):
        for b in range(B):
            rows = cu[b] + A[q, b]
            rdQ[q] += float(g[q, b]) * dd[rows]
            np.add.at(rdD, rows, float(g[q, b]) * qd[q])
    assert np.allclose(dQ, rdQ, rtol=1e-12, atol=1e-12) and np.allclose(dD, rdD, rtol=1e-12, atol=1e-12)
    rp, ci = oracle.csr_build_varlen(A, cu)
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0) and rp[-1] == Nq * B * Lq
    assert np.array_equal(np.sort(ci), np.arange(Nq * B * Lq))
    for r in range(T):
        srcs = ci[rp[r]:rp[r + 1]]
        assert np.all(np.diff(srcs) > 0)  # stable: ascending source id
        b = (srcs // Lq) % B
        assert np.all(cu[b] + A.reshape(-1)[srcs] == r)


def test_empty_documents_act_as_removed():
    rng = np.random.default_rng(12)
    Nq, Lq = 3, 5
    lens = np.array([4, 0, 6, 0, 0, 3], np.int32)
    keep = np.flatnonzero(lens > 0)
    B = len(lens)
    cu = inputs.cu_seqlens(lens)
    Q = _rows(7, Nq * Lq).reshape(Nq, Lq, 128)
    D = _rows(8, int(cu[-1]))
    A = np.full((Nq, B, Lq), -1, np.int32)
    for b in keep:
        A[:, b] = rng.integers(0, lens[b], size=(Nq, Lq))
    g = rng.standard_normal((Nq, B)).astype(np.float32)
    dQ, dD = oracle.bwd_varlen(Q, D, cu, oracle.F16, A, g)
    cu2 = inputs.cu_seqlens(lens[keep])
    dQ2, dD2 = oracle.bwd_varlen(Q, D, cu2, oracle.F16, A[:, keep], g[:, keep])
    assert np.array_equal(dQ, dQ2) and np.array_equal(dD, dD2)
    rp, ci = oracle.csr_build_varlen(A, cu)
    rp2, ci2 = oracle.csr_build_varlen(A[:, keep], cu2)
    assert np.array_equal(rp, rp2)
    # source ids refer to the full document numbering
    q, rem = np.divmod(ci2, len(keep) * Lq)
    bk, i = np.divmod(rem, Lq)
    assert np.array_equal(ci, (q * B + keep[bk]) * Lq + i)


def test_euler_homogeneity_with_forward_argmax():
    w = inputs.make("colbert_rerank_varlen", B=30, Nq=4, Ld=(1, 40))
    s, A = oracle.fwd_varlen(w["Q"], w["D_packed"], w["cu_seqlens"], oracle.F16)
    g = np.random.default_rng(2).standard_normal(s.shape).astype(np.float32)
    dQ, dD = oracle.bwd_varlen(w["Q"], w["D_packed"], w["cu_seqlens"], oracle.F16, A, g)
    lhs = np.sum(dQ * w["Q"].astype(np.float64))
    mid = np.sum(g.astype(np.float64) * s)
    rhs = np.sum(dD * w["D_packed"].astype(np.float64))
    assert lhs == pytest.approx(mid, rel=1e-9) and rhs == pytest.approx(mid, rel=1e-9)
