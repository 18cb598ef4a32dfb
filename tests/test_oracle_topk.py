"""Pins for the oracle's pair scoring, top-K selection and two-stage scan
(test infrastructure; no GPU).

Top-K is checked against numpy's stable sort (lexsort on score, then index),
against invariants (values non-increasing, every kept score at least every
dropped one, equal scores by ascending index) and special cases (-inf last,
all-equal rows).  Pair scoring is checked against a numpy brute force on
tiny inputs and against the already-pinned full forward.  The two-stage scan
reduces to the plain top-K of the fp16 scores when every document is a
candidate, and its candidates are the top-K1 of the INT8 scores.
"""
import numpy as np
import pytest

import oracle
from late_interaction_retrieval_amd import inputs


def np_topk(s, K):
    idx = np.empty((s.shape[0], K), np.int32)
    for q in range(s.shape[0]):
        order = np.lexsort((np.arange(s.shape[1]), -s[q].astype(np.float64)))
        idx[q] = order[:K]
    return idx, np.take_along_axis(s, idx, 1)


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("K", [1, 5, 37])
def test_topk_matches_stable_sort_with_many_ties(seed, K):
    rng = np.random.default_rng(seed)
    s = rng.integers(-4, 5, size=(6, 37)).astype(np.float32) * 0.5  # many equal scores
    s[0, 3] = -np.inf
    idx, val = oracle.topk(s, K)
    ridx, rval = np_topk(s, K)
    assert np.array_equal(idx, ridx) and np.array_equal(val, rval)


def test_topk_invariants_random():
    rng = np.random.default_rng(7)
    s = rng.standard_normal((5, 1000)).astype(np.float32)
    s[:, ::7] = s[:, 1::7]  # exact duplicates
    K = 50
    idx, val = oracle.topk(s, K)
    for q in range(5):
        assert np.all(np.diff(val[q]) <= 0)
        assert np.array_equal(val[q], s[q, idx[q]])
        dropped = np.setdiff1d(np.arange(1000), idx[q])
        assert val[q, -1] >= s[q, dropped].max()
        for k in range(K - 1):
            if val[q, k] == val[q, k + 1]:
                assert idx[q, k] < idx[q, k + 1]
        # a dropped document equal to the last kept one has a larger index
        tie = dropped[s[q, dropped] == val[q, -1]]
        assert np.all(tie > idx[q][val[q] == val[q, -1]].max())


def test_topk_special_cases():
    s = np.array([[2.0, 2.0, 2.0, 2.0], [-np.inf, 1.0, -np.inf, 0.0]], np.float32)
    idx, val = oracle.topk(s, 4)
    assert idx[0].tolist() == [0, 1, 2, 3]
    assert idx[1].tolist() == [1, 3, 0, 2]
    assert np.isneginf(val[1, 2:]).all()
    with pytest.raises(ValueError):
        oracle.topk(s, 5)


def test_pairs_brute_force_tiny():
    rng = np.random.default_rng(3)
    Nq, Lq, d = 3, 4, 128
    lens = np.array([5, 1, 7, 3], np.int32)
    cu = inputs.cu_seqlens(lens)
    Q = (rng.standard_normal((Nq, Lq, d)) * 0.1).astype(np.float16)
    D = (rng.standard_normal((int(cu[-1]), d)) * 0.1).astype(np.float16)
    pq = np.array([2, 0, 1, 2, 0], np.int32)
    pb = np.array([3, 0, 2, 1, 3], np.int32)
    s, a = oracle.fwd_pairs(Q, D, cu, oracle.F16, pq, pb)
    for p in range(5):
        doc = D[cu[pb[p]]:cu[pb[p] + 1]].astype(np.float64)
        sim = Q[pq[p]].astype(np.float64) @ doc.T
        assert s[p] == pytest.approx(sim.max(1).sum(), rel=1e-12, abs=1e-12)
        assert np.array_equal(a[p], sim.argmax(1))


def test_pairs_equal_full_forward():
    w = inputs.make("colbert_rerank_varlen", B=60, Nq=5)
    s_full, a_full = oracle.fwd_varlen(w["Q"], w["D_packed"], w["cu_seqlens"], oracle.F16)
    rng = np.random.default_rng(4)
    pq = rng.integers(0, 5, size=40).astype(np.int32)
    pb = rng.integers(0, 60, size=40).astype(np.int32)
    s, a = oracle.fwd_pairs(w["Q"], w["D_packed"], w["cu_seqlens"], oracle.F16, pq, pb)
    assert np.array_equal(s, s_full[pq, pb]) and np.array_equal(a, a_full[pq, pb])


def _two_stage_inputs(B):
    w8 = inputs.make("int8_varlen", B=B, Nq=3)
    w16 = inputs.make("int8_varlen", B=B, Nq=3)  # same seeds: the same rows before quantisation
    return w8, inputs.fp16_of_int8_workload(w16)


def test_two_stage_reduces_to_plain_topk_when_every_document_is_a_candidate():
    B = 40
    w8, (Q16, D16) = _two_stage_inputs(B)
    cand, cval, final, fval = oracle.two_stage_topk(w8["Q"], w8["q_scale"], w8["D_packed"], w8["d_scale"],
                                                    Q16, D16, w8["cu_seqlens"], oracle.F16, B, 7)
    s16, _ = oracle.fwd_varlen(Q16, D16, w8["cu_seqlens"], oracle.F16)
    for q in range(3):
        order = np.lexsort((np.arange(B), -s16[q]))[:7]
        assert np.array_equal(final[q], order)
        assert np.array_equal(fval[q], s16[q][order])


def test_two_stage_candidates_are_the_int8_topk():
    B = 50
    w8, (Q16, D16) = _two_stage_inputs(B)
    cand, cval, final, fval = oracle.two_stage_topk(w8["Q"], w8["q_scale"], w8["D_packed"], w8["d_scale"],
                                                    Q16, D16, w8["cu_seqlens"], oracle.F16, 12, 4)
    s8, _ = oracle.fwd_i8(w8["Q"], w8["q_scale"], w8["D_packed"], w8["d_scale"], w8["cu_seqlens"])
    ridx, rval = np_topk(s8, 12)
    assert np.array_equal(cand, ridx) and np.array_equal(cval, rval)
    for q in range(3):
        assert set(final[q]) <= set(cand[q])
        assert np.all(np.diff(fval[q]) <= 0)
