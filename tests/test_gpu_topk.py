"""GPU parity of the pair-list forward, the per-query top-K and the two-stage
INT8 -> fp16 scan against the CPU oracle, through the C ABI.  Run on an
MI355X: pytest -m gpu.

Top-K selects from the same fp32 scores on both sides, so indices and values
must be bit-identical (ties by id).  Pair scores follow the fp16/bf16
tolerance; the two-stage candidates come from bit-exact INT8 scores, so the
candidate lists must be identical, and the final lists may differ only among
documents whose oracle scores are within the score tolerance of each other.
"""
import numpy as np
import pytest
import torch

import oracle
from late_interaction_retrieval_amd import inputs
from gpu_util import ARGMAX_TIE_TOL, DEV, SCORE_TOL_PER_QTOKEN, check_scores, oracle_dtype, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from late_interaction_retrieval_amd import binding
    assert torch.cuda.is_available()
    return binding


TOPK_CASES = [(1, 1, 1), (3, 5, 5), (4, 1000, 7), (2, 1000, 1000), (5, 100000, 100), (2, 3000, 1024)]


@pytest.mark.parametrize("case", TOPK_CASES, ids=[str(c) for c in TOPK_CASES])
def test_topk_bit_exact(bd, case):
    Nq, B, K = case
    rng = np.random.default_rng(sum(case))
    s = rng.standard_normal((Nq, B)).astype(np.float32)
    s[:, ::3] = np.round(s[:, ::3] * 4) / 4  # many exact ties
    s[0, rng.integers(0, B, size=max(1, B // 10))] = -np.inf
    idx, val = bd.maxsim_topk(to_dev(s), K)
    torch.cuda.synchronize()
    ridx, rval = oracle.topk(s, K)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    assert np.array_equal(val.cpu().numpy(), rval)


def test_topk_ties_follow_given_ids(bd):
    rng = np.random.default_rng(11)
    Nq, B, K = 3, 500, 40
    s = rng.integers(0, 6, size=(Nq, B)).astype(np.float32)
    ids = np.stack([rng.permutation(B) * 3 + 1 for _ in range(Nq)]).astype(np.int32)
    idx, val = bd.maxsim_topk(to_dev(s), K, ids=to_dev(ids))
    torch.cuda.synchronize()
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    for q in range(Nq):
        order = np.lexsort((ids[q], -s[q]))[:K]
        assert np.array_equal(idx[q], ids[q][order]) and np.array_equal(val[q], s[q][order])


PAIR_CASES = [(inputs.F16, 32, 40), (inputs.BF16, 32, 40), (inputs.F16, 100, 30), (inputs.BF16, 1024, 6),
              (inputs.F16, 7, 25)]


@pytest.mark.parametrize("case", PAIR_CASES, ids=[str(c) for c in PAIR_CASES])
def test_pairs_match_oracle(bd, case):
    dtn, Lq, P = case
    Nq, B = 5, 60
    rng = np.random.default_rng(Lq + P)
    Q = inputs.random_rows(Lq, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    lens = rng.integers(0, 200, size=B).astype(np.int32)
    lens[3] = 0
    cu = inputs.cu_seqlens(lens)
    Dp = inputs.random_rows(Lq + 1, int(cu[-1]), 128, dtn, stream=4)
    pq = rng.integers(0, Nq, size=P).astype(np.int32)
    pb = rng.integers(0, B, size=P).astype(np.int32)
    pb[0] = 3  # an empty document
    s, a = bd.maxsim_fwd_pairs(to_dev(Q, dtn), to_dev(Dp, dtn), to_dev(cu), to_dev(pq), to_dev(pb),
                               with_argmax=True)
    torch.cuda.synchronize()
    s, a = s.cpu().numpy(), a.cpu().numpy()
    s_ref, a_ref = oracle.fwd_pairs(Q, Dp, cu, oracle_dtype(dtn), pq, pb)
    check_scores(s, s_ref, Lq, "pairs %s" % (case,))
    assert np.all(a[0] == -1)
    # argmax: equal, or an in-range near-tie (oracle similarity of the GPU pick)
    for p in range(P):
        doc = pb[p]
        n = lens[doc]
        if n == 0:
            continue
        diff = a[p] != a_ref[p]
        if diff.any():
            assert np.all((a[p] >= 0) & (a[p] < n))
            qd = (Q[pq[p]].astype(np.float64) if dtn == inputs.F16 else
                  oracle.bf16_to_f64(Q[pq[p]]))
            dd = (Dp[cu[doc]:cu[doc + 1]].astype(np.float64) if dtn == inputs.F16 else
                  oracle.bf16_to_f64(Dp[cu[doc]:cu[doc + 1]]))
            full = qd @ dd.T
            got = full[np.arange(Lq), a[p]]
            assert np.all(got[diff] >= full.max(1)[diff] - ARGMAX_TIE_TOL)


def test_pairs_agree_with_full_forward(bd):
    w = inputs.make("colbert_rerank_varlen", B=300, Nq=6)
    Q, Dp, cu = to_dev(w["Q"]), to_dev(w["D_packed"]), to_dev(w["cu_seqlens"])
    full, _ = bd.maxsim_fwd_varlen(Q, Dp, cu, 300, with_argmax=False)
    rng = np.random.default_rng(5)
    pq = rng.integers(0, 6, size=500).astype(np.int32)
    pb = rng.integers(0, 300, size=500).astype(np.int32)
    s, _ = bd.maxsim_fwd_pairs(Q, Dp, cu, to_dev(pq), to_dev(pb))
    torch.cuda.synchronize()
    ref = full.cpu().numpy()[pq, pb]
    assert np.abs(s.cpu().numpy() - ref).max() <= SCORE_TOL_PER_QTOKEN * 32


def two_stage_inputs(B, Nq):
    w8 = inputs.make("int8_varlen", B=B, Nq=Nq)
    Q16, D16 = inputs.fp16_of_int8_workload(w8)
    return w8, Q16, D16


@pytest.mark.parametrize("case", [(3, 400, 40, 10), (4, 2000, 100, 10), (2, 50, 50, 50)],
                         ids=["3x400", "4x2000", "all-candidates"])
def test_two_stage_matches_oracle(bd, case):
    Nq, B, K1, K2 = case
    w8, Q16, D16 = two_stage_inputs(B, Nq)
    cand, c8, top, tops = bd.maxsim_two_stage_topk(
        to_dev(w8["Q"]), to_dev(w8["q_scale"]), to_dev(w8["D_packed"]), to_dev(w8["d_scale"]),
        to_dev(Q16), to_dev(D16), to_dev(w8["cu_seqlens"]), int(w8["lens"].max()), K1, K2)
    torch.cuda.synchronize()
    cand, c8, top, tops = cand.cpu().numpy(), c8.cpu().numpy(), top.cpu().numpy(), tops.cpu().numpy()
    rc, rc8, rtop, rtops = oracle.two_stage_topk(w8["Q"], w8["q_scale"], w8["D_packed"], w8["d_scale"],
                                                 Q16, D16, w8["cu_seqlens"], oracle.F16, K1, K2)
    assert np.array_equal(cand, rc) and np.array_equal(c8, rc8), "INT8 candidate lists differ"
    tol = SCORE_TOL_PER_QTOKEN * w8["Lq"]
    for q in range(Nq):
        pq = np.full(K1, q, np.int32)
        s16 = oracle.fwd_pairs(Q16, D16, w8["cu_seqlens"], oracle.F16, pq, cand[q], want_argmax=False)
        by_doc = dict(zip(cand[q].tolist(), s16.tolist()))
        # every returned score is its document's score within tolerance, best first
        assert np.all(np.diff(tops[q]) <= 0)
        for doc, sc in zip(top[q], tops[q]):
            assert abs(by_doc[int(doc)] - sc) <= tol
        # the returned set differs from the oracle's only across near-ties at the cut
        kth = rtops[q][-1]
        for doc in set(top[q].tolist()) ^ set(rtop[q].tolist()):
            assert abs(by_doc[int(doc)] - kth) <= 2 * tol, "query %d: document %d is not a near-tie" % (q, doc)
