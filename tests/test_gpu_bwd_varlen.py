"""GPU parity of the packed-corpus (cu_seqlens) backward against the oracle:
inverse-grid CSR bit-exact, dD and dQ within relative Frobenius error 1e-3,
exact zeros on rows no query token selected, through the C ABI.  Run on an
MI355X: pytest -m gpu.

Both sides get the same argmax and upstream gradient (from the oracle's
forward or from seeded generators), so a near-tie argmax difference of the
forward cannot re-route a row."""
import numpy as np
import pytest
import torch

import oracle
from late_interaction_retrieval_amd import inputs
from gpu_util import GRAD_REL_TOL, check_grad, oracle_dtype, rel_fro, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from late_interaction_retrieval_amd import binding
    assert torch.cuda.is_available()
    return binding


def run(bd, Q, Dp, cu, dtn, A, g, max_Ld):
    dQ, dD, rp, ci = bd.maxsim_bwd_varlen(to_dev(Q, dtn), to_dev(Dp, dtn), to_dev(cu), max_Ld, to_dev(A),
                                          to_dev(g))
    torch.cuda.synchronize()
    return dQ.cpu().numpy(), dD.cpu().numpy(), rp.cpu().numpy(), ci.cpu().numpy()


def check(bd, Q, Dp, cu, dtn, A, g, where, max_Ld=None):
    lens = np.diff(cu)
    if max_Ld is None:
        max_Ld = max(1, int(lens.max(initial=1)))
    dQ, dD, rp, ci = run(bd, Q, Dp, cu, dtn, A, g, max_Ld)
    rp_ref, ci_ref = oracle.csr_build_varlen(A, cu)
    assert np.array_equal(rp, rp_ref), where + ": row_ptr"
    assert np.array_equal(ci[:rp_ref[-1]], ci_ref), where + ": col_idx"
    dQ_ref, dD_ref = oracle.bwd_varlen(Q, Dp, cu, oracle_dtype(dtn), A, g)
    rq, rd = check_grad(dQ, dQ_ref, "dQ", where), check_grad(dD, dD_ref, "dD", where)
    empty_rows = np.diff(rp_ref) == 0
    assert np.all(dD[empty_rows] == 0.0), where + ": rows without sources must be exactly 0"
    # deterministic: a second call is bit-identical
    dQ2, dD2, rp2, ci2 = run(bd, Q, Dp, cu, dtn, A, g, max_Ld)
    assert np.array_equal(dQ, dQ2) and np.array_equal(dD, dD2) and np.array_equal(ci[:rp[-1]], ci2[:rp[-1]])
    print("%s: %s; %s" % (where, rq, rd), flush=True)
    return dQ, dD


def corpus(seed, lens, dtn):
    cu = inputs.cu_seqlens(np.asarray(lens, np.int32))
    Dp = inputs.random_rows(seed, int(cu[-1]), 128, dtn, stream=4)
    return Dp, cu


# (Nq, Lq, document lengths): ragged, empty documents first / inside / last,
# lengths across the 16-row and 64-lane boundaries, one long document
CASES = [
    (1, 1, [1]),
    (2, 7, [3, 0, 5]),
    (3, 33, [0, 70, 1, 0, 17]),
    (9, 64, [64, 63, 65, 0]),
    (17, 100, [129, 2, 300, 0, 0, 31]),
    (5, 1024, [1024, 7]),
    (20, 32, list(range(0, 40, 3))),
    (1, 5, [4096]),
    # 2600 documents, a third of them empty: more (document, group) pairs than
    # the fill sums itself, so the documents' first slots come from their scan
    (2, 16, [int(x) for x in np.random.default_rng(26).integers(0, 31, size=2600) * (np.arange(2600) % 3 > 0)]),
    (4, 48, [1500, 0, 2100, 40]),
    # the fill's step counts and group sizes at its largest LDS (G x max_Ld = 16384), and
    # 40 short queries (groups of 8) over 1200 ragged documents
    (12, 200, [2048, 17, 0]), (17, 300, [700, 0, 512, 33]), (9, 600, [1024, 5, 900]),
    (40, 32, [int(x) for x in np.random.default_rng(40).integers(0, 181, size=1200)]),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c[:2]) + "x%d" % len(c[2]) for c in CASES])
@pytest.mark.parametrize("dtn", [inputs.F16, inputs.BF16])
def test_chain_forward_argmax(bd, case, dtn):
    """argmax from the oracle's packed forward, seeded upstream gradient."""
    Nq, Lq, lens = case
    seed = 1300 + Nq + Lq + len(lens)
    Q = inputs.random_rows(seed, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    Dp, cu = corpus(seed + 1, lens, dtn)
    _, A = oracle.fwd_varlen(Q, Dp, cu, oracle_dtype(dtn))
    g = np.random.default_rng(seed).standard_normal((Nq, len(lens))).astype(np.float32)
    check(bd, Q, Dp, cu, dtn, A, g, "%s %s" % (dtn, case[:2]))


def test_max_Ld_above_longest(bd):
    """max_Ld is an upper bound: a larger one changes nothing."""
    Nq, Lq, lens = 4, 40, [10, 0, 33, 5]
    Q = inputs.random_rows(5, Nq * Lq, 128, inputs.F16).reshape(Nq, Lq, 128)
    Dp, cu = corpus(6, lens, inputs.F16)
    _, A = oracle.fwd_varlen(Q, Dp, cu, oracle.F16)
    g = np.random.default_rng(5).standard_normal((Nq, len(lens))).astype(np.float32)
    a = check(bd, Q, Dp, cu, inputs.F16, A, g, "max_Ld 33", max_Ld=33)
    b = check(bd, Q, Dp, cu, inputs.F16, A, g, "max_Ld 500", max_Ld=500)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_all_documents_empty(bd):
    """T = 0: no rows, no sources, dQ all zero."""
    Nq, Lq, B = 3, 16, 4
    Q = inputs.random_rows(8, Nq * Lq, 128, inputs.BF16).reshape(Nq, Lq, 128)
    Dp = np.zeros((0, 128), np.uint16)
    cu = np.zeros(B + 1, np.int32)
    A = np.full((Nq, B, Lq), -1, np.int32)
    g = np.ones((Nq, B), np.float32)
    dQ, dD, rp, ci = run(bd, Q, Dp, cu, inputs.BF16, A, g, 8)
    assert dD.shape == (0, 128) and np.array_equal(rp, [0]) and np.all(dQ == 0.0)


def test_hot_tokens(bd):
    """Most query tokens select one of the first three rows of their document."""
    Nq, Lq = 16, 256
    lens = [512, 0, 300, 3, 512]
    rng = np.random.default_rng(91)
    Q = inputs.random_rows(91, Nq * Lq, 128, inputs.BF16).reshape(Nq, Lq, 128)
    Dp, cu = corpus(92, lens, inputs.BF16)
    A = np.full((Nq, len(lens), Lq), -1, np.int32)
    for b, n in enumerate(lens):
        if n:
            a = rng.integers(0, n, size=(Nq, Lq))
            hot = rng.random(a.shape) < 0.8
            a[hot] = rng.integers(0, min(3, n), size=int(hot.sum()))
            A[:, b] = a
    g = rng.standard_normal((Nq, len(lens))).astype(np.float32)
    check(bd, Q, Dp, cu, inputs.BF16, A, g, "hot tokens")


def test_padded_equivalence(bd):
    """Equal-length packed documents give the padded backward's results bit for bit."""
    Nq, Lq, B, Ld = 6, 48, 5, 40
    Q = inputs.random_rows(21, Nq * Lq, 128, inputs.F16).reshape(Nq, Lq, 128)
    Dp, cu = corpus(22, [Ld] * B, inputs.F16)
    A = np.random.default_rng(21).integers(0, Ld, size=(Nq, B, Lq)).astype(np.int32)
    g = np.random.default_rng(22).standard_normal((Nq, B)).astype(np.float32)
    dQ, dD, rp, ci = run(bd, Q, Dp, cu, inputs.F16, A, g, Ld)
    pQ, pD, prp, pci = bd.maxsim_bwd(to_dev(Q, inputs.F16), to_dev(Dp.reshape(B, Ld, 128), inputs.F16),
                                     to_dev(A), to_dev(g))
    assert np.array_equal(rp, prp.cpu().numpy()) and np.array_equal(ci, pci.cpu().numpy())
    assert np.array_equal(dQ, pQ.cpu().numpy()) and np.array_equal(dD.reshape(B, Ld, 128), pD.cpu().numpy())


def test_workload_colbert_rerank_varlen_full(bd):
    """The packed re-ranking corpus at full size (64 queries x 10000 documents of
    32..300 tokens, Lq = 32): seeded argmax uniform over each document's rows,
    seeded upstream gradient."""
    w = inputs.make("colbert_rerank_varlen")
    Nq, Lq, B = w["Nq"], w["Lq"], w["B"]
    lens = w["lens"]
    rng = np.random.default_rng([2, 9])
    A = (rng.random((Nq, B, Lq)) * lens[None, :, None]).astype(np.int32)
    g = rng.standard_normal((Nq, B)).astype(np.float32)
    check(bd, w["Q"], w["D_packed"], w["cu_seqlens"], inputs.F16, A, g, "colbert_rerank_varlen",
          max_Ld=w["Ld_max"])


def test_workload_contrastive_train_varlen_full(bd):
    """The ragged training workload at full size (64 x 64 pairs, Lq = 1024,
    documents of 256..1024 tokens): seeded argmax uniform over each document's
    rows, an InfoNCE-shaped upstream gradient of seeded scores."""
    from gpu_util import infonce_grad
    w = inputs.make("contrastive_train_varlen")
    Nq, Lq, B = w["Nq"], w["Lq"], w["B"]
    lens = w["lens"]
    rng = np.random.default_rng([7, 3])
    A = (rng.random((Nq, B, Lq)) * lens[None, :, None]).astype(np.int32)
    fake_scores = rng.standard_normal((Nq, B)) * 0.05 + np.eye(Nq) * 0.1
    g = infonce_grad(fake_scores, w["tau"]).astype(np.float32)
    check(bd, w["Q"], w["D_packed"], w["cu_seqlens"], inputs.BF16, A, g, "contrastive_train_varlen",
          max_Ld=w["Ld_max"])
