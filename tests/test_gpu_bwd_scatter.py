"""GPU parity of the atomic-scatter backward (dD by fp32 atomic adds, no CSR)
against the oracle, padded and packed, and of the autograd op that dispatches
between the two reductions.  Gradients within relative Frobenius error 1e-3,
rows no source selects exactly 0.  Run on an MI355X: pytest -m gpu."""
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


def check_grads(dQ, dD, dQ_ref, dD_ref, sources_per_row, where):
    rq, rd = check_grad(dQ, dQ_ref, "dQ", where), check_grad(dD, dD_ref, "dD", where)
    assert np.all(dD.reshape(-1, 128)[sources_per_row == 0] == 0.0), where + ": untouched rows must be 0"
    print("%s: %s; %s" % (where, rq, rd), flush=True)


PADDED = [(1, 1, 1, 1), (2, 7, 3, 5), (3, 33, 4, 70), (1, 32, 50, 180), (17, 100, 3, 129), (4, 1024, 2, 1024)]


@pytest.mark.parametrize("shape", PADDED, ids=[str(s) for s in PADDED])
@pytest.mark.parametrize("dtn", [inputs.F16, inputs.BF16])
def test_padded(bd, shape, dtn):
    Nq, Lq, B, Ld = shape
    seed = 1700 + sum(shape)
    Q = inputs.random_rows(seed, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    D = inputs.random_rows(seed + 1, B * Ld, 128, dtn, stream=4).reshape(B, Ld, 128)
    _, A = oracle.fwd_padded(Q, D, oracle_dtype(dtn))
    g = np.random.default_rng(seed).standard_normal((Nq, B)).astype(np.float32)
    Qd, Dd, Ad, gd = to_dev(Q, dtn), to_dev(D, dtn), to_dev(A), to_dev(g)
    dQ, dD = bd.maxsim_bwd_scatter(Qd, Dd, Ad, gd)
    torch.cuda.synchronize()
    dQ_ref, dD_ref = oracle.bwd(Q, D, oracle_dtype(dtn), A, g)
    rp, _ = oracle.csr_build(A, Ld)
    check_grads(dQ.cpu().numpy(), dD.cpu().numpy(), dQ_ref, dD_ref, np.diff(rp), "%s %s" % (dtn, shape))
    # dQ comes from the same gather as the CSR path: bit-identical
    cQ, _, _, _ = bd.maxsim_bwd(Qd, Dd, Ad, gd)
    assert torch.equal(dQ, cQ)


VARLEN = [(2, 7, [3, 0, 5]), (3, 33, [0, 70, 1, 0, 17]), (1, 32, [180] * 9 + [0, 31]), (5, 1024, [1024, 7])]


@pytest.mark.parametrize("case", VARLEN, ids=[str(c[:2]) + "x%d" % len(c[2]) for c in VARLEN])
@pytest.mark.parametrize("dtn", [inputs.F16, inputs.BF16])
def test_packed(bd, case, dtn):
    Nq, Lq, lens = case
    seed = 1800 + Nq + Lq + len(lens)
    Q = inputs.random_rows(seed, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    cu = inputs.cu_seqlens(np.asarray(lens, np.int32))
    Dp = inputs.random_rows(seed + 1, int(cu[-1]), 128, dtn, stream=4)
    _, A = oracle.fwd_varlen(Q, Dp, cu, oracle_dtype(dtn))
    g = np.random.default_rng(seed).standard_normal((Nq, len(lens))).astype(np.float32)
    dQ, dD = bd.maxsim_bwd_scatter(to_dev(Q, dtn), to_dev(Dp, dtn), to_dev(A), to_dev(g), cu_seqlens=to_dev(cu),
                                   max_Ld=max(1, max(lens)))
    torch.cuda.synchronize()
    dQ_ref, dD_ref = oracle.bwd_varlen(Q, Dp, cu, oracle_dtype(dtn), A, g)
    rp, _ = oracle.csr_build_varlen(A, cu)
    check_grads(dQ.cpu().numpy(), dD.cpu().numpy(), dQ_ref, dD_ref, np.diff(rp), "%s %s" % (dtn, case[:2]))


def test_workload_colbert_tiny_full(bd):
    """The single-query workload (1 x 1000 documents of 180 tokens, Lq = 32), the
    low-contention case the scatter is for: 0.18 sources per row."""
    w = inputs.make("colbert_tiny")
    B, Ld = w["B"], w["Ld_max"]
    D = w["D_packed"].reshape(B, Ld, 128)
    assert bd.maxsim_bwd_prefer_scatter(w["Nq"], w["Lq"], B, B * Ld)
    _, A = oracle.fwd_padded(w["Q"], D, oracle.F16)
    g = np.random.default_rng([3, 1]).standard_normal((1, B)).astype(np.float32)
    dQ, dD = bd.maxsim_bwd_scatter(to_dev(w["Q"], inputs.F16), to_dev(D, inputs.F16), to_dev(A), to_dev(g))
    torch.cuda.synchronize()
    dQ_ref, dD_ref = oracle.bwd(w["Q"], D, oracle.F16, A, g)
    rp, _ = oracle.csr_build(A, Ld)
    check_grads(dQ.cpu().numpy(), dD.cpu().numpy(), dQ_ref, dD_ref, np.diff(rp), "colbert_tiny")


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("deterministic", [True, False])
def test_autograd_op(bd, packed, deterministic):
    """torch autograd through the op: scores and gradients of sum(w * scores)
    against the oracle's forward and backward."""
    Nq, Lq, lens = 3, 20, [40, 0, 17, 33]
    dtn = inputs.F16
    Q = inputs.random_rows(31, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    wts = np.random.default_rng(33).standard_normal((Nq, len(lens))).astype(np.float32)
    Qt = to_dev(Q, dtn).requires_grad_(True)
    if packed:
        cu = inputs.cu_seqlens(np.asarray(lens, np.int32))
        D = inputs.random_rows(32, int(cu[-1]), 128, dtn, stream=4)
        Dt = to_dev(D, dtn).requires_grad_(True)
        s = bd.maxsim(Qt, Dt, cu_seqlens=to_dev(cu), max_Ld=max(lens), deterministic=deterministic)
        s_ref, A = oracle.fwd_varlen(Q, D, cu, oracle.F16)
        dQ_ref, dD_ref = oracle.bwd_varlen(Q, D, cu, oracle.F16, A, wts)
        _, a_gpu = bd.maxsim_fwd_varlen(to_dev(Q, dtn), to_dev(D, dtn), to_dev(cu), max(lens))
    else:
        B, Ld = 4, 40  # every row of a padded document is scored, so all rows are real here
        D = inputs.random_rows(32, B * Ld, 128, dtn, stream=4).reshape(B, Ld, 128)
        Dt = to_dev(D, dtn).requires_grad_(True)
        s = bd.maxsim(Qt, Dt, deterministic=deterministic)
        s_ref, A = oracle.fwd_padded(Q, D, oracle.F16)
        dQ_ref, dD_ref = oracle.bwd(Q, D, oracle.F16, A, wts)
        _, a_gpu = bd.maxsim_fwd(to_dev(Q, dtn), to_dev(D, dtn))
    # the gradient follows the argmax: this seed has no near-tie that could re-route a row
    assert np.array_equal(a_gpu.cpu().numpy(), A), "a near-tie argmax at this seed; pick another"
    (s * to_dev(wts)).sum().backward()
    got = s.detach().cpu().numpy().astype(np.float64)
    fin = np.isfinite(s_ref)  # an empty document scores -inf on both sides
    assert np.array_equal(np.isneginf(got), ~fin)
    assert np.abs(got[fin] - s_ref[fin]).max() <= 1e-3 * Lq
    # the op returns gradients in the input dtype (fp16): compare at that precision
    eq = rel_fro(Qt.grad.float().cpu().numpy(), dQ_ref)
    ed = rel_fro(Dt.grad.float().cpu().numpy(), dD_ref)
    assert eq <= 2e-3 and ed <= 2e-3, (eq, ed)
