"""The allocation-free backward (maxsim_bwd_noalloc) against maxsim_bwd on the
GPU, through the C ABI: the same kernels, with the library's own scratch array
as the workspace, give the same bits.  Two calls in a row share the array; the
second, smaller one must not be disturbed by what the first left in it.
Run on an MI355X: pytest -m gpu."""
import numpy as np
import pytest
import torch

import oracle
from late_interaction_retrieval_amd import inputs
from gpu_util import check_grad, infonce_grad, oracle_dtype, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from late_interaction_retrieval_amd import binding
    assert torch.cuda.is_available()
    return binding


def case(seed, Nq, Lq, B, Ld, dtn, hot=0.0):
    Q = inputs.random_rows(seed, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    D = inputs.random_rows(seed + 1, B * Ld, 128, dtn, stream=4).reshape(B, Ld, 128)
    rng = np.random.default_rng(seed)
    A = rng.integers(0, Ld, size=(Nq, B, Lq)).astype(np.int32)
    if hot:
        sel = rng.random(A.shape) < hot
        A[sel] = rng.integers(0, 4, size=int(sel.sum()))
    g = rng.standard_normal((Nq, B)).astype(np.float32)
    return Q, D, A, g


def run_both(bd, Q, D, A, g, dtn):
    Qd, Dd, Ad, gd = to_dev(Q, dtn), to_dev(D, dtn), to_dev(A), to_dev(g)
    Nq, Lq, _ = Q.shape
    B, Ld, _ = D.shape
    ref = bd.maxsim_bwd(Qd, Dd, Ad, gd)
    # outputs prefilled with garbage: the call must overwrite them
    dQ = torch.full((Nq, Lq, 128), float("nan"), device=Qd.device)
    dD = torch.full((B, Ld, 128), float("nan"), device=Qd.device)
    rp = torch.full((B * Ld + 1,), -7, dtype=torch.int32, device=Qd.device)
    ci = torch.full((Nq * B * Lq,), -7, dtype=torch.int32, device=Qd.device)
    torch.cuda.synchronize()
    got = bd.maxsim_bwd_noalloc(Qd, Dd, Ad, gd, dQ, dD, rp, ci)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ref], [t.cpu().numpy() for t in got]


def check(ref, got, Q, D, A, g, dtn, where):
    rQ, rD, rrp, rci = ref
    gQ, gD, grp, gci = got
    assert np.array_equal(grp, rrp), where + ": row_ptr"
    assert np.array_equal(gci[:rrp[-1]], rci[:rrp[-1]]), where + ": col_idx"
    assert np.array_equal(gQ, rQ) and np.array_equal(gD, rD), where + ": gradients differ from maxsim_bwd"
    rp_o, ci_o = oracle.csr_build(A, D.shape[1])
    assert np.array_equal(grp, rp_o) and np.array_equal(gci[:rp_o[-1]], ci_o), where + ": CSR vs oracle"
    dQ_o, dD_o = oracle.bwd(Q, D, oracle_dtype(dtn), A, g)
    print("%s: %s; %s" % (where, check_grad(gQ, dQ_o, "dQ", where), check_grad(gD, dD_o, "dD", where)), flush=True)


def test_noalloc_matches_bwd_two_calls(bd):
    # first: the training shape's document length, hot rows (the heavy-row list in scratch)
    Q, D, A, g = case(2101, 16, 1024, 8, 1024, inputs.BF16, hot=0.3)
    ref, got = run_both(bd, Q, D, A, g, inputs.BF16)
    check(ref, got, Q, D, A, g, inputs.BF16, "noalloc first call")
    # second, smaller: few query rows, so dQ is split over document chunks
    # whose partial sums also live in the scratch array
    Q, D, A, g = case(2102, 1, 32, 300, 100, inputs.F16)
    ref, got = run_both(bd, Q, D, A, g, inputs.F16)
    check(ref, got, Q, D, A, g, inputs.F16, "noalloc second call")


def test_noalloc_training_step(bd):
    """The training workload's backward (64 x 64 pairs, Lq = Ld = 1024) through
    the allocation-free entry point equals maxsim_bwd bit for bit."""
    w = inputs.make("contrastive_train")
    Nq, Lq, B, Ld = w["Nq"], w["Lq"], w["B"], w["Ld_max"]
    D = w["D_packed"].reshape(B, Ld, 128)
    rng = np.random.default_rng([0, 4, 9])
    A = rng.integers(0, Ld, size=(Nq, B, Lq)).astype(np.int32)
    g = infonce_grad(rng.standard_normal((Nq, B)) * 0.05, w["tau"]).astype(np.float32)
    ref, got = run_both(bd, w["Q"], D, A, g, inputs.BF16)
    for r, x, n in zip(ref, got, ("dQ", "dD", "row_ptr", "col_idx")):
        assert np.array_equal(r, x), "training shape: %s differs from maxsim_bwd" % n


def test_noalloc_refuses_a_shape_beyond_its_scratch(bd):
    Q = torch.zeros((1, 32, 128), dtype=torch.float16, device="cuda:0")
    D = torch.zeros((100000, 180, 128), dtype=torch.float16, device="cuda:0")
    A = torch.zeros((1, 100000, 32), dtype=torch.int32, device="cuda:0")
    g = torch.zeros((1, 100000), device="cuda:0")
    dQ = torch.empty((1, 32, 128), device="cuda:0")
    dD = torch.empty((100000, 180, 128), device="cuda:0")
    rp = torch.empty(100000 * 180 + 1, dtype=torch.int32, device="cuda:0")
    ci = torch.empty(100000 * 32, dtype=torch.int32, device="cuda:0")
    with pytest.raises(bd.MaxSimError) as e:
        bd.maxsim_bwd_noalloc(Q, D, A, g, dQ, dD, rp, ci)
    assert e.value.status == bd.MAXSIM_ERR_SCRATCH
