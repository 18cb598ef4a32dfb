"""GPU parity of the Chamfer distance (paper Section 4.2, "Generalization to
Chamfer Distance") against the oracle, through the C ABI.

Forward: every squared distance within 1e-6 relative of the oracle's (fp32
arithmetic on fp32 points: a few ulps), and every index equal to the
oracle's or a near-tie (its exact distance within 2e-6 relative of the
minimum).  Backward: both CSR maps bit-exact, gradients within 1e-5 relative
Frobenius error; the selections fed to both sides come from the oracle or a
seeded generator.  Run on an MI355X: pytest -m gpu."""
import numpy as np
import pytest
import torch

import oracle
from late_interaction_retrieval_amd import inputs
from gpu_util import rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
DIST_REL = 1e-6
TIE_REL = 2e-6
GRAD_REL = 1e-5


@pytest.fixture(scope="module")
def bd():
    from late_interaction_retrieval_amd import binding
    assert torch.cuda.is_available()
    return binding


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def exact_dist(A, B, idx):
    """fp64 squared distance from every A point to B[idx] (idx >= 0)."""
    out = np.empty(idx.shape, np.float64)
    for b in range(A.shape[0]):
        out[b] = ((A[b].astype(np.float64) - B[b][idx[b]].astype(np.float64)) ** 2).sum(1)
    return out


def check_direction(A, B, dist, idx, where, sample=None):
    rows = slice(None) if sample is None else sample
    d_ref, i_ref = oracle.chamfer_nn(A[:, rows], B)
    dist, idx = dist[:, rows], idx[:, rows]
    if B.shape[1] == 0:
        assert np.all(np.isposinf(dist)) and np.all(idx == -1), where
        return 0
    assert np.all((idx >= 0) & (idx < B.shape[1])), where + ": index out of range"
    err = np.abs(dist.astype(np.float64) - d_ref)
    assert np.all(err <= DIST_REL * d_ref), "%s: max rel dist err %.3g" % (where, (err / np.maximum(d_ref, 1e-30)).max())
    diff = idx != i_ref
    if diff.any():
        d_at = exact_dist(A[:, rows], B, idx)
        assert np.all(d_at[diff] <= d_ref[diff] * (1 + TIE_REL)), where + ": index is not a near-tie"
    return int(diff.sum())


# (16, 100, 20000): the P -> Q direction fills the chip with 8 source points
# per lane and Q -> P takes 4, so the two run as separate launches
SHAPES = [(1, 1, 1), (1, 50, 70), (3, 33, 17), (2, 200, 5), (2, 3000, 17), (1, 2049, 513), (1, 5000, 4000),
          (4, 16, 2100), (2, 10, 0), (2, 0, 10), (16, 100, 20000)]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_forward(bd, shape):
    Bt, N, M = shape
    P, Q = inputs.point_clouds(300 + N + M, Bt, N, M)
    dp, ip, dq, iq = (t.cpu().numpy() for t in bd.maxsim_chamfer_fwd(dev(P), dev(Q)))
    torch.cuda.synchronize()
    n1 = check_direction(P, Q, dp, ip, "P->Q %s" % (shape,)) if N else 0
    n2 = check_direction(Q, P, dq, iq, "Q->P %s" % (shape,)) if M else 0
    print("%s: near-tie index differences %d, %d" % (shape, n1, n2), flush=True)


def test_forward_integer_grid_ties(bd):
    """Small-integer coordinates make every distance exact in fp32: equal
    distances are exact ties, and the first index must win, bit for bit."""
    rng = np.random.default_rng(9)
    P = rng.integers(-3, 4, (2, 300, 3)).astype(np.float32)
    Q = rng.integers(-3, 4, (2, 257, 3)).astype(np.float32)
    dp, ip, dq, iq = (t.cpu().numpy() for t in bd.maxsim_chamfer_fwd(dev(P), dev(Q)))
    d_ref, i_ref = oracle.chamfer_nn(P, Q)
    assert np.array_equal(ip, i_ref) and np.array_equal(dp.astype(np.float64), d_ref)
    d_ref, i_ref = oracle.chamfer_nn(Q, P)
    assert np.array_equal(iq, i_ref) and np.array_equal(dq.astype(np.float64), d_ref)


def run_bwd(bd, P, Q, ip, iq, gp, gq):
    out = bd.maxsim_chamfer_bwd(dev(P), dev(Q), dev(ip), dev(iq), dev(gp), dev(gq))
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def check_bwd(bd, P, Q, ip, iq, gp, gq, where):
    dP, dQ, rp_p, ci_p, rp_q, ci_q = run_bwd(bd, P, Q, ip, iq, gp, gq)
    N, M = P.shape[1], Q.shape[1]
    r, c = oracle.chamfer_csr(iq, N)
    assert np.array_equal(rp_p, r) and np.array_equal(ci_p[:r[-1]], c), where + ": CSR of P"
    r, c = oracle.chamfer_csr(ip, M)
    assert np.array_equal(rp_q, r) and np.array_equal(ci_q[:r[-1]], c), where + ": CSR of Q"
    dP_ref, dQ_ref = oracle.chamfer_bwd(P, Q, ip, iq, gp, gq)
    ep, eq = rel_fro(dP, dP_ref), rel_fro(dQ, dQ_ref)
    assert ep <= GRAD_REL and eq <= GRAD_REL, "%s: rel err dP %.3g dQ %.3g" % (where, ep, eq)
    again = run_bwd(bd, P, Q, ip, iq, gp, gq)
    assert all(np.array_equal(x, y) for x, y in zip((dP, dQ, rp_p, rp_q), again[:2] + again[2::2]))
    print("%s: rel err dP %.2e dQ %.2e" % (where, ep, eq), flush=True)


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 50, 70), (3, 33, 17), (2, 3000, 17), (1, 5000, 4000)],
                         ids=str)
def test_backward_oracle_selections(bd, shape):
    Bt, N, M = shape
    P, Q = inputs.point_clouds(400 + N, Bt, N, M)
    _, ip, _, iq = oracle.chamfer(P, Q)
    rng = np.random.default_rng(N + M)
    gp = rng.standard_normal((Bt, N)).astype(np.float32)
    gq = rng.standard_normal((Bt, M)).astype(np.float32)
    check_bwd(bd, P, Q, ip, iq, gp, gq, "bwd %s" % (shape,))


def test_backward_hot_destination_and_unselected(bd):
    """Every Q point selects P point 0 (one bucket of all M sources), and
    some selections are -1 (they add nothing)."""
    Bt, N, M = 2, 40, 5000
    P, Q = inputs.point_clouds(77, Bt, N, M)
    rng = np.random.default_rng(77)
    ip = rng.integers(0, M, (Bt, N)).astype(np.int32)
    ip[:, ::7] = -1
    iq = np.zeros((Bt, M), np.int32)
    iq[1, ::3] = -1
    gp = rng.standard_normal((Bt, N)).astype(np.float32)
    gq = rng.standard_normal((Bt, M)).astype(np.float32)
    check_bwd(bd, P, Q, ip, iq, gp, gq, "hot destination")


def test_backward_very_hot_destinations(bd):
    """Buckets of tens of thousands of sources (every Q point selects one of two
    P points, every P point one of three Q points): the whole-workgroup path."""
    Bt, N, M = 2, 3000, 40000
    P, Q = inputs.point_clouds(88, Bt, N, M)
    rng = np.random.default_rng(88)
    ip = rng.integers(0, 3, (Bt, N)).astype(np.int32)
    iq = rng.integers(0, 2, (Bt, M)).astype(np.int32)
    iq[:, ::5] = rng.integers(0, N, (Bt, len(range(0, M, 5))))
    gp = rng.standard_normal((Bt, N)).astype(np.float32)
    gq = rng.standard_normal((Bt, M)).astype(np.float32)
    check_bwd(bd, P, Q, ip, iq, gp, gq, "very hot destinations")


def test_workload_chamfer_100k_sampled(bd):
    """100K-point clouds (the page's largest): the GPU forward on all points,
    the oracle on 1500 sampled points per direction; the backward at full size
    with seeded selections and the page's loss weights (1/N, 1/M)."""
    w = inputs.make_chamfer("chamfer_100k")
    P, Q = w["P"], w["Q"]
    dp, ip, dq, iq = (t.cpu().numpy() for t in bd.maxsim_chamfer_fwd(dev(P), dev(Q)))
    rng = np.random.default_rng(100)
    check_direction(P, Q, dp, ip, "100k P->Q", np.sort(rng.choice(w["N"], 1500, replace=False)))
    check_direction(Q, P, dq, iq, "100k Q->P", np.sort(rng.choice(w["M"], 1500, replace=False)))
    sp = rng.integers(0, w["M"], (1, w["N"])).astype(np.int32)
    sq = rng.integers(0, w["N"], (1, w["M"])).astype(np.int32)
    gp = np.full((1, w["N"]), 1.0 / w["N"], np.float32)
    gq = np.full((1, w["M"]), 1.0 / w["M"], np.float32)
    check_bwd(bd, P, Q, sp, sq, gp, gq, "100k backward")


def test_workload_chamfer_batch(bd):
    """32 pairs of 2048-point clouds: all points checked against the oracle."""
    w = inputs.make_chamfer("chamfer_batch")
    P, Q = w["P"], w["Q"]
    dp, ip, dq, iq = (t.cpu().numpy() for t in bd.maxsim_chamfer_fwd(dev(P), dev(Q)))
    check_direction(P, Q, dp, ip, "batch P->Q")
    check_direction(Q, P, dq, iq, "batch Q->P")


def test_autograd_loss(bd):
    """chamfer_distance with torch autograd: the loss and its gradients against
    the oracle's (selections from the oracle; this seed has no near-tie)."""
    P, Q = inputs.point_clouds(5, 2, 300, 200)
    Pt, Qt = dev(P).requires_grad_(True), dev(Q).requires_grad_(True)
    loss = bd.chamfer_distance(Pt, Qt)
    _, ip, _, iq = oracle.chamfer(P, Q)
    _, gip, _, giq = (t.cpu().numpy() for t in bd.maxsim_chamfer_fwd(dev(P), dev(Q)))
    assert np.array_equal(gip, ip) and np.array_equal(giq, iq), "a near-tie at this seed; pick another"
    np.testing.assert_allclose(loss.detach().cpu().numpy(), oracle.chamfer_loss(P, Q), rtol=1e-5)
    loss.sum().backward()
    gp = np.full((2, 300), 1 / 300, np.float32)
    gq = np.full((2, 200), 1 / 200, np.float32)
    dP_ref, dQ_ref = oracle.chamfer_bwd(P, Q, ip, iq, gp, gq)
    assert rel_fro(Pt.grad.cpu().numpy(), dP_ref) <= GRAD_REL
    assert rel_fro(Qt.grad.cpu().numpy(), dQ_ref) <= GRAD_REL
