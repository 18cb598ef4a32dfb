"""GPU parity of the backward: inverse-grid CSR (bit-exact), destination-owned
dD and gathered dQ (relative Frobenius error <= 1e-3, exact zeros on rows no
query token selected), through the C ABI.  Run on an MI355X: pytest -m gpu.

Both sides get the same argmax and upstream gradient, taken from the oracle
or from seeded generators, so a legitimate near-tie argmax difference of the
forward cannot re-route a row."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from late_interaction_retrieval_amd import inputs
from gpu_util import GRAD_REL_TOL, check_grad, infonce_grad, oracle_dtype, pad_width, rel_fro, to_dev

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden", "maxsim_hand.json")


@pytest.fixture(scope="module")
def bd():
    from late_interaction_retrieval_amd import binding
    assert torch.cuda.is_available()
    return binding


def run_bwd(bd, Q, D, dtn, A, g):
    dQ, dD, rp, ci = bd.maxsim_bwd(to_dev(Q, dtn), to_dev(D, dtn), to_dev(A), to_dev(g))
    torch.cuda.synchronize()
    return dQ.cpu().numpy(), dD.cpu().numpy(), rp.cpu().numpy(), ci.cpu().numpy()


def check_bwd(bd, Q, D, dtn, A, g, where):
    dQ, dD, rp, ci = run_bwd(bd, Q, D, dtn, A, g)
    Ld = D.shape[1]
    rp_ref, ci_ref = oracle.csr_build(A, Ld)
    assert np.array_equal(rp, rp_ref), where + ": row_ptr"
    assert np.array_equal(ci[:rp_ref[-1]], ci_ref), where + ": col_idx"
    dQ_ref, dD_ref = oracle.bwd(Q, D, oracle_dtype(dtn), A, g)
    rq, rd = check_grad(dQ, dQ_ref, "dQ", where), check_grad(dD, dD_ref, "dD", where)
    empty_rows = np.diff(rp_ref).reshape(D.shape[0], Ld) == 0
    assert np.all(dD[empty_rows] == 0.0), where + ": rows without sources must be exactly 0"
    # second call: bit-identical (deterministic, atomic-free)
    dQ2, dD2, rp2, ci2 = run_bwd(bd, Q, D, dtn, A, g)
    assert np.array_equal(dQ, dQ2) and np.array_equal(dD, dD2) and np.array_equal(ci[:rp[-1]], ci2[:rp[-1]])
    print("%s: %s; %s" % (where, rq, rd), flush=True)


def test_golden_hand_case(bd):
    g = json.load(open(GOLD))
    f, bw = g["fwd_padded"], g["bwd"]
    Q = pad_width(np.array(f["Q"], np.float16))
    D = pad_width(np.array(f["D"], np.float16))
    A = np.array(f["argmax"], np.int32)
    gg = np.array(bw["g"], np.float32)
    dQ, dD, rp, ci = run_bwd(bd, Q, D, inputs.F16, A, gg)
    assert np.array_equal(rp, np.array(bw["row_ptr"]))
    assert np.array_equal(ci, np.array(bw["col_idx"]))
    assert np.array_equal(dQ[..., :2], np.array(bw["dQ"], np.float32)) and np.all(dQ[..., 2:] == 0)
    assert np.array_equal(dD[..., :2], np.array(bw["dD"], np.float32)) and np.all(dD[..., 2:] == 0)


SHAPES = [(1, 1, 1, 1), (2, 7, 3, 5), (3, 33, 4, 70), (9, 64, 5, 64), (17, 100, 3, 129), (4, 1024, 2, 1024),
          (20, 32, 7, 300), (1, 5, 1, 4096),
          # groups of 8 and 4 queries (1025..4096-row documents), and more (document, group)
          # pairs than the fill sums itself (the documents' first slots from their own scan)
          (9, 40, 3, 1500), (5, 64, 2, 3000), (1, 32, 3000, 50), (33, 16, 150, 40),
          # every number of 64-source steps per query in the fill (Lq 65 .. 1024), groups of 8
          # (Lq <= 256) and 16, and the largest fill LDS: 8 x 2048 and 16 x 1024 (query, row)
          # slots, and 4 queries per group at 4096 rows
          (20, 65, 3, 600), (40, 256, 2, 2048), (17, 257, 2, 700), (9, 513, 2, 300),
          (33, 1024, 2, 1024), (9, 1024, 2, 4096)]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
@pytest.mark.parametrize("dtn", [inputs.F16, inputs.BF16])
def test_chain_forward_argmax(bd, shape, dtn):
    """argmax and g from the oracle forward (InfoNCE-style g), then backward on both sides."""
    Nq, Lq, B, Ld = shape
    seed = 900 + sum(shape)
    Q = inputs.random_rows(seed, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    D = inputs.random_rows(seed + 1, B * Ld, 128, dtn, stream=4).reshape(B, Ld, 128)
    s, A = oracle.fwd_padded(Q, D, oracle_dtype(dtn))
    if Nq == B:
        g = infonce_grad(s, 0.02).astype(np.float32)
    else:
        g = np.random.default_rng(seed).standard_normal((Nq, B)).astype(np.float32)
    check_bwd(bd, Q, D, dtn, A, g, "%s %s" % (dtn, shape))


@pytest.mark.parametrize("shape", [(5, 40, 7, 90), (2, 16, 2500, 20)], ids=["7docs", "2500docs"])
@pytest.mark.parametrize("dtn", [inputs.F16, inputs.BF16])
def test_forward_with_empty_documents_then_backward(bd, shape, dtn):
    """Padded documents with d_lens = 0: the forward writes argmax -1 for every
    token of them, and the backward fed the forward's own output drops those
    sources (no CSR entry, no dQ term, zero dD rows), as the oracle does."""
    Nq, Lq, B, Ld = shape
    seed = 950 + B
    Q = inputs.random_rows(seed, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    D = inputs.random_rows(seed + 1, B * Ld, 128, dtn, stream=4).reshape(B, Ld, 128)
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, Ld + 1, size=B).astype(np.int32)
    lens[rng.random(B) < 0.3] = 0
    lens[1] = 0
    s, a = bd.maxsim_fwd(to_dev(Q, dtn), to_dev(D, dtn), to_dev(lens))
    torch.cuda.synchronize()
    A = a.cpu().numpy()
    assert np.all(A[:, lens == 0] == -1) and np.all(A[:, lens > 0] >= 0)
    g = rng.standard_normal((Nq, B)).astype(np.float32)
    check_bwd(bd, Q, D, dtn, A, g, "empty documents %s %s" % (dtn, shape))


def test_hot_tokens(bd):
    """Most query tokens select one of three hot document tokens (contention)."""
    Nq, Lq, B, Ld = 16, 256, 4, 512
    rng = np.random.default_rng(77)
    Q = inputs.random_rows(77, Nq * Lq, 128, inputs.BF16).reshape(Nq, Lq, 128)
    D = inputs.random_rows(78, B * Ld, 128, inputs.BF16).reshape(B, Ld, 128)
    A = rng.integers(0, Ld, size=(Nq, B, Lq)).astype(np.int32)
    hot = rng.random(A.shape) < 0.8
    A[hot] = rng.integers(0, 3, size=int(hot.sum()))
    g = rng.standard_normal((Nq, B)).astype(np.float32)
    check_bwd(bd, Q, D, inputs.BF16, A, g, "hot tokens")


def test_workload_contrastive_train_full(bd):
    """The training workload at full size (64 x 64 pairs, Lq = Ld = 1024): seeded
    argmax (uniform) and an InfoNCE-shaped upstream gradient of seeded scores."""
    w = inputs.make("contrastive_train")
    Nq, Lq, B, Ld = w["Nq"], w["Lq"], w["B"], w["Ld_max"]
    D = w["D_packed"].reshape(B, Ld, 128)
    rng = np.random.default_rng([0, 4, 7])
    A = rng.integers(0, Ld, size=(Nq, B, Lq)).astype(np.int32)
    fake_scores = rng.standard_normal((Nq, B)) * 0.05 + np.eye(Nq) * 0.1
    g = infonce_grad(fake_scores, w["tau"]).astype(np.float32)
    check_bwd(bd, w["Q"], D, inputs.BF16, A, g, "contrastive_train")


@pytest.fixture(scope="module")
def train_ref():
    """The training workload (64 x 64 pairs, Lq = Ld = 1024, bf16) and the
    oracle's forward over all 4096 pairs (about 10 s on 16 host threads)."""
    w = inputs.make("contrastive_train")
    D = w["D_packed"].reshape(w["B"], w["Ld_max"], 128)
    s_ref, a_ref, m_ref = oracle.fwd_padded(w["Q"], D, oracle.BF16, want_rowmax=True)
    return w, D, s_ref, a_ref, m_ref


def test_workload_contrastive_forward_full(bd, train_ref):
    """Forward of the training workload: every one of the 4096 pairs against
    the oracle (scores within 1e-3 * Lq, argmax equal or a near-tie)."""
    from gpu_util import check_argmax, check_scores
    w, D, s_ref, a_ref, m_ref = train_ref
    Nq, Lq, B, Ld = w["Nq"], w["Lq"], w["B"], w["Ld_max"]
    s, a = bd.maxsim_fwd(to_dev(w["Q"], inputs.BF16), to_dev(D, inputs.BF16))
    torch.cuda.synchronize()
    s, a = s.cpu().numpy(), a.cpu().numpy()
    err = check_scores(s, s_ref, Lq, "train fwd")
    cu = inputs.cu_seqlens(np.full(B, Ld, np.int32))
    sim = oracle.sim_at(w["Q"], w["D_packed"], cu, oracle.BF16, a)
    flips = check_argmax(a, a_ref, m_ref, sim, np.full(B, Ld), "train fwd")
    print("contrastive_train forward: 4096 pairs, max |dscore| %.3g, %d of %d argmax near-tie flips"
          % (err, flips, a.size), flush=True)


def test_workload_contrastive_train_chain(bd, train_ref):
    """The whole training step at full size, as the parity protocol states it:
    the GPU forward's argmax, the InfoNCE gradient computed once in fp64 from
    the oracle's scores (tau = 0.02), then the backward on both sides with
    that same argmax and gradient."""
    w, D, s_ref, _, _ = train_ref
    s, a = bd.maxsim_fwd(to_dev(w["Q"], inputs.BF16), to_dev(D, inputs.BF16))
    torch.cuda.synchronize()
    g = infonce_grad(s_ref, w["tau"]).astype(np.float32)
    check_bwd(bd, w["Q"], D, inputs.BF16, a.cpu().numpy(), g, "contrastive_train chain")


def test_workload_contrastive_train_hot_rows(bd):
    """The training shape with half of every document's sources on 8 hot rows
    (4096 sources each): those rows take the whole-workgroup path."""
    w = inputs.make("contrastive_train")
    Nq, Lq, B, Ld = w["Nq"], w["Lq"], w["B"], w["Ld_max"]
    D = w["D_packed"].reshape(B, Ld, 128)
    rng = np.random.default_rng([0, 4, 8])
    A = rng.integers(0, Ld, size=(Nq, B, Lq)).astype(np.int32)
    hot = rng.random(A.shape) < 0.5
    A[hot] = rng.integers(0, 8, size=int(hot.sum()))
    g = rng.standard_normal((Nq, B)).astype(np.float32) * 0.01
    check_bwd(bd, w["Q"], D, inputs.BF16, A, g, "contrastive_train hot rows")
