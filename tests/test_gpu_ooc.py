"""GPU parity of the out-of-core forward (corpus in host memory, streamed in
blocks through two device buffers) against the oracle, padded and packed,
through the C ABI.  Scores within 1e-3 * Lq, argmax equal or a near-tie, and
the same bits as the resident forward on the same documents.  Run on an
MI355X: pytest -m gpu."""
import numpy as np
import pytest
import torch

import oracle
from late_interaction_retrieval_amd import inputs
from gpu_util import check_argmax, check_scores, oracle_dtype, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from late_interaction_retrieval_amd import binding
    assert torch.cuda.is_available()
    return binding


def host_t(a, dtn, pinned):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if dtn == inputs.BF16 else torch.from_numpy(a)
    return t.pin_memory() if pinned else t


PADDED = [  # (Nq, Lq, B, Ld, block_docs, with d_lens)
    (1, 32, 37, 60, 8, False),
    (2, 100, 50, 33, 50, True),
    (3, 17, 20, 129, 64, False),
    (1, 1024, 9, 300, 4, True),
    (4, 40, 13, 16, 1, False),
]


@pytest.mark.parametrize("case", PADDED, ids=[str(c) for c in PADDED])
@pytest.mark.parametrize("dtn", [inputs.F16, inputs.BF16])
def test_padded(bd, case, dtn):
    Nq, Lq, B, Ld, blk, use_lens = case
    seed = 2100 + Nq + Lq + B
    Q = inputs.random_rows(seed, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    D = inputs.random_rows(seed + 1, B * Ld, 128, dtn, stream=4).reshape(B, Ld, 128)
    lens = np.random.default_rng(seed).integers(0, Ld + 1, B).astype(np.int32) if use_lens else None
    Qd = to_dev(Q, dtn)
    ld_dev = None if lens is None else to_dev(lens)
    Dh = host_t(D, dtn, pinned=True)  # held until the copies have run
    s, a = bd.maxsim_fwd_host_stream(Qd, Dh, blk, d_lens=ld_dev, with_argmax=True)
    s_res, a_res = bd.maxsim_fwd(Qd, to_dev(D, dtn), ld_dev)
    torch.cuda.synchronize()
    s, a = s.cpu().numpy(), a.cpu().numpy()
    assert np.array_equal(s, s_res.cpu().numpy()) and np.array_equal(a, a_res.cpu().numpy())
    L = np.full(B, Ld, np.int32) if lens is None else lens
    cu = inputs.cu_seqlens(L)
    Dp = np.concatenate([D[b, :L[b]] for b in range(B)]) if cu[-1] else D[0, :0]
    s_ref, a_ref, m_ref = oracle.fwd_varlen(Q, Dp, cu, oracle_dtype(dtn), want_rowmax=True)
    check_scores(s, s_ref, Lq, "ooc padded")
    sim = oracle.sim_at(Q, Dp, cu, oracle_dtype(dtn), a)
    check_argmax(a, a_ref, m_ref, sim, L, "ooc padded")


PACKED = [  # (Nq, Lq, lengths, max_Ld, block_docs)
    (2, 32, [5, 0, 40, 17, 0, 0, 33, 1], 40, 3),
    (1, 64, [300] * 7 + [12], 300, 2),
    (3, 20, [0, 0, 0], 4, 2),
    (5, 33, list(range(0, 90, 7)), 100, 16),
]


@pytest.mark.parametrize("case", PACKED, ids=[str(c[:2]) + "x%d" % len(c[2]) for c in PACKED])
@pytest.mark.parametrize("pinned,dtn", [(True, inputs.F16), (False, inputs.F16), (True, inputs.BF16)],
                         ids=["pinned-f16", "pageable-f16", "pinned-bf16"])
def test_packed(bd, case, pinned, dtn):
    Nq, Lq, lens, max_Ld, blk = case
    seed = 2200 + Nq + Lq + len(lens)
    Q = inputs.random_rows(seed, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    cu = inputs.cu_seqlens(np.asarray(lens, np.int32))
    Dp = inputs.random_rows(seed + 1, max(int(cu[-1]), 1), 128, dtn, stream=4)[:int(cu[-1])]
    Qd, cud = to_dev(Q, dtn), to_dev(cu)
    Dh = host_t(Dp, dtn, pinned)
    s, a = bd.maxsim_fwd_host_stream(Qd, Dh, blk, cu_seqlens_host=torch.from_numpy(cu), cu_seqlens=cud,
                                     max_Ld=max_Ld, with_argmax=True)
    s_res, a_res = bd.maxsim_fwd_varlen(Qd, to_dev(Dp, dtn), cud, max_Ld)
    torch.cuda.synchronize()
    s, a = s.cpu().numpy(), a.cpu().numpy()
    assert np.array_equal(s, s_res.cpu().numpy()) and np.array_equal(a, a_res.cpu().numpy())
    s_ref, a_ref, m_ref = oracle.fwd_varlen(Q, Dp, cu, oracle_dtype(dtn), want_rowmax=True)
    check_scores(s, s_ref, Lq, "ooc packed")
    sim = oracle.sim_at(Q, Dp, cu, oracle_dtype(dtn), a)
    check_argmax(a, a_ref, m_ref, sim, np.asarray(lens), "ooc packed")


def test_back_to_back_calls_share_staging(bd):
    """Two calls on one stream with one staging buffer: the second may not
    overwrite a block the first is still scoring."""
    dtn = inputs.BF16
    Nq, Lq, B, Ld, blk = 2, 64, 40, 200, 6
    Q = inputs.random_rows(7, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    D1 = inputs.random_rows(8, B * Ld, 128, dtn, stream=4).reshape(B, Ld, 128)
    D2 = inputs.random_rows(9, B * Ld, 128, dtn, stream=4).reshape(B, Ld, 128)
    Qd = to_dev(Q, dtn)
    staging = torch.empty(bd.maxsim_fwd_host_stream_staging_bytes(Nq, Lq, Ld, blk, False), dtype=torch.uint8,
                          device="cuda:0")
    H1, H2 = host_t(D1, dtn, True), host_t(D2, dtn, True)
    s1, _ = bd.maxsim_fwd_host_stream(Qd, H1, blk, staging=staging)
    s2, _ = bd.maxsim_fwd_host_stream(Qd, H2, blk, staging=staging)
    torch.cuda.synchronize()
    for s, D in ((s1, D1), (s2, D2)):
        s_ref, _ = oracle.fwd_padded(Q, D, oracle.BF16)
        check_scores(s.cpu().numpy(), s_ref, Lq, "back to back")


def test_colpali_query_sampled(bd):
    """The ColPali shape the pages stream (Lq = Ld = 1024, bf16), one query
    against 600 host documents in blocks of 256 (a ragged last block), all
    scores checked against the oracle on a sample of 24 documents."""
    w = inputs.make("colpali_fwd", Nq=1, B=600)
    B, Ld = w["B"], w["Ld_max"]
    D = w["D_packed"].reshape(B, Ld, 128)
    Qd = to_dev(w["Q"], inputs.BF16)
    Dh = host_t(D, inputs.BF16, True)
    s, a = bd.maxsim_fwd_host_stream(Qd, Dh, 256, with_argmax=True)
    torch.cuda.synchronize()
    s, a = s.cpu().numpy(), a.cpu().numpy()
    docs = np.sort(np.random.default_rng(5).choice(B, 24, replace=False))
    s_ref, a_ref, m_ref = oracle.fwd_padded(w["Q"], D[docs], oracle.BF16, want_rowmax=True)
    check_scores(s[:, docs], s_ref, 1024, "colpali ooc")
    cu = inputs.cu_seqlens(np.full(len(docs), Ld, np.int32))
    sim = oracle.sim_at(w["Q"], D[docs].reshape(-1, 128), cu, oracle.BF16, a[:, docs])
    check_argmax(a[:, docs], a_ref, m_ref, sim, np.full(len(docs), Ld), "colpali ooc")
