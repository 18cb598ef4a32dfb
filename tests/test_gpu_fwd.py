"""GPU parity of the fused forward (fp16 / bf16, padded and cu_seqlens) against
the CPU oracle, through the C ABI.  Run on an MI355X: pytest -m gpu."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from late_interaction_retrieval_amd import inputs
from gpu_util import (DEV, check_argmax, check_scores, oracle_dtype, pad_width, sub_corpus, to_dev)

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden", "maxsim_hand.json")


@pytest.fixture(scope="module")
def bd():
    from late_interaction_retrieval_amd import binding
    assert torch.cuda.is_available()
    return binding


def run_padded(bd, Q, D, dtn, lens=None, with_argmax=True):
    s, a = bd.maxsim_fwd(to_dev(Q, dtn), to_dev(D, dtn), None if lens is None else to_dev(lens),
                         with_argmax=with_argmax)
    torch.cuda.synchronize()
    return s.cpu().numpy(), (a.cpu().numpy() if a is not None else None)


def run_varlen(bd, Q, Dp, cu, dtn, with_argmax=True):
    lens = np.diff(cu)
    s, a = bd.maxsim_fwd_varlen(to_dev(Q, dtn), to_dev(Dp, dtn), to_dev(cu), max(1, int(lens.max(initial=1))),
                                with_argmax=with_argmax)
    torch.cuda.synchronize()
    return s.cpu().numpy(), (a.cpu().numpy() if a is not None else None)


def full_check_varlen(bd, Q, Dp, cu, dtn, where):
    odt = oracle_dtype(dtn)
    s_ref, a_ref, m_ref = oracle.fwd_varlen(Q, Dp, cu, odt, want_rowmax=True)
    s, a = run_varlen(bd, Q, Dp, cu, dtn)
    Lq = Q.shape[1]
    check_scores(s, s_ref, Lq, where)
    sim = oracle.sim_at(Q, Dp, cu, odt, a)
    check_argmax(a, a_ref, m_ref, sim, np.diff(cu), where)
    s2, a2 = run_varlen(bd, Q, Dp, cu, dtn, with_argmax=False)
    assert np.array_equal(s2, s), where + ": scores differ with and without argmax"
    return s, a


@pytest.mark.parametrize("dtn", [inputs.F16, inputs.BF16])
def test_golden_hand_case(bd, dtn):
    g = json.load(open(GOLD))["fwd_padded"]
    f = np.array(g["Q"], np.float32)
    dd = np.array(g["D"], np.float32)
    if dtn == inputs.F16:
        Q, D = pad_width(f.astype(np.float16)), pad_width(dd.astype(np.float16))
    else:
        Q, D = pad_width(inputs.f32_to_bf16_bits(f)), pad_width(inputs.f32_to_bf16_bits(dd))
    lens = np.array(g["d_lens"], np.int32)
    s, a = run_padded(bd, Q, D, dtn, lens)
    assert np.array_equal(s, np.array(g["scores"], np.float32))
    assert np.array_equal(a, np.array(g["argmax"]))
    cu = inputs.cu_seqlens(lens)
    Dp = np.concatenate([D[b, :lens[b]] for b in range(len(lens))])
    s, a = run_varlen(bd, Q, Dp, cu, dtn)
    assert np.array_equal(s, np.array(g["scores"], np.float32))
    assert np.array_equal(a, np.array(g["argmax"]))


SHAPES = [  # Nq, Lq, B, (Ld lo, hi)
    (1, 1, 3, (1, 1)),
    (1, 7, 5, (1, 40)),
    (2, 16, 7, (16, 16)),
    (1, 32, 40, (100, 180)),
    (3, 31, 9, (0, 70)),
    (5, 33, 11, (1, 129)),
    (40, 32, 17, (32, 300)),
    (3, 128, 6, (60, 200)),
    (2, 300, 4, (1, 513)),
    # 513..768 tokens: whole queries in 768-row slabs (three 32-row blocks per wave)
    (2, 513, 5, (0, 300)),
    (1, 600, 4, (1, 700)),
    (3, 768, 3, (250, 260)),
    (1, 1024, 3, (1000, 1100)),
    (2, 1000, 2, (64, 64)),
    # short queries (one 32-row block each): documents packed by 32-token
    # sub-tile, many empty / one-token documents, bounds chunks crossed
    (17, 24, 300, (0, 100)),
    (2, 17, 5000, (1, 40)),
    (16, 32, 2100, (0, 3)),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
@pytest.mark.parametrize("dtn", [inputs.F16, inputs.BF16])
def test_random_shapes_varlen_and_padded(bd, shape, dtn):
    Nq, Lq, B, (lo, hi) = shape
    seed = sum(shape[:3]) + lo + hi
    Q = inputs.random_rows(seed, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    lens = np.random.default_rng(seed).integers(lo, hi + 1, size=B).astype(np.int32)
    cu = inputs.cu_seqlens(lens)
    Dp = inputs.random_rows(seed + 1, int(cu[-1]), 128, dtn, stream=4)
    where = "%s %s" % (dtn, shape)
    s, a = full_check_varlen(bd, Q, Dp, cu, dtn, where)
    # padded + d_lens gives bit-identical results (same tiles, same order)
    Ld = max(1, int(lens.max()))
    Dpad = inputs.pad_packed(Dp, cu, Ld)
    s2, a2 = run_padded(bd, Q, Dpad, dtn, lens)
    assert np.array_equal(s2, s) and np.array_equal(a2, a), where + ": padded != varlen"


# Skewed corpora for the split of documents into streams (contiguous ranges
# balanced by tokens plus a per-document cost): a long run of empty documents
# first, then short ones, then a few long ones; 32-token queries (scores
# summed in registers) and 40-token queries (summed through LDS); and more
# documents than two rounds of the workgroup search cover (B > 512^2).
SKEWED = [  # Nq, Lq, B, empty, short (lo, hi), long, (lo, hi)
    (3, 32, 5000, 3000, (1, 40), 100, (200, 600)),
    (3, 40, 5000, 3000, (1, 40), 100, (200, 600)),
    (20, 32, 1200, 10, (32, 300), 2, (3000, 4000)),
    (2, 32, 300000, 0, (0, 2), 0, (0, 0)),
    (33, 32, 700, 0, (32, 32), 0, (0, 0)),
    (16, 32, 3, 1, (1, 1), 1, (256, 256)),
    (64, 32, 2000, 200, (0, 64), 50, (255, 513)),
]


@pytest.mark.parametrize("shape", SKEWED, ids=[str(s) for s in SKEWED])
def test_skewed_corpus_stream_split(bd, shape):
    Nq, Lq, B, n_empty, (slo, shi), n_long, (llo, lhi) = shape
    rng = np.random.default_rng(B + Lq)
    lens = np.zeros(B, np.int32)
    n_short = B - n_empty - n_long
    lens[n_empty:n_empty + n_short] = rng.integers(slo, shi + 1, size=n_short)
    lens[B - n_long:] = rng.integers(llo, lhi + 1, size=n_long)
    cu = inputs.cu_seqlens(lens)
    Q = inputs.random_rows(B + 1, Nq * Lq, 128, inputs.F16).reshape(Nq, Lq, 128)
    Dp = inputs.random_rows(B + 2, int(cu[-1]), 128, inputs.F16, stream=4)
    # every score is written: prefill with NaN, which no document can give
    scores = torch.full((Nq, B), float("nan"), dtype=torch.float32, device=DEV)
    s, a = bd.maxsim_fwd_varlen(to_dev(Q, inputs.F16), to_dev(Dp, inputs.F16), to_dev(cu), max(1, int(lens.max())),
                                scores=scores)
    torch.cuda.synchronize()
    s, a = s.cpu().numpy(), a.cpu().numpy()
    assert not np.isnan(s).any(), "some documents were never scored"
    s_ref, a_ref, m_ref = oracle.fwd_varlen(Q, Dp, cu, oracle.F16, want_rowmax=True)
    where = "skewed %s" % (shape,)
    check_scores(s, s_ref, Lq, where)
    check_argmax(a, a_ref, m_ref, oracle.sim_at(Q, Dp, cu, oracle.F16, a), lens, where)
    # scores only (for 32-token queries: tiles that run across documents)
    scores.fill_(float("nan"))
    s0, _ = bd.maxsim_fwd_varlen(to_dev(Q, inputs.F16), to_dev(Dp, inputs.F16), to_dev(cu), max(1, int(lens.max())),
                                 scores=scores, with_argmax=False)
    torch.cuda.synchronize()
    assert np.array_equal(s0.cpu().numpy(), s), where + ": scores differ without the argmax"


@pytest.mark.parametrize("dtn", [inputs.F16, inputs.BF16])
@pytest.mark.parametrize("Lq", [64, 600])
def test_very_long_documents(bd, dtn, Lq):
    """Documents of 100000 and 70000 tokens (390 and 274 tiles each) beside a
    5-token one: tile offsets and sub-tile codes far from zero, one document
    per stream, packed and padded (with d_lens) bit for bit."""
    Nq = 2
    lens = np.array([100000, 5, 70000], np.int32)
    cu = inputs.cu_seqlens(lens)
    Q = inputs.random_rows(31 + Lq, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    Dp = inputs.random_rows(32 + Lq, int(cu[-1]), 128, dtn, stream=4)
    s, a = bd.maxsim_fwd_varlen(to_dev(Q, dtn), to_dev(Dp, dtn), to_dev(cu), int(lens.max()))
    torch.cuda.synchronize()
    s, a = s.cpu().numpy(), a.cpu().numpy()
    s_ref, a_ref, m_ref = oracle.fwd_varlen(Q, Dp, cu, oracle_dtype(dtn), want_rowmax=True)
    where = "long documents %s Lq %d" % (dtn, Lq)
    check_scores(s, s_ref, Lq, where)
    check_argmax(a, a_ref, m_ref, oracle.sim_at(Q, Dp, cu, oracle_dtype(dtn), a), lens, where)
    # padded: the same rows in [3, 100000] with d_lens
    Dpad = np.zeros((3, int(lens.max()), 128), Dp.dtype)
    for b in range(3):
        Dpad[b, :lens[b]] = Dp[cu[b]:cu[b + 1]]
    s2, a2 = bd.maxsim_fwd(to_dev(Q, dtn), to_dev(Dpad, dtn), to_dev(lens))
    torch.cuda.synchronize()
    assert np.array_equal(s2.cpu().numpy(), s) and np.array_equal(a2.cpu().numpy(), a), where + ": padded differs"


@pytest.mark.parametrize("dtn", [inputs.F16, inputs.BF16])
@pytest.mark.parametrize("Nq,Lq", [(20, 32), (1, 32), (2, 16), (1, 7)])
def test_first_token_max_ragged_tails(bd, dtn, Nq, Lq):
    """Every document starts with the token closest to every query row, with
    partial 32-token (and, for the few-row kernel, 16-token) sub-tiles.  Rows
    past a document's end are read as copies of its first token; the maxima
    must not change and every argmax must stay inside the document."""
    # one unit query row repeated, and that row as every document's first
    # token: similarity 1 at token 0, about N(0, 1/128) elsewhere
    row = inputs.random_rows(63, 1, 128, dtn)
    Q = np.repeat(row, Nq * Lq, axis=0).reshape(Nq, Lq, 128)
    lens = np.array([1, 15, 17, 31, 33, 47, 100, 129, 255, 257, 300], np.int32)
    cu = inputs.cu_seqlens(lens)
    Dp = inputs.random_rows(64, int(cu[-1]), 128, dtn, stream=4)
    for b in range(len(lens)):
        Dp[cu[b]] = row[0]
    s, a = full_check_varlen(bd, Q, Dp, cu, dtn, "first-token max %s Nq %d Lq %d" % (dtn, Nq, Lq))
    assert np.all(a == 0)


def test_many_documents_per_stream(bd):
    """64 queries x 32 tokens over 300000 documents of 0..2 tokens: about 4700
    documents per stream, more than the scores-only kernel keeps in LDS, so it
    reads document ends from memory.  Scores-only equals the argmax launch bit
    for bit; a seeded sample of documents is checked against the oracle."""
    Nq, Lq, B = 64, 32, 300000
    rng = np.random.default_rng(77)
    lens = rng.integers(0, 3, size=B).astype(np.int32)
    cu = inputs.cu_seqlens(lens)
    Q = inputs.random_rows(78, Nq * Lq, 128, inputs.F16).reshape(Nq, Lq, 128)
    Dp = inputs.random_rows(79, int(cu[-1]), 128, inputs.F16, stream=4)
    Qd, Dd, cud = to_dev(Q, inputs.F16), to_dev(Dp, inputs.F16), to_dev(cu)
    scores = torch.full((Nq, B), float("nan"), dtype=torch.float32, device=DEV)
    s0, _ = bd.maxsim_fwd_varlen(Qd, Dd, cud, 2, scores=scores, with_argmax=False)
    s1, a1 = bd.maxsim_fwd_varlen(Qd, Dd, cud, 2)
    torch.cuda.synchronize()
    s0, s1, a1 = s0.cpu().numpy(), s1.cpu().numpy(), a1.cpu().numpy()
    assert not np.isnan(s0).any()
    assert np.array_equal(s0, s1)
    docs = np.sort(rng.choice(B, size=2000, replace=False))
    docs[0], docs[-1] = 0, B - 1
    sub, subcu = sub_corpus(Dp, cu, docs)
    s_ref, a_ref, m_ref = oracle.fwd_varlen(Q, sub, subcu, oracle.F16, want_rowmax=True)
    check_scores(s0[:, docs], s_ref, Lq, "many documents per stream")
    check_argmax(a1[:, docs], a_ref, m_ref, oracle.sim_at(Q, sub, subcu, oracle.F16, a1[:, docs]), np.diff(subcu),
                 "many documents per stream")


def test_padding_never_selected_all_negative(bd):
    """All valid similarities negative, padding rows huge: padding is never picked."""
    Q = np.full((2, 40, 128), 0.05, np.float16)
    D = np.full((3, 70, 128), -0.02, np.float16)
    D[:, 50:] = 30.0
    D[1, 17] = -0.01
    lens = np.array([50, 50, 0], np.int32)
    s, a = run_padded(bd, Q, D, inputs.F16, lens)
    s_ref, a_ref = oracle.fwd_padded(Q, D, oracle.F16, d_lens=lens)
    check_scores(s, s_ref, 40, "all-negative")
    # document 0: every valid token ties, any of them is a correct argmax
    assert np.all((a[:, 0] >= 0) & (a[:, 0] < 50))
    assert np.all(a[:, 1] == 17) and np.all(a[:, 2] == -1)
    assert np.all(np.isneginf(s[:, 2]))


@pytest.mark.parametrize("dtn", [inputs.F16, inputs.BF16])
def test_signed_basis_gives_exactly_lq(bd, dtn):
    d, Lq = 128, 96
    rng = np.random.default_rng(5)
    ks = rng.integers(0, d, size=Lq)
    sg = rng.choice([-1.0, 1.0], size=Lq).astype(np.float32)
    Qf = np.zeros((1, Lq, d), np.float32)
    Qf[0, np.arange(Lq), ks] = sg
    others = inputs.random_rows(6, 300, d, dtn)
    if dtn == inputs.F16:
        Q, basis = Qf.astype(np.float16), Qf[0].astype(np.float16)
    else:
        Q, basis = inputs.f32_to_bf16_bits(Qf), inputs.f32_to_bf16_bits(Qf[0])
    Dp = np.concatenate([others[:150], basis, others[150:]])
    Dp = Dp[rng.permutation(len(Dp))]
    cu = np.array([0, len(Dp)], np.int32)
    s, a = run_varlen(bd, Q, Dp, cu, dtn)
    assert s[0, 0] == np.float32(Lq)


def test_deterministic_reruns(bd):
    Q = inputs.random_rows(70, 64 * 32, 128, inputs.F16).reshape(64, 32, 128)
    lens = inputs.lengths(0, 70, 300, 32, 300)
    cu = inputs.cu_seqlens(lens)
    Dp = inputs.random_rows(71, int(cu[-1]), 128, inputs.F16)
    s1, a1 = run_varlen(bd, Q, Dp, cu, inputs.F16)
    s2, a2 = run_varlen(bd, Q, Dp, cu, inputs.F16)
    assert np.array_equal(s1, s2) and np.array_equal(a1, a2)


# ---------------------------------------------------------------------------
# Workload-sized runs: the GPU runs the whole workload in the same launch
# configuration the benchmark times; the oracle checks a seeded sample of
# documents (all of them for the tiny workload).
# ---------------------------------------------------------------------------
def sampled_check(bd, w, docs, where):
    dtn = w["dtype"]
    Q, Dp, cu = w["Q"], w["D_packed"], w["cu_seqlens"]
    s, a = run_varlen(bd, Q, Dp, cu, dtn)
    sub, subcu = sub_corpus(Dp, cu, docs)
    odt = oracle_dtype(dtn)
    s_ref, a_ref, m_ref = oracle.fwd_varlen(Q, sub, subcu, odt, want_rowmax=True)
    check_scores(s[:, docs], s_ref, w["Lq"], where)
    sim = oracle.sim_at(Q, sub, subcu, odt, a[:, docs])
    flips = check_argmax(a[:, docs], a_ref, m_ref, sim, np.diff(subcu), where)
    print("%s: %d docs checked, %d argmax near-tie flips" % (where, len(docs), flips), flush=True)
    return s, a


def test_workload_colbert_tiny_full(bd):
    w = inputs.make("colbert_tiny")
    sampled_check(bd, w, np.arange(w["B"]), "colbert_tiny")
    # the padded path (fixed Ld = 180) gives the same bits
    Dpad = w["D_packed"].reshape(w["B"], 180, 128)
    s, a = run_padded(bd, w["Q"], Dpad, inputs.F16)
    s2, a2 = run_varlen(bd, w["Q"], w["D_packed"], w["cu_seqlens"], inputs.F16)
    assert np.array_equal(s, s2) and np.array_equal(a, a2)


def test_workload_colbert_rerank_varlen_full(bd):
    """The re-ranking workload at full size: 64 queries x 10,000 documents of
    32..300 tokens, every score and argmax against the oracle."""
    w = inputs.make("colbert_rerank_varlen")
    s, _ = sampled_check(bd, w, np.arange(w["B"]), "colbert_rerank_varlen")
    # the launch the benchmark times (no argmax) writes every score, and the
    # same bits as with the argmax
    scores = torch.full((w["Nq"], w["B"]), float("nan"), dtype=torch.float32, device=DEV)
    s0, _ = bd.maxsim_fwd_varlen(to_dev(w["Q"], inputs.F16), to_dev(w["D_packed"], inputs.F16),
                                 to_dev(w["cu_seqlens"]), 300, scores=scores, with_argmax=False)
    torch.cuda.synchronize()
    assert np.array_equal(s0.cpu().numpy(), s)
    # padded to 300 with d_lens (the padded comparison run): identical scores
    Dpad = inputs.pad_packed(w["D_packed"], w["cu_seqlens"], 300)
    s2, _ = run_padded(bd, w["Q"], Dpad, inputs.F16, w["lens"], with_argmax=False)
    assert np.array_equal(s, s2)


def stream_edge_docs(B, nstreams, rng, n):
    """n seeded document indices of B, always including the first and last
    document and both sides of several stream boundaries of a grid that
    splits the documents into nstreams contiguous ranges."""
    edges = [(k * B) // nstreams for k in range(1, nstreams)]
    pick = set([0, B - 1])
    for e in edges:
        pick.update([e - 1, e])
    for b in rng.permutation(B):
        if len(pick) >= n:
            break
        pick.add(int(b))
    return np.array(sorted(pick))


def test_workload_colpali_subset(bd):
    """ColPali at full size on the GPU (4 x 1024-token queries, 10,000 documents
    of 1024 tokens, bf16, argmax, the benchmark's launch); a seeded subset of
    1,000 documents, including both sides of stream boundaries, through the
    oracle."""
    w = inputs.make("colpali_fwd")
    docs = stream_edge_docs(w["B"], 32, np.random.default_rng(11), 1000)
    assert len(docs) == 1000
    sampled_check(bd, w, docs, "colpali_fwd")


def test_workload_contrastive_train_varlen_forward(bd):
    """The ragged training workload's forward (64 queries x 1024 tokens, 64 packed
    documents of 256..1024 tokens, bf16, argmax): 12 documents through the oracle."""
    w = inputs.make("contrastive_train_varlen")
    docs = np.sort(np.random.default_rng(3).choice(w["B"], size=12, replace=False))
    sampled_check(bd, w, docs, "contrastive_train_varlen")
