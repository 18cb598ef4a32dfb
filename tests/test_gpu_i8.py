"""GPU parity of the INT8 x INT8 forward: bit-exact scores and argmax against the
oracle, through the C ABI.  Run on an MI355X: pytest -m gpu."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from late_interaction_retrieval_amd import inputs
from gpu_util import pad_width, sub_corpus, to_dev

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden", "maxsim_hand.json")


@pytest.fixture(scope="module")
def bd():
    from late_interaction_retrieval_amd import binding
    assert torch.cuda.is_available()
    return binding


def run_i8(bd, Q, qs, Dp, ds, cu, with_argmax=True):
    lens = np.diff(cu)
    s, a = bd.maxsim_fwd_i8(to_dev(Q), to_dev(qs), to_dev(Dp), to_dev(ds), to_dev(cu),
                            max(1, int(lens.max(initial=1))), with_argmax=with_argmax)
    torch.cuda.synchronize()
    return s.cpu().numpy(), (a.cpu().numpy() if a is not None else None)


def assert_bits_equal(got, ref, where):
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    bad = got.view(np.uint32) != ref.view(np.uint32)
    assert not bad.any(), "%s: %d scores differ, first at %s: %r vs %r" % (
        where, int(bad.sum()), np.argwhere(bad)[0], got[bad][0], ref[bad][0])


def test_golden_hand_case(bd):
    g = json.load(open(GOLD))["fwd_i8"]
    Q = pad_width(np.array(g["Q"], np.int8))
    Dp = pad_width(np.array(g["D"], np.int8))
    s, a = run_i8(bd, Q, np.array(g["q_scale"], np.float32), Dp, np.array(g["d_scale"], np.float32),
                  np.array(g["cu_seqlens"], np.int32))
    exp = np.array([[float(v) for v in row] for row in g["scores"]], np.float32)
    assert_bits_equal(s, exp, "golden")
    assert np.array_equal(a, np.array(g["argmax"]))


SHAPES = [(1, 1, 4, (1, 3)), (2, 7, 9, (0, 40)), (3, 32, 20, (32, 512)), (40, 32, 13, (1, 100)),
          (1, 300, 5, (10, 600)), (2, 1024, 3, (100, 200)),
          # more queries in a slab than threads in the workgroup (single-token queries:
          # the per-query sums wrap around the workgroup), and two slabs of 512 queries
          (600, 1, 7, (1, 300)), (520, 2, 3, (5, 90)),
          # the thread-per-query sums: 8-row groups at one address (1, 3, 5 and 7 groups)
          # and, for a length that is no multiple of 8, the row-by-row read-ahead
          (5, 8, 9, (0, 50)), (3, 24, 7, (10, 200)), (2, 40, 6, (1, 520)), (2, 56, 5, (30, 300)),
          (4, 20, 11, (1, 300))]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_random_shapes_bit_exact(bd, shape):
    Nq, Lq, B, (lo, hi) = shape
    seed = 500 + sum(shape[:3]) + lo + hi
    Q, qs = inputs.random_rows(seed, Nq * Lq, 128, inputs.I8)
    lens = np.random.default_rng(seed).integers(lo, hi + 1, size=B).astype(np.int32)
    cu = inputs.cu_seqlens(lens)
    Dp, ds = inputs.random_rows(seed + 1, int(cu[-1]), 128, inputs.I8, stream=4)
    Q, qs = Q.reshape(Nq, Lq, 128), qs.reshape(Nq, Lq)
    s_ref, a_ref = oracle.fwd_i8(Q, qs, Dp, ds, cu)
    s, a = run_i8(bd, Q, qs, Dp, ds, cu)
    assert_bits_equal(s, s_ref, str(shape))
    assert np.array_equal(a, a_ref)
    s2, _ = run_i8(bd, Q, qs, Dp, ds, cu, with_argmax=False)
    assert_bits_equal(s2, s_ref, str(shape) + " no argmax")


def test_duplicate_tokens_tie_to_first(bd):
    Q, qs = inputs.random_rows(41, 64, 128, inputs.I8)
    D, ds = inputs.random_rows(42, 90, 128, inputs.I8)
    Dp = np.concatenate([D, D[::-1]])
    dsp = np.concatenate([ds, ds[::-1]])
    cu = np.array([0, 180], np.int32)
    Q, qs = Q.reshape(2, 32, 128), qs.reshape(2, 32)
    s_ref, a_ref = oracle.fwd_i8(Q, qs, Dp, dsp, cu)
    s, a = run_i8(bd, Q, qs, Dp, dsp, cu)
    assert_bits_equal(s, s_ref, "dup")
    assert np.array_equal(a, a_ref) and np.all(a < 90)


def test_first_token_max_ragged_tails(bd):
    """Every document starts with the token that best matches every query row,
    and lengths leave partial 16-token sub-tiles.  Rows past a document's end
    are read as copies of its first token, so they tie the maximum: the argmax
    must still be the first index, 0, and scores bit-exact."""
    Nq, Lq = 3, 32
    # one query row repeated (half of the rows negated), and that row as every
    # document's first token: token 0 is the exact maximum of the positive rows
    row, sc = inputs.random_rows(61, 1, 128, inputs.I8)
    sign = np.where(np.arange(Nq * Lq) % 2 == 0, 1, -1).astype(np.int8)
    Q = (row * sign[:, None]).reshape(Nq, Lq, 128)
    qs = np.full((Nq, Lq), sc[0], np.float32)
    lens = np.array([1, 15, 17, 31, 33, 47, 100, 129, 255, 257], np.int32)
    cu = inputs.cu_seqlens(lens)
    Dp, ds = inputs.random_rows(62, int(cu[-1]), 128, inputs.I8, stream=4)
    for b in range(len(lens)):
        Dp[cu[b]] = row[0]
        ds[cu[b]] = sc[0]
    s_ref, a_ref = oracle.fwd_i8(Q, qs, Dp, ds, cu)
    assert np.all(a_ref[:, :, 0::2] == 0)  # rows i = 0, 2, ... are the positive copies
    s, a = run_i8(bd, Q, qs, Dp, ds, cu)
    assert_bits_equal(s, s_ref, "first-token max")
    assert np.array_equal(a, a_ref)


@pytest.mark.parametrize("Lq", [32, 300])
def test_negative_maxima_and_scale_range(bd, Lq):
    """Row maxima that are negative (one- and two-token documents, about half
    of their rows, and tokens that negate query rows), rows that mix signs,
    zero dots and exact ties, and document scales spread over [2^-100, 2^40]
    plus the header's ends 2^-125 and 2^100.  The kernel holds negative values
    halved until the end; scores and argmax must still be bit-exact."""
    rng = np.random.default_rng(77 + Lq)
    Nq = 3
    Q = rng.integers(-127, 128, (Nq, Lq, 128)).astype(np.int8)
    qs = (2.0 ** rng.uniform(-8, 4, (Nq, Lq))).astype(np.float32)
    lens = np.array([1, 2, 16, 17, 40, 300, 5], np.int32)
    cu = inputs.cu_seqlens(lens)
    T = int(cu[-1])
    D = rng.integers(-127, 128, (T, 128)).astype(np.int8)
    # documents 0..2 (1, 2 and 16 tokens): every token the negation of a query
    # row; document 3: every other token so, and one all-zero token
    flat = Q.reshape(-1, 128).astype(np.int16)
    for b in range(3):
        for j in range(cu[b], cu[b + 1]):
            D[j] = np.clip(-flat[rng.integers(0, flat.shape[0])], -127, 127).astype(np.int8)
    for j in range(cu[3], cu[4], 2):
        D[j] = np.clip(-flat[rng.integers(0, flat.shape[0])], -127, 127).astype(np.int8)
    D[cu[3] + 1] = 0
    D[cu[4] + 3] = D[cu[4] + 7]  # exact ties within a document
    ds = (2.0 ** rng.uniform(-100, 40, T)).astype(np.float32)
    ds[cu[5]] = np.float32(2.0 ** -125)
    ds[cu[5] + 1] = np.float32(2.0 ** 100)
    ds[cu[4] + 7] = ds[cu[4] + 3]
    s_ref, a_ref = oracle.fwd_i8(Q, qs, D, ds, cu)
    s, a = run_i8(bd, Q, qs, D, ds, cu)
    assert_bits_equal(s, s_ref, "negative maxima, Lq %d" % Lq)
    assert np.array_equal(a, a_ref)
    s2, _ = run_i8(bd, Q, qs, D, ds, cu, with_argmax=False)
    assert_bits_equal(s2, s_ref, "negative maxima, Lq %d, no argmax" % Lq)
    assert np.any(s_ref[:, :3] < 0)  # the anti-aligned documents do give negative maxima


def test_workload_int8_subset(bd):
    w = inputs.make("int8_varlen")
    s, a = run_i8(bd, w["Q"], w["q_scale"], w["D_packed"], w["d_scale"], w["cu_seqlens"])
    # a seeded 5,000-document subset (5 % of the corpus) with the first and
    # last documents and both sides of the stream boundaries of a 256-stream grid
    rng = np.random.default_rng(2)
    edges = [(k * w["B"]) // 256 for k in range(1, 256)]
    pick = set([0, w["B"] - 1] + [e - 1 for e in edges] + edges)
    for b in rng.permutation(w["B"]):
        if len(pick) >= 5000:
            break
        pick.add(int(b))
    docs = np.array(sorted(pick))
    sub, subcu, subds = sub_corpus(w["D_packed"], w["cu_seqlens"], docs, w["d_scale"])
    s_ref, a_ref = oracle.fwd_i8(w["Q"], w["q_scale"], sub, subds, subcu)
    assert_bits_equal(s[:, docs], s_ref, "int8_varlen")
    assert np.array_equal(a[:, docs], a_ref)
    print("int8_varlen: %d of %d documents bit-exact (scores and argmax)" % (len(docs), w["B"]), flush=True)
