"""Pins for the oracle's fp16 / bf16 forward (CPU only).

Each test checks the oracle against something other than itself: values
worked out by hand (tests/golden), the exhaustive numpy decoding of every
16-bit pattern, numpy brute force (materialise S, max, first argmax), special
cases that reduce to a GEMV, and invariants of Eq. (1) that hold exactly.
"""
import json
import os

import numpy as np
import pytest

import oracle
from late_interaction_retrieval_amd import inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden", "maxsim_hand.json")


def as_dtype(x, dt):
    """fp64 array -> oracle input (fp16 array or bf16 bits); values must be representable."""
    x = np.asarray(x, np.float64)
    if dt == oracle.F16:
        y = x.astype(np.float16)
        assert np.array_equal(y.astype(np.float64), x)
        return y
    bits = inputs.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(inputs.bf16_bits_to_f32(bits).astype(np.float64), x)
    return bits


def decoded(a):
    if a.dtype == np.float16:
        return a.astype(np.float64)
    return inputs.bf16_bits_to_f32(a).astype(np.float64)


def brute(Q, D, lens):
    """numpy brute force: the materialised S = Q D^T, masked, then max / first argmax."""
    Qd, Dd = decoded(Q), decoded(D)
    S = np.einsum("qik,bjk->qbij", Qd, Dd)
    Ld = Dd.shape[1]
    valid = np.arange(Ld)[None, :] < np.asarray(lens)[:, None]  # [B, Ld]
    S = np.where(valid[None, :, None, :], S, -np.inf)
    m = S.max(axis=3)
    a = S.argmax(axis=3).astype(np.int32)
    a[:, np.asarray(lens) == 0, :] = -1
    return m.sum(axis=2), a, m


# --------------------------------------------------------------------------
def test_decode_f16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.f16_to_f64(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])
    # sign of zero
    assert np.array_equal(np.signbit(got[finite]), np.signbit(ref[finite]))


def test_decode_bf16_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    # bf16 is by definition the upper half of a binary32
    with np.errstate(invalid="ignore"):
        ref = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    got = oracle.bf16_to_f64(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_golden_hand_case(dt):
    g = json.load(open(GOLD))["fwd_padded"]
    Q, D = as_dtype(g["Q"], dt), as_dtype(g["D"], dt)
    s, a = oracle.fwd_padded(Q, D, dt, d_lens=np.array(g["d_lens"]))
    assert np.array_equal(s, np.array(g["scores"]))
    assert np.array_equal(a, np.array(g["argmax"]))


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_golden_hand_case_varlen(dt):
    """The same documents packed by cu_seqlens give identical results."""
    g = json.load(open(GOLD))["fwd_padded"]
    Q, D = as_dtype(g["Q"], dt), as_dtype(g["D"], dt)
    lens = np.array(g["d_lens"], np.int32)
    cu = inputs.cu_seqlens(lens)
    packed = np.concatenate([D[b, :lens[b]] for b in range(len(lens))])
    s, a = oracle.fwd_varlen(Q, packed, cu, dt)
    assert np.array_equal(s, np.array(g["scores"]))
    assert np.array_equal(a, np.array(g["argmax"]))


@pytest.mark.parametrize("dt,seed", [(oracle.F16, 1), (oracle.BF16, 2), (oracle.F16, 3)])
def test_brute_force_random(dt, seed):
    rng = np.random.default_rng(seed)
    Nq, Lq, B, Ld, d = 3, 5, 6, 9, 16
    dtn = inputs.F16 if dt == oracle.F16 else inputs.BF16
    Q = inputs.random_rows(seed, Nq * Lq, d, dtn).reshape(Nq, Lq, d)
    D = inputs.random_rows(seed + 100, B * Ld, d, dtn).reshape(B, Ld, d)
    lens = rng.integers(0, Ld + 1, size=B).astype(np.int32)
    lens[0], lens[1] = 0, Ld
    s, a, rm = oracle.fwd_padded(Q, D, dt, d_lens=lens, want_rowmax=True)
    sb, ab, mb = brute(Q, D, lens)
    np.testing.assert_allclose(s[:, 1:], sb[:, 1:], rtol=1e-13, atol=1e-13)
    assert np.all(np.isneginf(s[:, 0])) and np.all(np.isneginf(sb[:, 0]))
    np.testing.assert_allclose(rm[np.isfinite(mb)], mb[np.isfinite(mb)], rtol=1e-13, atol=1e-13)
    assert np.array_equal(a, ab)


def test_padded_equals_varlen_random():
    rng = np.random.default_rng(7)
    Nq, Lq, B, Ld, d = 2, 7, 8, 11, 32
    Q = inputs.random_rows(7, Nq * Lq, d, inputs.BF16).reshape(Nq, Lq, d)
    lens = rng.integers(0, Ld + 1, size=B).astype(np.int32)
    cu = inputs.cu_seqlens(lens)
    packed = inputs.random_rows(8, int(cu[-1]), d, inputs.BF16)
    padded = inputs.pad_packed(packed, cu, Ld)
    padded[padded == 0] = 0x7F00  # garbage in the padding must not matter
    for b in range(B):
        padded[b, :lens[b]] = packed[cu[b]:cu[b + 1]]
    s1, a1 = oracle.fwd_padded(Q, padded, oracle.BF16, d_lens=lens)
    s2, a2 = oracle.fwd_varlen(Q, packed, cu, oracle.BF16)
    assert np.array_equal(s1, s2) and np.array_equal(a1, a2)


def test_single_doc_token_is_gemv():
    """Ld = 1: score = sum_i <Q_i, D_0> = <sum_i Q_i, D_0>, a matrix-vector product."""
    Q = inputs.random_rows(11, 4 * 6, 32, inputs.F16).reshape(4, 6, 32)
    D = inputs.random_rows(12, 5, 32, inputs.F16).reshape(5, 1, 32)
    s, a = oracle.fwd_padded(Q, D, oracle.F16)
    ref = Q.astype(np.float64).sum(axis=1) @ D[:, 0].astype(np.float64).T
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-13)
    assert np.all(a == 0)


def test_single_query_token_is_max_of_gemv():
    """Lq = 1: score = max_j (D_b Q_0)_j."""
    Q = inputs.random_rows(13, 3, 64, inputs.BF16).reshape(3, 1, 64)
    D = inputs.random_rows(14, 4 * 10, 64, inputs.BF16).reshape(4, 10, 64)
    s, a = oracle.fwd_padded(Q, D, oracle.BF16)
    Qd, Dd = decoded(Q), decoded(D)
    for q in range(3):
        for b in range(4):
            v = Dd[b] @ Qd[q, 0]
            assert s[q, b] == pytest.approx(v.max(), rel=1e-13, abs=1e-14)
            assert a[q, b, 0] == int(np.argmax(v))


@pytest.mark.parametrize("dt", [oracle.F16, oracle.BF16])
def test_signed_basis_score_equals_lq(dt):
    """Q rows are +-e_k and D contains each of them among unit rows: score = Lq exactly."""
    d, Lq = 128, 40
    rng = np.random.default_rng(5)
    ks = rng.integers(0, d, size=Lq)
    sg = rng.choice([-1.0, 1.0], size=Lq)
    Qf = np.zeros((1, Lq, d))
    Qf[0, np.arange(Lq), ks] = sg
    dtn = inputs.F16 if dt == oracle.F16 else inputs.BF16
    others = inputs.random_rows(6, 60, d, dtn)
    basis = as_dtype(Qf[0], dt)
    D = np.concatenate([others[:30], basis, others[30:]])[None]
    perm = rng.permutation(D.shape[1])
    D = D[:, perm]
    s, a = oracle.fwd_padded(as_dtype(Qf, dt), D, dt)
    assert s[0, 0] == float(Lq)
    Dd = decoded(D)[0]
    for i in range(Lq):
        assert Dd[a[0, 0, i], ks[i]] == sg[i]


def test_padding_never_selected_when_all_negative():
    Q = np.full((1, 3, 8), 0.25, np.float16)
    D = np.full((2, 6, 8), -0.5, np.float16)
    D[:, 4:] = 60000.0  # huge padding rows
    D[1, 2] = -0.125
    lens = np.array([4, 4], np.int32)
    s, a = oracle.fwd_padded(Q, D, oracle.F16, d_lens=lens)
    assert np.all(a[0, 0] == 0)  # all valid equal: first index
    assert np.all(a[0, 1] == 2)
    assert s[0, 0] == 3 * (8 * 0.25 * -0.5)
    assert s[0, 1] == 3 * (8 * 0.25 * -0.125)


def _grid(rng, shape):
    """Dyadic values k/64, |k| <= 64: every product and sum below is exact in fp64."""
    return rng.integers(-64, 65, size=shape) / 64.0


def test_doc_token_permutation_invariance():
    rng = np.random.default_rng(21)
    Q = as_dtype(_grid(rng, (2, 6, 16)), oracle.F16)
    D = as_dtype(_grid(rng, (3, 12, 16)), oracle.F16)
    s, a = oracle.fwd_padded(Q, D, oracle.F16)
    perm = rng.permutation(12)
    s2, a2 = oracle.fwd_padded(Q, D[:, perm], oracle.F16)
    assert np.array_equal(s, s2)
    # the winner is the same document token (values may tie: compare the vectors)
    Dd = decoded(D)
    for q in range(2):
        for b in range(3):
            for i in range(6):
                v1 = decoded(Q)[q, i] @ Dd[b, a[q, b, i]]
                v2 = decoded(Q)[q, i] @ Dd[b, perm[a2[q, b, i]]]
                assert v1 == v2


def test_query_chunks_add_up():
    """The sum of maxima decomposes over query-token chunks (Section 4.1)."""
    rng = np.random.default_rng(22)
    Q = as_dtype(_grid(rng, (2, 9, 16)), oracle.BF16)
    D = as_dtype(_grid(rng, (4, 7, 16)), oracle.BF16)
    s, _ = oracle.fwd_padded(Q, D, oracle.BF16)
    s1, _ = oracle.fwd_padded(np.ascontiguousarray(Q[:, :4]), D, oracle.BF16)
    s2, _ = oracle.fwd_padded(np.ascontiguousarray(Q[:, 4:]), D, oracle.BF16)
    assert np.array_equal(s, s1 + s2)


def test_appending_doc_tokens_never_lowers_score():
    rng = np.random.default_rng(23)
    Q = inputs.random_rows(23, 2 * 5, 32, inputs.F16).reshape(2, 5, 32)
    D = inputs.random_rows(24, 3 * 10, 32, inputs.F16).reshape(3, 10, 32)
    lens_short = np.array([3, 6, 1], np.int32)
    s_short, _ = oracle.fwd_padded(Q, D, oracle.F16, d_lens=lens_short)
    s_long, _ = oracle.fwd_padded(Q, D, oracle.F16, d_lens=lens_short + rng.integers(0, 4, 3))
    assert np.all(s_long >= s_short)


def test_power_of_two_scaling_is_exact():
    Q = inputs.random_rows(25, 2 * 4, 32, inputs.F16).reshape(2, 4, 32)
    D = inputs.random_rows(26, 3 * 5, 32, inputs.F16).reshape(3, 5, 32)
    s, a = oracle.fwd_padded(Q, D, oracle.F16)
    s4, a4 = oracle.fwd_padded((Q.astype(np.float32) * 4).astype(np.float16), D, oracle.F16)
    assert np.array_equal(s4, 4 * s) and np.array_equal(a, a4)


def test_sim_at_matches_rowmax():
    Q = inputs.random_rows(27, 2 * 5, 128, inputs.BF16).reshape(2, 5, 128)
    lens = np.array([4, 0, 9], np.int32)
    cu = inputs.cu_seqlens(lens)
    D = inputs.random_rows(28, int(cu[-1]), 128, inputs.BF16)
    s, a, rm = oracle.fwd_varlen(Q, D, cu, oracle.BF16, want_rowmax=True)
    v = oracle.sim_at(Q, D, cu, oracle.BF16, a)
    assert np.array_equal(v, rm)
    assert np.all(np.isneginf(v[:, 1])) and np.all(a[:, 1] == -1)
