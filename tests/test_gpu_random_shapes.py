"""Seeded random shapes through every kernel family, against the oracle.

The hand-picked shapes of the other GPU tests aim at known edges; these draw
query counts and lengths, corpus sizes and document-length ranges at random
(fixed seeds), so that each run also crosses combinations nobody picked:
lengths that are and are not multiples of the 8-row sum groups and 16- or
32-token sub-tiles, documents that end anywhere inside a sub-tile, empty
documents, hot rows.  Each case uses the same checks as the family's own
tests: fp16/bf16 scores within the tolerance and every argmax a near-tie
(padded and packed bit-identical), INT8 bit-exact, CSR maps bit-exact and
gradients within 1e-3 of the oracle (FM §4.1 Alg. 2, §4.2 Alg. 3, §4.3; the
Chamfer case FM §4.2 "Generalization to Chamfer Distance")."""
import numpy as np
import pytest
import torch

import oracle
from late_interaction_retrieval_amd import inputs
import test_gpu_bwd as tb
import test_gpu_bwd_varlen as tv
import test_gpu_chamfer as tc
import test_gpu_fwd as tf
import test_gpu_i8 as ti

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    from late_interaction_retrieval_amd import binding
    assert torch.cuda.is_available()
    return binding


def forward_case(rng):
    kind = str(rng.choice(["f16", "bf16", "i8"]))
    Nq = int(rng.choice([1, 2, 3, 5, 8, 16, 33, 64]))
    Lq = int(rng.choice([1, 7, 8, 13, 16, 20, 24, 31, 32, 40, 48, 56, 64, 100, 128, 257, 300, 513, 600, 1000, 1024]))
    if Nq * Lq > 40000:
        Lq = 32
    B = int(rng.integers(1, 400))
    lo = int(rng.integers(0, 60))
    hi = lo + int(rng.integers(0, 600))
    lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    while B > 1 and Nq * Lq * int(lens.sum()) > 3e7:  # the oracle's work
        B = max(1, B // 2)
        lens = lens[:B]
    return kind, Nq, Lq, lens, int(rng.integers(1 << 30))


@pytest.mark.parametrize("case", range(24))
def test_forward_random(bd, case):
    kind, Nq, Lq, lens, seed = forward_case(np.random.default_rng(9100 + case))
    cu = inputs.cu_seqlens(lens)
    T = int(cu[-1])
    where = "%s Nq %d Lq %d B %d T %d" % (kind, Nq, Lq, len(lens), T)
    if kind == "i8":
        Q, qs = inputs.random_rows(seed, Nq * Lq, 128, inputs.I8)
        Dp, ds = inputs.random_rows(seed + 1, max(T, 1), 128, inputs.I8, stream=4)
        Dp, ds = Dp[:T], ds[:T]
        Q, qs = Q.reshape(Nq, Lq, 128), qs.reshape(Nq, Lq)
        s_ref, a_ref = oracle.fwd_i8(Q, qs, Dp, ds, cu)
        s, a = ti.run_i8(bd, Q, qs, Dp, ds, cu)
        ti.assert_bits_equal(s, s_ref, where)
        assert np.array_equal(a, a_ref), where
        s2, _ = ti.run_i8(bd, Q, qs, Dp, ds, cu, with_argmax=False)
        ti.assert_bits_equal(s2, s_ref, where + " no argmax")
    else:
        dtn = inputs.F16 if kind == "f16" else inputs.BF16
        Q = inputs.random_rows(seed, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
        Dp = inputs.random_rows(seed + 1, max(T, 1), 128, dtn, stream=4)[:T]
        tf.full_check_varlen(bd, Q, Dp, cu, dtn, where)


@pytest.mark.parametrize("case", range(12))
def test_backward_random(bd, case):
    rng = np.random.default_rng(9300 + case)
    dtn = inputs.F16 if rng.random() < 0.5 else inputs.BF16
    Nq = int(rng.choice([1, 2, 3, 5, 8, 17, 33]))
    Lq = int(rng.choice([1, 7, 32, 64, 100, 129, 256, 300, 513, 1024]))
    B = int(rng.integers(1, 40))
    Ld = int(rng.choice([1, 5, 31, 64, 100, 200, 513, 1024, 2000]))
    while B > 1 and Nq * Lq * B * 128 > 4e8:
        B //= 2
    hot = rng.random() < 0.3
    seed = int(rng.integers(1 << 30))
    r2 = np.random.default_rng(seed)
    g = r2.standard_normal((Nq, B)).astype(np.float32)
    Q = inputs.random_rows(seed, Nq * Lq, 128, dtn).reshape(Nq, Lq, 128)
    if case % 2 == 0:  # padded
        where = "padded Nq %d Lq %d B %d Ld %d hot %d" % (Nq, Lq, B, Ld, hot)
        D = inputs.random_rows(seed + 1, B * Ld, 128, dtn, stream=4).reshape(B, Ld, 128)
        A = r2.integers(0, Ld, size=(Nq, B, Lq)).astype(np.int32)
        if hot:
            A[r2.random(A.shape) < 0.6] = min(3, Ld - 1)
        tb.check_bwd(bd, Q, D, dtn, A, g, where)
    else:  # packed, empty documents allowed
        lens = r2.integers(0, Ld + 1, size=B).astype(np.int32)
        cu = inputs.cu_seqlens(lens)
        where = "packed Nq %d Lq %d B %d Ld 0..%d hot %d" % (Nq, Lq, B, Ld, hot)
        T = int(cu[-1])
        Dp = inputs.random_rows(seed + 1, max(T, 1), 128, dtn, stream=4)[:T]
        A = np.full((Nq, B, Lq), -1, np.int32)
        for b in range(B):
            if lens[b] > 0:
                A[:, b, :] = r2.integers(0, lens[b], size=(Nq, Lq))
                if hot:
                    A[:, b, :][r2.random((Nq, Lq)) < 0.6] = 0
        tv.check(bd, Q, Dp, cu, dtn, A, g, where)


@pytest.mark.parametrize("case", range(10))
def test_chamfer_random(bd, case):
    rng = np.random.default_rng(9500 + case)
    Bt = int(rng.choice([1, 2, 3, 8, 16, 32, 64, 200]))
    N = int(rng.choice([1, 5, 17, 100, 257, 1000, 2048, 3000, 9000, 20000]))
    M = int(rng.choice([1, 5, 17, 100, 257, 1000, 2048, 3000, 9000, 20000]))
    while Bt > 1 and Bt * N * M > 6e7:
        Bt //= 2
    while Bt * N * M > 6e7:
        N = max(1, N // 2)
    where = "Bt %d N %d M %d" % (Bt, N, M)
    P, Q = inputs.point_clouds(int(rng.integers(1 << 30)), Bt, N, M)
    dp, ip, dq, iq = (t.cpu().numpy() for t in bd.maxsim_chamfer_fwd(tc.dev(P), tc.dev(Q)))
    torch.cuda.synchronize()
    tc.check_direction(P, Q, dp, ip, where + " P->Q")
    tc.check_direction(Q, P, dq, iq, where + " Q->P")
    gp = rng.standard_normal((Bt, N)).astype(np.float32)
    gq = rng.standard_normal((Bt, M)).astype(np.float32)
    _, ipo, _, iqo = oracle.chamfer(P, Q)
    tc.check_bwd(bd, P, Q, ipo, iqo, gp, gq, where + " bwd")
