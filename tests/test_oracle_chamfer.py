"""Pins of the Chamfer-distance oracle (paper Section 4.2, "Generalization to
Chamfer Distance") against facts that do not come from the oracle itself: an
independent nearest-neighbour search (scipy's k-d tree), closed forms on
hand-built clouds, invariances, a stable library argsort for the inverse map,
exact finite differences and exact identities for the gradients."""
import numpy as np
import pytest
from scipy.spatial import cKDTree

import oracle
from late_interaction_retrieval_amd import inputs


def clouds(seed, Bt, N, M):
    return inputs.point_clouds(seed, Bt, N, M)


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 50, 70), (3, 33, 17), (2, 200, 5)])
def test_nearest_neighbour_matches_kdtree(shape):
    """A k-d tree finds the same nearest point (ties aside) and distance."""
    Bt, N, M = shape
    P, Q = clouds(11 + N, Bt, N, M)
    dist, idx = oracle.chamfer_nn(P, Q)
    for b in range(Bt):
        d_kd, i_kd = cKDTree(Q[b].astype(np.float64)).query(P[b].astype(np.float64), k=1)
        np.testing.assert_allclose(dist[b], d_kd ** 2, rtol=1e-12, atol=1e-15)
        # where the tree picked another index, that point is exactly as near
        diff = idx[b] != i_kd
        if diff.any():
            alt = ((P[b][diff].astype(np.float64) - Q[b][i_kd[diff]].astype(np.float64)) ** 2).sum(1)
            np.testing.assert_allclose(dist[b][diff], alt, rtol=1e-12)


def test_lattice_closed_form():
    """Q on an integer grid, P = grid points moved by less than half a cell:
    the nearest point is the grid point each P point came from, at the squared
    length of its offset."""
    g = np.stack(np.meshgrid(np.arange(4), np.arange(3), np.arange(5), indexing="ij"), -1).reshape(-1, 3)
    Q = g.astype(np.float32)
    rng = np.random.default_rng(3)
    off = (rng.random((len(g), 3)) - 0.5).astype(np.float32) * np.float32(0.8)
    perm = rng.permutation(len(g))
    P = (Q[perm] + off).astype(np.float32)
    dist, idx = oracle.chamfer_nn(P, Q)
    assert np.array_equal(idx[0], perm)
    exact = ((P.astype(np.float64) - Q[perm].astype(np.float64)) ** 2).sum(1)
    np.testing.assert_allclose(dist[0], exact, rtol=1e-15)


def test_identical_clouds_and_single_points():
    P, _ = clouds(5, 1, 64, 1)
    dp, ip, dq, iq = oracle.chamfer(P, P)
    assert np.all(dp == 0) and np.array_equal(ip[0], np.arange(64)) and np.array_equal(iq[0], np.arange(64))
    assert np.all(oracle.chamfer_loss(P, P) == 0)
    p = np.array([[[1.0, 2.0, 3.0]]], np.float32)
    q = np.array([[[1.5, 0.0, -1.0]]], np.float32)
    assert oracle.chamfer_loss(p, q)[0] == 2 * (0.25 + 4.0 + 16.0)


def test_ties_take_the_first_index():
    """Two equally near points: the first one is selected."""
    P = np.zeros((1, 1, 3), np.float32)
    Q = np.array([[[0, 0, 2], [1, 0, 0], [0, -1, 0], [0, 1, 0]]], np.float32)
    _, idx = oracle.chamfer_nn(P, Q)
    assert idx[0, 0] == 1


def test_empty_target_cloud():
    P, _ = clouds(6, 2, 4, 1)
    dist, idx = oracle.chamfer_nn(P, np.zeros((2, 0, 3), np.float32))
    assert np.all(np.isposinf(dist)) and np.all(idx == -1)


def test_invariances():
    """Translation and permutation of the target cloud; scaling by 2^k scales
    distances by 4^k exactly; the symmetric loss does not depend on the order
    of the two clouds."""
    P, Q = clouds(7, 2, 40, 55)
    dist, idx = oracle.chamfer_nn(P, Q)
    t = np.array([0.25, -1.5, 3.0], np.float32)
    d2, i2 = oracle.chamfer_nn(P + t, Q + t)
    assert np.array_equal(i2, idx)
    np.testing.assert_allclose(d2, dist, rtol=1e-5)
    perm = np.random.default_rng(1).permutation(55)
    d3, i3 = oracle.chamfer_nn(P, Q[:, perm])
    assert np.array_equal(perm[i3], idx) and np.array_equal(d3, dist)
    d4, i4 = oracle.chamfer_nn(P * np.float32(4), Q * np.float32(4))
    assert np.array_equal(i4, idx) and np.array_equal(d4, dist * 16)
    np.testing.assert_allclose(oracle.chamfer_loss(P, Q), oracle.chamfer_loss(Q, P), rtol=1e-15)


@pytest.mark.parametrize("shape", [(1, 30, 20), (3, 17, 41), (2, 5, 1)])
def test_inverse_map_matches_stable_argsort(shape):
    Bt, N, M = shape
    P, Q = clouds(13 + N, Bt, N, M)
    _, idx = oracle.chamfer_nn(P, Q)
    rp, ci = oracle.chamfer_csr(idx, M)
    dst = (np.arange(Bt)[:, None] * M + idx).reshape(-1)
    assert np.array_equal(rp, np.concatenate([[0], np.cumsum(np.bincount(dst, minlength=Bt * M))]))
    assert np.array_equal(ci, np.argsort(dst, kind="stable"))


def test_inverse_map_skips_unselected_and_hot_destination():
    idx = np.array([[2, -1, 2, 0, 2, -1, 2]], np.int32)
    rp, ci = oracle.chamfer_csr(idx, 4)
    assert np.array_equal(rp, [0, 1, 1, 5, 5]) and np.array_equal(ci, [3, 0, 2, 4, 6])


def weighted_loss(P, Q, ip, iq, gp, gq):
    """sum gp*|P - Q[ip]|^2 + sum gq*|Q - P[iq]|^2 with the selections fixed, in fp64."""
    P = P.astype(np.float64)
    Q = Q.astype(np.float64)
    Bt = P.shape[0]
    tot = 0.0
    for b in range(Bt):
        tot += (gp[b] * ((P[b] - Q[b][ip[b]]) ** 2).sum(1)).sum()
        tot += (gq[b] * ((Q[b] - P[b][iq[b]]) ** 2).sum(1)).sum()
    return tot


def test_gradient_finite_differences_exact():
    """On a dyadic grid the loss (selections fixed) is a quadratic whose
    central differences are exact in fp64: every coordinate's derivative."""
    rng = np.random.default_rng(21)
    Bt, N, M = 2, 6, 5
    P = (rng.integers(-64, 64, (Bt, N, 3)) / 32).astype(np.float32)
    Q = (rng.integers(-64, 64, (Bt, M, 3)) / 32).astype(np.float32)
    _, ip, _, iq = oracle.chamfer(P, Q)
    gp = (rng.integers(-8, 8, (Bt, N)) / 8).astype(np.float32)
    gq = (rng.integers(-8, 8, (Bt, M)) / 8).astype(np.float32)
    dP, dQ = oracle.chamfer_bwd(P, Q, ip, iq, gp, gq)
    h = 2.0 ** -6
    for X, G in ((P, dP), (Q, dQ)):
        for pos in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[pos] += np.float32(h)
            Xm[pos] -= np.float32(h)
            if X is P:
                fp, fm = weighted_loss(Xp, Q, ip, iq, gp, gq), weighted_loss(Xm, Q, ip, iq, gp, gq)
            else:
                fp, fm = weighted_loss(P, Xp, ip, iq, gp, gq), weighted_loss(P, Xm, ip, iq, gp, gq)
            assert (fp - fm) / (2 * h) == G[pos], pos


def test_gradient_identities():
    """Moving both clouds together changes nothing: the gradients sum to 0.
    The loss is homogeneous of degree 2: <dP, P> + <dQ, Q> = 2 * loss."""
    P, Q = clouds(31, 3, 90, 70)
    _, ip, _, iq = oracle.chamfer(P, Q)
    rng = np.random.default_rng(4)
    gp = rng.standard_normal((3, 90)).astype(np.float32)
    gq = rng.standard_normal((3, 70)).astype(np.float32)
    dP, dQ = oracle.chamfer_bwd(P, Q, ip, iq, gp, gq)
    for b in range(3):
        np.testing.assert_allclose(dP[b].sum(0) + dQ[b].sum(0), 0, atol=1e-12)
    lhs = (dP * P.astype(np.float64)).sum() + (dQ * Q.astype(np.float64)).sum()
    np.testing.assert_allclose(lhs, 2 * weighted_loss(P, Q, ip, iq, gp, gq), rtol=1e-12)


def test_gradient_single_pair_closed_form():
    """One point each: L = (gp + gq)|p - q|^2, dP = 2 (gp + gq)(p - q) = -dQ."""
    p = np.array([[[1.0, 2.0, 3.0]]], np.float32)
    q = np.array([[[0.5, 4.0, 2.0]]], np.float32)
    dP, dQ = oracle.chamfer_bwd(p, q, np.zeros((1, 1), np.int32), np.zeros((1, 1), np.int32),
                                np.array([[0.25]], np.float32), np.array([[0.5]], np.float32))
    assert np.array_equal(dP[0, 0], 2 * 0.75 * np.array([0.5, -2.0, 1.0]))
    assert np.array_equal(dQ[0, 0], -dP[0, 0])


def test_gradient_unselected_sources_add_nothing():
    P, Q = clouds(41, 1, 8, 6)
    _, ip, _, iq = oracle.chamfer(P, Q)
    gp, gq = np.ones((1, 8), np.float32), np.ones((1, 6), np.float32)
    ip2 = ip.copy()
    ip2[0, 3] = -1
    dP, dQ = oracle.chamfer_bwd(P, Q, ip, iq, gp, gq)
    dP2, dQ2 = oracle.chamfer_bwd(P, Q, ip2, iq, gp, gq)
    gp0 = gp.copy()
    gp0[0, 3] = 0
    dP0, dQ0 = oracle.chamfer_bwd(P, Q, ip, iq, gp0, gq)
    assert np.array_equal(dQ2, dQ0)
    assert np.array_equal(np.delete(dP2[0], 3, 0), np.delete(dP0[0], 3, 0))
