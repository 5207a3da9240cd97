"""Pins of the oracle's statistics, ridge solve and reconstruction error."""
import math

import numpy as np
import pytest
import scipy.linalg

from oracle import (accumulate_gram, accumulate_stats, backward_substitution, cholesky_lower, stats_from_gram,
                    epsilon_direct, epsilon_from_stats, forward_substitution,
                    residual_target, ridge_lambda, solve_dw)


def test_stats_brute_force(rng):
    n, D = 5, 3
    a, dl = rng.normal(size=(n, D)), rng.normal(size=(n, D))
    w = rng.normal(size=(D, D))  # not symmetric: a transposed W must fail
    G, C, r2 = accumulate_stats(a, dl, w)
    R = [[sum(dl[r][k] * w[k][j] for k in range(D)) for j in range(D)] for r in range(n)]
    for i in range(D):
        for j in range(D):
            assert abs(G[i, j] - sum(a[r][i] * a[r][j] for r in range(n))) < 1e-12
            assert abs(C[i, j] - sum(a[r][i] * R[r][j] for r in range(n))) < 1e-12
    assert abs(r2 - sum(R[r][j] ** 2 for r in range(n) for j in range(D))) < 1e-12


def test_stats_invariants(rng):
    a, dl, w = rng.normal(size=(40, 6)), rng.normal(size=(40, 6)), rng.normal(size=(6, 6))
    G, C, r2 = accumulate_stats(a, dl, w)
    assert abs(np.trace(G) - np.sum(a * a)) < 1e-11
    np.testing.assert_allclose(G, G.T, rtol=0, atol=0)
    assert np.linalg.eigvalsh(G).min() > -1e-10
    # residual target of A_full = A_loc + delta
    np.testing.assert_allclose(residual_target(a, a + dl, w), dl @ w, rtol=1e-13)
    G0, C0, r0 = accumulate_stats(a, np.zeros_like(dl), w)
    assert np.all(C0 == 0) and r0 == 0


def test_stats_additive_over_steps(rng):
    steps = [(rng.normal(size=(9, 5)), rng.normal(size=(9, 5))) for _ in range(4)]
    w = rng.normal(size=(5, 5))
    Gs, Cs, rs = np.zeros((5, 5)), np.zeros((5, 5)), 0.0
    for a, dl in steps:
        G, C, r2 = accumulate_stats(a, dl, w)
        Gs += G; Cs += C; rs += r2
    Ga, Ca, ra = accumulate_stats(np.concatenate([s[0] for s in steps]),
                                  np.concatenate([s[1] for s in steps]), w)
    np.testing.assert_allclose(Gs, Ga, rtol=1e-13)
    np.testing.assert_allclose(Cs, Ca, rtol=1e-12, atol=1e-13)
    assert abs(rs - ra) < 1e-11 * ra


def test_gram_brute_force(rng):
    """The grouped sums as explicit outer products over rows (tiny shape,
    non-square-symmetric data: a swapped operand or a transpose fails)."""
    n, D = 5, 3
    a, dl = rng.normal(size=(n, D)), rng.normal(size=(n, D))
    G, M, H = accumulate_gram(a, dl)
    for i in range(D):
        for j in range(D):
            assert abs(G[i, j] - sum(a[r][i] * a[r][j] for r in range(n))) < 1e-12
            assert abs(M[i, j] - sum(a[r][i] * dl[r][j] for r in range(n))) < 1e-12
            assert abs(H[i, j] - sum(dl[r][i] * dl[r][j] for r in range(n))) < 1e-12
    assert abs(M[0, 1] - M[1, 0]) > 1e-3  # M is not symmetric on this data


def test_gram_regrouping_equals_stats(rng):
    """C = (A_loc^T dA) W and r2 = <dA^T dA, W W^T> equal A_loc^T (dA W) and
    ||dA W||^2 (associativity; the printed closed form groups the product
    this way), for a non-symmetric W and over several steps."""
    D = 7
    w = rng.normal(size=(D, D))
    Gs, Ms, Hs = np.zeros((D, D)), np.zeros((D, D)), np.zeros((D, D))
    Gr, Cr, rr = np.zeros((D, D)), np.zeros((D, D)), 0.0
    for _ in range(3):
        a, dl = rng.normal(size=(11, D)), rng.normal(size=(11, D))
        G, M, H = accumulate_gram(a, dl)
        Gs, Ms, Hs = Gs + G, Ms + M, Hs + H
        g, c, r = accumulate_stats(a, dl, w)
        Gr, Cr, rr = Gr + g, Cr + c, rr + r
    G2, C2, r2 = stats_from_gram(Gs, Ms, Hs, w)
    np.testing.assert_allclose(G2, Gr, rtol=1e-13)
    np.testing.assert_allclose(C2, Cr, rtol=1e-11, atol=1e-12)
    assert abs(r2 - rr) <= 1e-12 * rr
    # the transposed products give different numbers on this data
    assert abs(float(np.sum(Hs * (w.T @ w))) - rr) > 1e-6 * rr
    assert np.abs(Ms.T @ w - Cr).max() > 1e-6


def test_gram_invariants(rng):
    a, dl = rng.normal(size=(40, 6)), rng.normal(size=(40, 6))
    G, M, H = accumulate_gram(a, dl)
    np.testing.assert_allclose(H, H.T, rtol=0, atol=0)
    assert np.linalg.eigvalsh(H).min() > -1e-10
    assert abs(np.trace(H) - np.sum(dl * dl)) < 1e-11
    # no history: dA = 0 gives M = 0, H = 0, hence C = 0 and r2 = 0
    _, M0, H0 = accumulate_gram(a, np.zeros_like(dl))
    _, C0, r0 = stats_from_gram(G, M0, H0, rng.normal(size=(6, 6)))
    assert not M0.any() and not H0.any() and not C0.any() and r0 == 0.0


def _spd(rng, D, n=None):
    a = rng.normal(size=(n or 3 * D, D))
    return a, a.T @ a


def test_cholesky_against_lapack(rng):
    _, G = _spd(rng, 12)
    L, info = cholesky_lower(G)
    assert info == 0
    assert np.all(np.triu(L, 1) == 0)
    np.testing.assert_allclose(L @ L.T, G, rtol=1e-13, atol=1e-12)
    np.testing.assert_allclose(L, np.linalg.cholesky(G), rtol=1e-12, atol=1e-12)


def test_triangular_solves_against_lapack(rng):
    _, G = _spd(rng, 10)
    L = np.linalg.cholesky(G)
    B = rng.normal(size=(10, 4))
    np.testing.assert_allclose(forward_substitution(L, B),
                               scipy.linalg.solve_triangular(L, B, lower=True), rtol=1e-11)
    np.testing.assert_allclose(backward_substitution(L, B),
                               scipy.linalg.solve_triangular(L.T, B, lower=False), rtol=1e-11)


def test_cholesky_reports_failing_pivot():
    A = np.diag([1.0, 0.0, 2.0])
    _, info = cholesky_lower(A)
    assert info == 2
    dW, info = solve_dw(np.diag([1.0, -1.0, 1.0]), np.ones((3, 3)), 0.0)
    assert info == 2 and np.all(np.isnan(dW))


def test_solve_against_lapack_and_residual(rng):
    a, G = _spd(rng, 24)
    C = a.T @ rng.normal(size=(a.shape[0], 24))
    lam = ridge_lambda(G, 0.0, 1e-3)
    dW, info = solve_dw(G, C, lam)
    assert info == 0
    A = G + lam * np.eye(24)
    np.testing.assert_allclose(dW, np.linalg.solve(A, C), rtol=1e-10, atol=1e-12)
    assert np.linalg.norm(A @ dW - C) / np.linalg.norm(C) <= 1e-10


def test_lambda_reading():
    G = np.diag([2.0, 4.0, 6.0])
    assert ridge_lambda(G, 0.0, 1e-3) == pytest.approx(1e-3 * 4.0)
    assert ridge_lambda(G, 0.5, 0.0) == 0.5


def test_diagonal_closed_form(rng):
    g = rng.uniform(0.5, 3.0, size=6)
    C = rng.normal(size=(6, 6))
    dW, _ = solve_dw(np.diag(g), C, 0.25)
    np.testing.assert_allclose(dW, C / (g + 0.25)[:, None], rtol=1e-13)


def test_planted_dw_recovered(rng):
    # target exactly linear in A_loc: R = A_loc dW*  =>  dW = (G+lam I)^-1 G dW*
    D = 16
    a = rng.normal(size=(200, D))
    dWs = rng.normal(size=(D, D)) * 0.1
    w = rng.normal(size=(D, D)) / math.sqrt(D)
    # delta such that delta W = a dWs  ->  delta = a dWs W^-1
    delta = a @ dWs @ np.linalg.inv(w)
    G, C, r2 = accumulate_stats(a, delta, w)
    dW0, _ = solve_dw(G, C, 0.0)
    np.testing.assert_allclose(dW0, dWs, rtol=1e-8, atol=1e-9)
    assert epsilon_from_stats(G, C, r2, dW0) < 1e-12 * r2
    lam = ridge_lambda(G, 0.0, 1e-3)
    dWl, _ = solve_dw(G, C, lam)
    np.testing.assert_allclose(dWl, np.linalg.solve(G + lam * np.eye(D), G @ dWs), rtol=1e-9, atol=1e-11)


def test_large_lambda_limit(rng):
    a, G = _spd(rng, 8)
    dl, w = rng.normal(size=a.shape), rng.normal(size=(8, 8))
    G, C, r2 = accumulate_stats(a, dl, w)
    dW, _ = solve_dw(G, C, 1e12)
    assert np.abs(dW).max() < 1e-8
    assert epsilon_from_stats(G, C, r2, dW) == pytest.approx(r2, rel=1e-8)


def test_relative_lambda_scale_invariant(rng):
    a, dl, w = rng.normal(size=(60, 8)), rng.normal(size=(60, 8)), rng.normal(size=(8, 8))
    G, C, _ = accumulate_stats(a, dl, w)
    d1, _ = solve_dw(G, C, ridge_lambda(G, 0.0, 1e-3))
    d2, _ = solve_dw(7.5 * G, 7.5 * C, ridge_lambda(7.5 * G, 0.0, 1e-3))
    np.testing.assert_allclose(d1, d2, rtol=1e-12, atol=1e-14)


def test_epsilon_stats_equals_direct(rng):
    # several steps, then eps from the statistics == eps on the stored rows
    D = 10
    w = rng.normal(size=(D, D)) / math.sqrt(D)
    A_loc, A_full = [], []
    G, C, r2 = np.zeros((D, D)), np.zeros((D, D)), 0.0
    for _ in range(3):
        al = rng.normal(size=(30, D))
        af = al + 0.3 * rng.normal(size=(30, D)) + 0.2 * al @ rng.normal(size=(D, D))
        g, c, r = accumulate_stats(al, af - al, w)
        G += g; C += c; r2 += r
        A_loc.append(al); A_full.append(af)
    A_loc, A_full = np.concatenate(A_loc), np.concatenate(A_full)
    lam = ridge_lambda(G, 0.0, 1e-3)
    dW, _ = solve_dw(G, C, lam)
    e_s = epsilon_from_stats(G, C, r2, dW)
    e_d = epsilon_direct(A_loc, A_full, w, dW)
    assert abs(e_s - e_d) <= 1e-10 * e_d
    # bounds: 0 <= eps <= r2 - lam |dW|^2 <= r2 (dW = 0 is feasible)
    assert 0 <= e_s <= r2 - lam * np.sum(dW * dW) + 1e-9 * r2
    # ridge optimum shortcut: eps = r2 - <dW, C> - lam |dW|^2
    assert abs(e_s - (r2 - np.sum(dW * C) - lam * np.sum(dW * dW))) <= 1e-9 * r2
    # eps at the optimum is below eps at a perturbed point (minimiser check)
    pert = dW + 1e-3 * rng.normal(size=dW.shape)
    obj = lambda x: epsilon_from_stats(G, C, r2, x) + lam * np.sum(x * x)  # noqa: E731
    assert obj(dW) < obj(pert)
