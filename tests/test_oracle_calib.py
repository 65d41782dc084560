"""Pins of the oracle's one-pass calibration and ridge solve: a Hadamard design whose
answer is known in closed form, a library least-squares solve of the page's objective,
the normal equations, noiseless recovery, the large-lambda limit, chunk invariance and
optimality of the objective."""

import numpy as np
import pytest

import oracle
from ridge_map_kv_amd import synth


def _stats(xS, xl, chunks=1):
    st = oracle.calib_new(xS.shape[1], len(xl), np.asarray(xl[0]).shape[1])
    for part in np.array_split(np.arange(xS.shape[0]), chunks):
        oracle.calib_accumulate(st, xS[part], [y[part] for y in xl])
    return st


def _hadamard_design(n=2048, d=64, shift=0.0, seed=5, d_out=None):
    d_out = d_out or d
    H = synth.sylvester_hadamard(n).astype(np.float64)
    X = H[:, 1:d + 1]                       # columns 1..d: +-1, zero column means
    W = synth.sparse_dyadic_matrix(d_out, d, seed).astype(np.float64)
    c = np.random.default_rng(seed).integers(-8, 9, size=d_out) / 4.0
    m = np.random.default_rng(seed + 1).integers(-4, 5, size=d) / 2.0 * (shift != 0)
    xS = X + m
    Y = xS @ W.T + c
    return xS, Y, W, c, m


@pytest.mark.parametrize("lam", [1e-4, 0.03, 1.0])
@pytest.mark.parametrize("shift", [0.0, 1.0])
@pytest.mark.parametrize("d_out", [64, 40, 96])
def test_hadamard_closed_form(lam, shift, d_out):
    # centred X^T X = n I, so alpha = lam n and A = W n (n + lam n)^-1 = W / (1 + lam);
    # b = mu_l - A mu_S = (W m + c) - W m / (1 + lam) = c + lam / (1 + lam) W m.
    # d_out != 64: a rectangular map (output width differs from the split state's width)
    n, d = 2048, 64
    xS, Y, W, c, m = _hadamard_design(n, d, shift, d_out=d_out)
    st = _stats(xS, Y[None], chunks=3)
    mu_S, mu_l, XtX, YtX = oracle.centred_moments(st)
    np.testing.assert_allclose(XtX, n * np.eye(d), atol=1e-9)
    assert oracle.ridge_alpha(XtX, lam) == pytest.approx(lam * n, rel=1e-14)
    A, b = oracle.solve(st, lam)
    np.testing.assert_allclose(A[0], W / (1 + lam), atol=1e-12)
    np.testing.assert_allclose(b[0], c + lam / (1 + lam) * (W @ m), atol=1e-10)


def _gauss_problem(n=3000, d=24, noise=0.3, seed=7, shift=0.5, d_out=None):
    d_out = d_out or d
    g = np.random.default_rng(seed)
    xS = g.standard_normal((n, d)) @ (np.eye(d) + 0.3 * g.standard_normal((d, d))) + shift
    W = g.standard_normal((d_out, d)) / np.sqrt(d)
    c = g.standard_normal(d_out)
    Y = xS @ W.T + c + noise * g.standard_normal((n, d_out))
    return xS, Y, W, c


@pytest.mark.parametrize("lam", [1e-3, 0.03, 0.5])
@pytest.mark.parametrize("d_out", [24, 9, 40])
def test_matches_lstsq_of_objective(lam, d_out):
    # Solve the page's objective another way: least squares on [x_S, 1] with sqrt(alpha) I
    # rows that penalise A but not b.  alpha from the centred trace = n * sum of variances
    # over the d_in input features (d_out != d_in: a rectangular map).
    xS, Y, _, _ = _gauss_problem(d_out=d_out)
    n, d = xS.shape
    alpha = lam * n * np.var(xS, axis=0).sum() / d
    aug = np.vstack([np.hstack([xS, np.ones((n, 1))]),
                     np.hstack([np.sqrt(alpha) * np.eye(d), np.zeros((d, 1))])])
    rhs = np.vstack([Y, np.zeros((d, d_out))])
    sol, *_ = np.linalg.lstsq(aug, rhs, rcond=None)
    A_ref, b_ref = sol[:d].T, sol[d]
    A, b = oracle.solve(_stats(xS, Y[None]), lam)
    np.testing.assert_allclose(A[0], A_ref, rtol=1e-8, atol=1e-10)
    np.testing.assert_allclose(b[0], b_ref, rtol=1e-8, atol=1e-10)


def test_one_pass_equals_direct_centring():
    xS, Y, _, _ = _gauss_problem(seed=8)
    A, b = oracle.solve(_stats(xS, Y[None], chunks=4), 0.03)
    A2, b2 = oracle.fit_direct(xS, Y, 0.03)
    np.testing.assert_allclose(A[0], A2, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(b[0], b2, rtol=1e-9, atol=1e-11)


def test_normal_equations_and_bias_identity():
    xS, Y, _, _ = _gauss_problem(seed=9)
    st = _stats(xS, np.stack([Y, 2 * Y - 1]))
    lam = 0.01
    A, b = oracle.solve(st, lam)
    mu_S, mu_l, XtX, YtX = oracle.centred_moments(st)
    alpha = oracle.ridge_alpha(XtX, lam)
    for l in range(2):
        R = (XtX + alpha * np.eye(XtX.shape[0])) @ A[l].T - YtX[l].T
        assert np.linalg.norm(R) / np.linalg.norm(YtX[l]) < 1e-12
        np.testing.assert_allclose(b[l], mu_l[l] - A[l] @ mu_S, rtol=1e-13, atol=1e-13)


def test_objective_is_minimal():
    xS, Y, _, _ = _gauss_problem(n=800, d=10, seed=10)
    lam = 0.05
    st = _stats(xS, Y[None])
    A, b = oracle.solve(st, lam)
    alpha = oracle.ridge_alpha(oracle.centred_moments(st)[2], lam)
    f0 = oracle.ridge_objective(xS, Y, A[0], b[0], alpha)
    g = np.random.default_rng(0)
    for _ in range(20):
        dA = 1e-3 * g.standard_normal(A[0].shape)
        db = 1e-3 * g.standard_normal(b[0].shape)
        assert oracle.ridge_objective(xS, Y, A[0] + dA, b[0] + db, alpha) > f0


def test_noiseless_recovery_small_lambda():
    xS, Y, W, c = _gauss_problem(noise=0.0, seed=11)
    A, b = oracle.solve(_stats(xS, Y[None]), 1e-10)
    np.testing.assert_allclose(A[0], W, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(b[0], c, rtol=1e-6, atol=1e-7)


def test_large_lambda_limit():
    xS, Y, W, c = _gauss_problem(seed=12)
    st = _stats(xS, Y[None])
    A, b = oracle.solve(st, 1e9)
    assert np.abs(A).max() < 1e-8
    np.testing.assert_allclose(b[0], Y.mean(axis=0), rtol=1e-7, atol=1e-7)


def test_chunk_split_invariance():
    xS, Y, _, _ = _gauss_problem(seed=13)
    s1 = _stats(xS, Y[None], chunks=1)
    s5 = _stats(xS, Y[None], chunks=5)
    assert s1.n == s5.n
    np.testing.assert_allclose(s1.G, s5.G, rtol=1e-12)
    np.testing.assert_allclose(s1.YX, s5.YX, rtol=1e-12)
    np.testing.assert_allclose(s1.s_S, s5.s_S, rtol=1e-12)


def test_rejects_negative_lambda_and_empty():
    xS, Y, _, _ = _gauss_problem(n=50, d=4)
    with pytest.raises(ValueError):
        oracle.solve(_stats(xS, Y[None]), -1.0)
    with pytest.raises(ValueError):
        oracle.solve(oracle.calib_new(4, 1), 0.1)


def test_synthetic_calibration_model_near_identity():
    # The synthetic layer inputs follow W_true = I + U diag(0.5) V^T: a fit with many rows
    # and small lambda lands near it.
    d, rows = 32, 20000
    xS, xl = synth.calib_data(d, 1, rows, seed=3, noise_scale=0.1)
    A, b = oracle.solve(_stats(xS.astype(np.float64), xl.astype(np.float64)), 1e-6)
    U, V = synth.true_map_factors(d, 3, 0)
    Wt = np.eye(d) + 0.5 * U.astype(np.float64) @ V.T.astype(np.float64)
    assert np.linalg.norm(A[0] - Wt) / np.linalg.norm(Wt) < 0.01
