"""CPU pins of the oracle's folded form (fold_map, fill_rows_folded).

The folded form claims two identities for every input row x: the projections of the
normalised prediction equal P x + c up to the row scale, and |A x + b|^2 equals
|R x + r|^2 + kappa.  Each check below compares against the plain flow computed another
way (fill_rows, or the prediction written out here), a factor-free closed form worked
out by hand, or a library routine (scipy's QR) that reaches the same triangular factor
by a different algorithm."""

import numpy as np
import pytest
import scipy.linalg

import oracle


def _layer(g, d_out, d_in, kv, near_identity=True):
    if near_identity and d_out == d_in:
        A = np.eye(d_in) + 0.05 * g.standard_normal((d_out, d_in))
    else:
        A = g.standard_normal((d_out, d_in)) / np.sqrt(d_in)
    b = 0.3 * g.standard_normal(d_out)
    w = 1.0 + 0.1 * g.standard_normal(d_out)
    W_K = g.standard_normal((kv, d_out)) / np.sqrt(d_out)
    W_V = g.standard_normal((kv, d_out)) / np.sqrt(d_out)
    return A, b, w, W_K, W_V


@pytest.mark.parametrize("d_out,d_in,near", [(40, 40, True), (40, 40, False), (48, 32, False),
                                             (96, 64, False)])
def test_sum_of_squares_identity(d_out, d_in, near):
    g = np.random.default_rng(d_out * 100 + d_in)
    A, b, w, W_K, W_V = _layer(g, d_out, d_in, 16, near)
    P, c, R, r, kappa = oracle.fold_map(A, b, w, W_K, W_V)
    x = g.standard_normal((25, d_in))
    plain = np.sum((x @ A.T + b) ** 2, axis=1)
    folded = np.sum((x @ R.T + r) ** 2, axis=1) + kappa
    np.testing.assert_allclose(folded, plain, rtol=1e-11)


@pytest.mark.parametrize("d_out,d_in", [(40, 40), (48, 32)])
def test_projection_identity(d_out, d_in):
    g = np.random.default_rng(7 + d_in)
    A, b, w, W_K, W_V = _layer(g, d_out, d_in, 16, False)
    P, c, R, r, kappa = oracle.fold_map(A, b, w, W_K, W_V)
    x = g.standard_normal((9, d_in))
    x_hat = x @ A.T + b
    ref = np.concatenate([(x_hat * w) @ W_K.T, (x_hat * w) @ W_V.T], axis=1)
    np.testing.assert_allclose(x @ P.T + c, ref, rtol=1e-11, atol=1e-12)


def test_factor_is_qr_triangle():
    # A = Q R_qr (reduced QR): R_qr^T R_qr = A^T A, so with the signs of R_qr's diagonal
    # made positive it is the unique Cholesky factor; r = Q^T b in the same sign
    # convention, and kappa = |b - Q Q^T b|^2.
    g = np.random.default_rng(11)
    A, b, w, W_K, W_V = _layer(g, 48, 32, 8, False)
    _, c_, R, r, kappa = oracle.fold_map(A, b, w, W_K, W_V)
    Q, Rq = scipy.linalg.qr(A, mode="economic")
    s = np.sign(np.diag(Rq))
    Rq = Rq * s[:, None]
    Q = Q * s[None, :]
    np.testing.assert_allclose(R, Rq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(r, Q.T @ b, rtol=1e-10, atol=1e-12)
    resid = b - Q @ (Q.T @ b)
    np.testing.assert_allclose(kappa, resid @ resid, rtol=1e-9)
    assert np.all(np.tril(R, -1) == 0.0) and np.all(np.diag(R) > 0)


def test_identity_map_closed_form():
    # A = I: R = I, r = b, kappa = 0, P = [W_K; W_V] diag(w), c = [W_K; W_V] (w * b).
    g = np.random.default_rng(3)
    d, kv = 32, 8
    _, b, w, W_K, W_V = _layer(g, d, d, kv)
    P, c, R, r, kappa = oracle.fold_map(np.eye(d), b, w, W_K, W_V)
    np.testing.assert_allclose(R, np.eye(d), atol=1e-15)
    np.testing.assert_allclose(r, b, rtol=1e-14)
    assert abs(kappa) <= 1e-13 * (b @ b)
    np.testing.assert_allclose(P[:kv], W_K * w[None, :], rtol=1e-15)
    np.testing.assert_allclose(P[kv:], W_V * w[None, :], rtol=1e-15)
    np.testing.assert_allclose(c[kv:], W_V @ (w * b), rtol=1e-13)


def test_diagonal_and_orthogonal_maps():
    g = np.random.default_rng(5)
    d, kv = 16, 8
    _, b, w, W_K, W_V = _layer(g, d, d, kv)
    s = 0.5 + g.random(d)                      # positive diagonal: R = diag(s), r = b
    _, _, R, r, kappa = oracle.fold_map(np.diag(s), b, w, W_K, W_V)
    np.testing.assert_allclose(R, np.diag(s), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r, b, rtol=1e-13)
    assert abs(kappa) <= 1e-12 * (b @ b)
    H = scipy.linalg.hadamard(d) / 4.0         # orthogonal and symmetric: R = I, r = H b
    _, _, R, r, kappa = oracle.fold_map(H, b, w, W_K, W_V)
    np.testing.assert_allclose(R, np.eye(d), atol=1e-14)
    np.testing.assert_allclose(r, H @ b, rtol=1e-13, atol=1e-14)
    assert abs(kappa) <= 1e-12 * (b @ b)


def test_tall_map_kappa_is_distance_to_column_space():
    # A = [I; 0] (d_out = 2 d_in): R = I, r = b[:d_in], kappa = |b[d_in:]|^2.
    g = np.random.default_rng(9)
    d_in, kv = 16, 8
    A = np.concatenate([np.eye(d_in), np.zeros((d_in, d_in))])
    _, b, w, W_K, W_V = _layer(g, 2 * d_in, d_in, kv)
    _, _, R, r, kappa = oracle.fold_map(A, b, w, W_K, W_V)
    np.testing.assert_allclose(R, np.eye(d_in), atol=1e-15)
    np.testing.assert_allclose(r, b[:d_in], rtol=1e-14)
    np.testing.assert_allclose(kappa, b[d_in:] @ b[d_in:], rtol=1e-13)


def test_wide_map_has_no_fold():
    g = np.random.default_rng(13)
    A, b, w, W_K, W_V = _layer(g, 16, 32, 8, False)   # A^T A has rank 16 < 32
    with pytest.raises(np.linalg.LinAlgError):
        oracle.fold_map(A, b, w, W_K, W_V)


@pytest.mark.parametrize("d_out,d_in,hd,knorm,vscale", [(64, 64, 16, False, False),
                                                         (64, 64, 16, True, True),
                                                         (96, 64, 32, False, True)])
def test_folded_fill_equals_plain_fill(d_out, d_in, hd, knorm, vscale):
    g = np.random.default_rng(d_out + hd)
    n_kv = 2
    A, b, w, W_K, W_V = _layer(g, d_out, d_in, n_kv * hd, d_out == d_in)
    kn = 1.0 + 0.2 * g.standard_normal(hd) if knorm else None
    vs = 0.5 + g.random(n_kv) if vscale else None
    x = g.standard_normal((11, d_in))
    pos = np.sort(g.choice(1000, 11, replace=False))
    kw = dict(eps=1e-5, theta=10000.0, n_kv=n_kv, hd=hd, k_norm_w=kn, v_scale=vs)
    K0, V0 = oracle.fill_rows(x, pos, A, b, w, W_K, W_V, **kw)
    P, c, R, r, kappa = oracle.fold_map(A, b, w, W_K, W_V)
    K1, V1 = oracle.fill_rows_folded(x, pos, P, c, R, r, kappa, d_out, **kw)
    np.testing.assert_allclose(K1, K0, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(V1, V0, rtol=1e-10, atol=1e-12)
