"""Pins of the oracle's fill (map prediction, RMSNorm, K/V projection, RoPE, paged
write) against closed forms, library routines and invariants.  Each test is chosen so
that a plausible slip (a transposed map, a missing eps, a wrong rotation sign or pair,
a wrong frequency exponent, writing outside the filled rows) fails it."""

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- map prediction

def test_identity_map_is_identity_fill():
    # Table 3's identity arm: x_hat = x_S exactly when A = I, b = 0.
    x = _rand((7, 16))
    out = oracle.predict_input(x, np.eye(16), np.zeros(16))
    assert np.array_equal(out, x)


def test_map_orientation_permutation():
    # A[o][i] = 1 where i = pi(o): x_hat[o] = x[pi(o)]; a transposed map gives pi^-1.
    d = 9
    pi = np.array([3, 0, 8, 1, 2, 7, 4, 6, 5])
    A = np.zeros((d, d))
    A[np.arange(d), pi] = 1.0
    x = np.arange(2 * d, dtype=np.float64).reshape(2, d)
    out = oracle.predict_input(x, A, np.zeros(d))
    assert np.array_equal(out, x[:, pi])
    assert not np.array_equal(out, x[:, np.argsort(pi)])


def test_map_bias_added_once():
    x = np.zeros((3, 4))
    b = np.array([1.0, -2.0, 0.5, 4.0])
    assert np.array_equal(oracle.predict_input(x, _rand((4, 4)), b), np.tile(b, (3, 1)))


# ---------------------------------------------------------------- RMSNorm

def test_rms_norm_matches_torch_library():
    x = _rand((5, 64), 1)
    w = 1 + 0.1 * _rand(64, 2)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(w),
                                       eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.rms_norm(x, w, 1e-5), ref, rtol=1e-13, atol=1e-14)


def test_rms_norm_scale_invariance_and_eps():
    x = _rand((4, 32), 3)
    w = 1 + 0.1 * _rand(32, 4)
    np.testing.assert_allclose(oracle.rms_norm(2 * x, w, 0.0), oracle.rms_norm(x, w, 0.0),
                               rtol=1e-14)
    # eps is inside the root: a zero row stays zero, a tiny row is not blown up
    z = np.zeros((1, 32))
    assert np.array_equal(oracle.rms_norm(z, w, 1e-5), z)
    small = np.full((1, 32), 1e-4)
    assert np.all(np.abs(oracle.rms_norm(small, np.ones(32), 1e-5)) < 0.05)


def test_one_hot_closed_form():
    # x_S = s e_j, A = I, b = 0:  K_pre = sqrt(d) w_j / sqrt(1 + eps d / s^2) W_K[:, j]
    d, kv, hd, n_kv, eps = 32, 8, 4, 2, 1e-5
    s, j = 0.7, 5
    x = np.zeros((1, d)); x[0, j] = s
    w = 1 + 0.1 * _rand(d, 5)
    WK = _rand((kv, d), 6); WV = _rand((kv, d), 7)
    K, V = oracle.fill_rows(x, [0], np.eye(d), np.zeros(d), w, WK, WV,
                            eps=eps, theta=10000.0, n_kv=n_kv, hd=hd)
    coef = np.sqrt(d) * w[j] / np.sqrt(1 + eps * d / s ** 2)
    np.testing.assert_allclose(K.reshape(-1), coef * WK[:, j], rtol=1e-13)
    np.testing.assert_allclose(V.reshape(-1), coef * WV[:, j], rtol=1e-13)


def test_head_layout_is_head_major():
    # column block [h*hd, (h+1)*hd) of the projection output is head h
    d, n_kv, hd = 8, 3, 4
    WK = np.zeros((n_kv * hd, d)); WK[1 * hd + 2, 0] = 1.0   # head 1, lane 2 reads x[0]
    h = np.zeros((1, d)); h[0, 0] = 3.0
    K, V = oracle.project_kv(h, WK, WK, n_kv, hd)
    expect = np.zeros((1, n_kv, hd)); expect[0, 1, 2] = 3.0
    assert np.array_equal(K, expect)


# ---------------------------------------------------------------- RoPE

def test_rope_inverse_frequencies_hand_values():
    np.testing.assert_allclose(oracle.rope_inv_freq(4, 100.0), [1.0, 0.1], rtol=1e-15)
    f = oracle.rope_inv_freq(128, 500000.0)
    assert f[0] == 1.0
    np.testing.assert_allclose(f[63], 500000.0 ** (-126 / 128), rtol=1e-14)


def test_rope_matches_complex_multiplication():
    # rotate-half pairing: z_j = k_j + i k_{j+hd/2} is multiplied by exp(i t f_j)
    rows, heads, hd, theta = 6, 3, 16, 500000.0
    k = _rand((rows, heads, hd), 8)
    pos = np.array([0, 1, 7, 100, 4095, 65535])
    out = oracle.rope_keys(k, pos, theta)
    z = k[..., : hd // 2] + 1j * k[..., hd // 2:]
    ang = pos[:, None] * (theta ** (-np.arange(0, hd, 2) / hd))[None, :]
    zr = z * np.exp(1j * ang)[:, None, :]
    np.testing.assert_allclose(out[..., : hd // 2], zr.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out[..., hd // 2:], zr.imag, rtol=1e-12, atol=1e-12)


def test_rope_position_one_first_pair_by_hand():
    k = np.zeros((1, 1, 4)); k[0, 0, 0] = 1.0          # unit vector on lane 0
    out = oracle.rope_keys(k, [1], 100.0)
    # lane 0 pairs with lane 2, frequency 1, angle 1 rad
    np.testing.assert_allclose(out[0, 0], [np.cos(1.0), 0.0, np.sin(1.0), 0.0], atol=1e-15)


def test_rope_invariants():
    rows, heads, hd = 5, 2, 8
    k = _rand((rows, heads, hd), 9)
    q = _rand((rows, heads, hd), 10)
    assert np.array_equal(oracle.rope_keys(k, np.zeros(rows), 5e5), k)
    pos = np.array([3, 10, 200, 999, 31])
    r = oracle.rope_keys(k, pos, 5e5)
    half = hd // 2
    np.testing.assert_allclose(r[..., :half] ** 2 + r[..., half:] ** 2,
                               k[..., :half] ** 2 + k[..., half:] ** 2, rtol=1e-12)
    # <R(m) q, R(n) k> depends only on m - n
    a = np.sum(oracle.rope_keys(q, pos, 5e5) * oracle.rope_keys(k, pos + 17, 5e5), -1)
    b = np.sum(oracle.rope_keys(q, pos + 1000, 5e5) * oracle.rope_keys(k, pos + 1017, 5e5), -1)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)


def test_values_are_not_rotated():
    d, n_kv, hd = 16, 2, 4
    x = np.tile(_rand((1, d), 11), (2, 1))
    A = np.eye(d) + 0.1 * _rand((d, d), 12)
    w = np.ones(d); WK = _rand((8, d), 13); WV = _rand((8, d), 14)
    K, V = oracle.fill_rows(x, [0, 999], A, np.zeros(d), w, WK, WV,
                            eps=1e-5, theta=5e5, n_kv=n_kv, hd=hd)
    assert np.array_equal(V[0], V[1])
    assert not np.allclose(K[0], K[1])


# ---------------------------------------------------------------- paged cache

def _tiny_layer(d, kv, seed):
    return dict(A=np.eye(d) + 0.05 * _rand((d, d), seed), b=_rand(d, seed + 1),
                norm_w=1 + 0.1 * _rand(d, seed + 2), W_K=_rand((kv, d), seed + 3),
                W_V=_rand((kv, d), seed + 4))


def test_paged_write_touches_only_filled_rows():
    N, T, d, n_kv, hd, ps = 12, 3, 16, 2, 4, 4
    filled, _, _ = oracle.partition(N, T, [2, 5])
    table = np.array([4, 0, 2], dtype=np.int32)          # 3 logical pages, 5 physical
    sentinel = -7.25
    kc = np.full((5, ps, n_kv, hd), sentinel); vc = kc.copy()
    x = _rand((N, d), 20)
    lay = _tiny_layer(d, n_kv * hd, 30)
    oracle.fill_paged_cache(kc, vc, x, filled, lay, block_table=table, page_size=ps,
                            eps=1e-5, theta=5e5, n_kv=n_kv, hd=hd)
    written = np.zeros((5, ps), dtype=bool)
    pg, sl = oracle.paged_location(filled, table, ps)
    written[pg, sl] = True
    assert np.all(kc[~written] == sentinel) and np.all(vc[~written] == sentinel)
    assert not np.any(kc[written] == sentinel)
    # row 6 lives on logical page 1 -> physical page 0, slot 2
    assert oracle.paged_location(6, table, ps) == (0, 2)
    K, V = oracle.fill_rows(x[[6]], [6], lay["A"], lay["b"], lay["norm_w"], lay["W_K"],
                            lay["W_V"], eps=1e-5, theta=5e5, n_kv=n_kv, hd=hd)
    np.testing.assert_allclose(kc[0, 2], K[0], rtol=1e-13)
    np.testing.assert_allclose(vc[0, 2], V[0], rtol=1e-13)


def test_permuted_table_same_logical_cache():
    N, T, d, n_kv, hd, ps = 12, 3, 16, 2, 4, 4
    filled, _, _ = oracle.partition(N, T, [1])
    x = _rand((N, d), 21)
    lay = _tiny_layer(d, n_kv * hd, 40)

    def logical(table, num):
        kc = np.zeros((num, ps, n_kv, hd)); vc = kc.copy()
        oracle.fill_paged_cache(kc, vc, x, filled, lay, block_table=table, page_size=ps,
                                eps=1e-5, theta=5e5, n_kv=n_kv, hd=hd)
        return kc[table].reshape(-1, n_kv, hd)[:N], vc[table].reshape(-1, n_kv, hd)[:N]

    a = logical(np.arange(3, dtype=np.int32), 3)
    b = logical(np.array([5, 1, 3], dtype=np.int32), 6)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_no_fill_leaves_cache_unchanged():
    kc = _rand((3, 4, 2, 4), 50); vc = _rand((3, 4, 2, 4), 51)
    k0, v0 = kc.copy(), vc.copy()
    oracle.fill_paged_cache(kc, vc, _rand((12, 16), 52), [], _tiny_layer(16, 8, 60),
                            block_table=np.arange(3), page_size=4, eps=1e-5, theta=5e5,
                            n_kv=2, hd=4)
    assert np.array_equal(kc, k0) and np.array_equal(vc, v0)


def test_rows_independent():
    d, n_kv, hd = 16, 2, 4
    x = _rand((6, d), 70)
    lay = _tiny_layer(d, n_kv * hd, 80)
    pos = np.arange(6) * 3
    kw = dict(eps=1e-5, theta=5e5, n_kv=n_kv, hd=hd)
    K, V = oracle.fill_rows(x, pos, lay["A"], lay["b"], lay["norm_w"], lay["W_K"], lay["W_V"], **kw)
    K2, V2 = oracle.fill_rows(x[3:], pos[3:], lay["A"], lay["b"], lay["norm_w"], lay["W_K"],
                              lay["W_V"], **kw)
    np.testing.assert_allclose(K[3:], K2, rtol=1e-14)
    np.testing.assert_allclose(V[3:], V2, rtol=1e-14)
