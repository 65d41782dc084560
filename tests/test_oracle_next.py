"""CPU pins of the oracle's widening functions: key normalization, value rescale,
int8 maps and exact-row selection from scores.

Each check leans on something other than the oracle's own formula: a library routine,
a closed form worked out here by hand, an invariant or brute force."""

import itertools

import numpy as np
import pytest
import torch

import oracle


def test_key_norm_is_torch_rms_norm_per_head():
    g = np.random.default_rng(0)
    K = g.standard_normal((7, 3, 16))
    w = 1.0 + 0.1 * g.standard_normal(16)
    got = oracle.key_norm(K, w, 1e-5)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(K), (16,), torch.from_numpy(w), 1e-5)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_key_norm_before_rope_closed_form():
    # x_S = s e_j, A = I, b = 0, norm weight w: the normalized input is h e_j with
    # h = s / sqrt(s^2 / d + eps) * w_j.  W_K sends feature j to element 0 of key head 0,
    # so head 0 before the key norm is [h, 0, ...] and every other head is zero.  The key
    # norm gives element 0 the value h / sqrt(h^2 / hd + eps) * wk_0, and RoPE at position
    # t (inverse frequency 1 for pair 0) turns it into (.. cos t, .. sin t) at (0, hd/2).
    # Applying RoPE first would put wk_{hd/2} on the sine term instead.
    d, n_kv, hd, eps, s, j, t = 64, 2, 16, 1e-6, 3.0, 5, 11
    g = np.random.default_rng(1)
    w = 1.0 + 0.1 * g.standard_normal(d)
    wk = 1.0 + 0.3 * g.standard_normal(hd)
    W_K = np.zeros((n_kv * hd, d))
    W_K[0, j] = 1.0
    W_V = g.standard_normal((n_kv * hd, d)) / np.sqrt(d)
    x = np.zeros((1, d))
    x[0, j] = s
    K, _ = oracle.fill_rows(x, [t], np.eye(d), np.zeros(d), w, W_K, W_V, eps=eps, theta=5e5,
                            n_kv=n_kv, hd=hd, k_norm_w=wk)
    h = s / np.sqrt(s * s / d + eps) * w[j]
    k0 = h / np.sqrt(h * h / hd + eps) * wk[0]
    want = np.zeros((n_kv, hd))
    want[0, 0] = k0 * np.cos(t)
    want[0, hd // 2] = k0 * np.sin(t)
    np.testing.assert_allclose(K[0], want, rtol=1e-12, atol=1e-12)


def test_key_norm_fixes_head_magnitude_after_rope():
    # with a unit key-norm weight and eps = 0 every key head has norm sqrt(hd), whatever
    # the input and the position (RoPE is a rotation)
    g = np.random.default_rng(2)
    d, n_kv, hd = 128, 4, 32
    x = g.standard_normal((9, d))
    A = np.eye(d) + 0.1 * g.standard_normal((d, d))
    K, V = oracle.fill_rows(x, np.arange(9) * 977, A, g.standard_normal(d), 1 + 0.1 * g.standard_normal(d),
                            g.standard_normal((n_kv * hd, d)), g.standard_normal((n_kv * hd, d)),
                            eps=0.0, theta=1e4, n_kv=n_kv, hd=hd, k_norm_w=np.ones(hd))
    np.testing.assert_allclose(np.linalg.norm(K, axis=-1), np.sqrt(hd), rtol=1e-12)
    assert not np.allclose(np.linalg.norm(V, axis=-1), np.sqrt(hd))


def test_value_scale_is_one_when_exact_equals_prediction():
    g = np.random.default_rng(3)
    d, n_kv, hd, c = 64, 2, 16, 10
    A = g.standard_normal((d, d)) / 8
    b = g.standard_normal(d)
    xs = g.standard_normal((c, d))
    s = oracle.value_scale(xs, xs @ A.T + b, A, b, 1 + 0.1 * g.standard_normal(d),
                           g.standard_normal((n_kv * hd, d)), eps=1e-5, n_kv=n_kv, hd=hd)
    np.testing.assert_allclose(s, 1.0, rtol=1e-13)


def test_value_scale_selection_closed_form():
    # W_V picks coordinates: head h's value is the normalized input restricted to the
    # coordinates sel_h.  With w = 1 and eps = 0 the value of row x is
    # sqrt(d) x[sel_h] / |x|, so the factor is the mean over rows of
    # (|xe[sel_h]| / |xe|) / (|xp[sel_h]| / |xp|), xp the prediction.
    g = np.random.default_rng(4)
    d, n_kv, hd, c = 32, 2, 4, 6
    sel = [np.array([0, 3, 7, 9]), np.array([12, 13, 20, 31])]
    W_V = np.zeros((n_kv * hd, d))
    for h in range(n_kv):
        for i, col in enumerate(sel[h]):
            W_V[h * hd + i, col] = 1.0
    A = np.eye(d) + 0.2 * g.standard_normal((d, d))
    b = 0.5 * g.standard_normal(d)
    xs = g.standard_normal((c, d))
    xe = g.standard_normal((c, d)) * 1.7
    xp = xs @ A.T + b
    want = []
    for h in range(n_kv):
        r = [(np.linalg.norm(xe[t, sel[h]]) / np.linalg.norm(xe[t])) /
             (np.linalg.norm(xp[t, sel[h]]) / np.linalg.norm(xp[t])) for t in range(c)]
        want.append(np.mean(r))
    got = oracle.value_scale(xs, xe, A, b, np.ones(d), W_V, eps=0.0, n_kv=n_kv, hd=hd)
    np.testing.assert_allclose(got, want, rtol=1e-12)


def test_fill_rows_value_scale_multiplies_heads():
    g = np.random.default_rng(5)
    d, n_kv, hd = 64, 4, 16
    args = (g.standard_normal((3, d)), [1, 2, 3], np.eye(d), np.zeros(d), np.ones(d),
            g.standard_normal((n_kv * hd, d)), g.standard_normal((n_kv * hd, d)))
    kw = dict(eps=1e-5, theta=5e5, n_kv=n_kv, hd=hd)
    K0, V0 = oracle.fill_rows(*args, **kw)
    sc = np.array([0.5, 1.0, 2.0, 1.25])
    K1, V1 = oracle.fill_rows(*args, **kw, v_scale=sc)
    np.testing.assert_array_equal(K0, K1)
    np.testing.assert_allclose(V1, V0 * sc[None, :, None], rtol=0, atol=0)


def test_quantize_map_hand_example():
    # row 0: scale 1/127, -0.5 * 127 = -63.5 -> -64 (half to even), 0.25 * 127 = 31.75 -> 32;
    # row 1 is zero; row 2: scale 3/127, 1.5 / scale = 63.5 -> 64
    A = np.array([[1.0, -0.5, 0.25], [0.0, 0.0, 0.0], [3.0, -3.0, 1.5]])
    q, s = oracle.quantize_map_int8(A)
    np.testing.assert_array_equal(q, [[127, -64, 32], [0, 0, 0], [127, -127, 64]])
    np.testing.assert_allclose(s, [1 / 127, 0.0, 3 / 127], rtol=1e-15)


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_quantize_map_error_bound_and_range(dtype):
    g = np.random.default_rng(6)
    A = g.standard_normal((40, 300)) * np.exp(g.standard_normal((40, 1)))
    A[7] = 0.0
    q, s = oracle.quantize_map_int8(A.astype(dtype), dtype)
    assert q.dtype == np.int8 and np.abs(q.astype(int)).max() <= 127
    nz = np.arange(40) != 7
    assert np.all(np.abs(q[nz].astype(int)).max(axis=1) == 127)
    assert np.all(q[7] == 0) and s[7] == 0
    err = np.abs(oracle.dequantize_map_int8(q, s) - A.astype(dtype).astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-5))


def test_quantize_float32_decisions_differ_only_at_ties():
    g = np.random.default_rng(7)
    A = g.standard_normal((64, 512)).astype(np.float32)
    q64, s64 = oracle.quantize_map_int8(A, np.float64)
    q32, s32 = oracle.quantize_map_int8(A, np.float32)
    diff = q64 != q32
    assert np.abs(q64.astype(int) - q32.astype(int)).max() <= 1
    frac = (A.astype(np.float64) / s64[:, None]) % 1.0
    assert np.all(np.abs(frac[diff] - 0.5) < 1e-4)


def test_select_exact_brute_force_validity():
    g = np.random.default_rng(8)
    for trial in range(200):
        P = int(g.integers(1, 9))
        sc = g.integers(0, 4, size=P).astype(float)
        k = int(g.integers(0, P + 1))
        S = oracle.select_exact(sc, k)
        assert S.size == k and np.all(np.diff(S) > 0)
        inside = set(S.tolist())
        for i in inside:
            for j in set(range(P)) - inside:
                assert sc[i] > sc[j] or (sc[i] == sc[j] and i < j)
        # the unique such set: compare with all subsets of size k
        best = [c for c in itertools.combinations(range(P), k)
                if all(sc[i] > sc[j] or (sc[i] == sc[j] and i < j)
                       for i in c for j in set(range(P)) - set(c))]
        assert len(best) == 1 and list(best[0]) == S.tolist()


def test_select_exact_count_of_the_attention_arm():
    # 10% of the 8B workload's 28,672 prefix rows
    P = 32768 - 4096
    k = int(round(0.1 * P))
    assert k == 2867
    sc = np.random.default_rng(9).random(P)
    S = oracle.select_exact(sc, k)
    assert S.size == k and sc[S].min() >= np.sort(sc)[::-1][k - 1]
