"""GPU parity of ridgefill_solve against the oracle and against closed forms."""

import numpy as np
import pytest
import torch

import oracle
from ridge_map_kv_amd import binding as B
from ridge_map_kv_amd import synth

from test_gpu_calib import bf16, f64, run_calib

pytestmark = pytest.mark.gpu
TOL = 5e-3


def gpu_solve(state, d, L, lam):
    A = torch.empty((L, d, d), dtype=torch.float32, device="cuda")
    Ab = torch.empty((L, d, d), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((L, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.ridgefill_solve_workspace_bytes(d, L), dtype=torch.uint8, device="cuda")
    B.ridgefill_solve(state, d, L, lam, A, b, Ab, ws)
    status = B.ridgefill_read_status(ws)
    return A.cpu().numpy().astype(np.float64), b.cpu().numpy().astype(np.float64), Ab, status


def rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("lam", [1e-4, 0.03, 1.0])
def test_solve_matches_oracle(lam):
    d, L, rows = 512, 3, 4000
    xS, xl = synth.calib_data(d, L, rows, seed=51, noise_scale=0.1, noise_dof=3.0, x_shift=0.25)
    xs_g, xl_g = bf16(xS), [bf16(y) for y in xl]
    state = run_calib([xs_g[:2500], xs_g[2500:]], [[y[:2500] for y in xl_g],
                                                   [y[2500:] for y in xl_g]], d, L)
    A, b, Ab, status = gpu_solve(state, d, L, lam)
    assert status == B.RF_OK
    st = oracle.calib_new(d, L)
    oracle.calib_accumulate(st, f64(xs_g), [f64(y) for y in xl_g])
    Ao, bo = oracle.solve(st, lam)
    for l in range(L):
        assert rel(A[l], Ao[l]) < TOL, (l, rel(A[l], Ao[l]))
        assert rel(b[l], bo[l]) < TOL, (l, rel(b[l], bo[l]))
    # the bf16 copy is the RNE rounding of the fp32 map
    assert torch.equal(Ab.cpu(), torch.from_numpy(A.astype(np.float32)).to(torch.bfloat16))
    # normal equations with the oracle's float64 moments
    _, _, XtX, YtX = oracle.centred_moments(st)
    alpha = oracle.ridge_alpha(XtX, lam)
    for l in range(L):
        R = (XtX + alpha * np.eye(d)) @ A[l].T - YtX[l].T
        assert np.linalg.norm(R) / np.linalg.norm(YtX[l]) < 1e-4


@pytest.mark.parametrize("lam", [1e-4, 0.03, 1.0])
def test_solve_hadamard_closed_form(lam):
    n, d, L = 2048, 256, 2
    H = synth.sylvester_hadamard(n).astype(np.float64)
    m = np.random.default_rng(61).integers(-2, 3, size=d) / 2.0
    X = H[:, 1:d + 1] + m
    Ws = [synth.sparse_dyadic_matrix(d, d, 62 + l).astype(np.float64) for l in range(L)]
    cs = [np.random.default_rng(70 + l).integers(-8, 9, size=d) / 4.0 for l in range(L)]
    Y = [X @ W.T + c for W, c in zip(Ws, cs)]
    xs_g, yl_g = bf16(X), [bf16(y) for y in Y]
    assert np.array_equal(f64(xs_g), X)
    A, b, _, status = gpu_solve(run_calib([xs_g], [yl_g], d, L), d, L, lam)
    assert status == B.RF_OK
    for l in range(L):
        np.testing.assert_allclose(A[l], Ws[l] / (1 + lam), atol=1e-5)
        np.testing.assert_allclose(b[l], cs[l] + lam / (1 + lam) * (Ws[l] @ m), atol=1e-4)


def test_noiseless_recovery_small_lambda():
    d, L, rows = 256, 1, 8192
    g = np.random.default_rng(71)
    X = g.standard_normal((rows, d)).astype(np.float32)
    U, V = synth.true_map_factors(d, 72, 0)
    W = np.eye(d) + 0.5 * U.astype(np.float64) @ V.T.astype(np.float64)
    c = g.standard_normal(d)
    xs_g = bf16(X)
    Y = f64(xs_g) @ W.T + c
    A, b, _, status = gpu_solve(run_calib([xs_g], [[bf16(Y)]], d, L), d, L, 1e-8)
    assert status == B.RF_OK
    # only the bf16 rounding of Y separates the data from an exact linear map
    assert rel(A[0], W) < TOL and rel(b[0], c) < TOL


def test_resolve_reuses_state_unchanged():
    d, L, rows = 256, 2, 2000
    xS, xl = synth.calib_data(d, L, rows, seed=81)
    state = run_calib([bf16(xS)], [[bf16(y) for y in xl]], d, L)
    before = state.clone()
    A1, b1, _, _ = gpu_solve(state, d, L, 0.01)
    gpu_solve(state, d, L, 0.5)
    A2, b2, _, _ = gpu_solve(state, d, L, 0.01)
    assert torch.equal(state, before)
    assert np.array_equal(A1, A2) and np.array_equal(b1, b2)


def test_not_spd_is_flagged():
    # a constant feature makes the centred X^T X singular; with lambda = 0 the first
    # pivot is exactly zero
    d, L, rows = 256, 1, 1024
    X = np.random.default_rng(91).standard_normal((rows, d)).astype(np.float32)
    X[:, 0] = 1.0
    _, _, _, status = gpu_solve(run_calib([bf16(X)], [[bf16(X)]], d, L), d, L, 0.0)
    assert status == B.RF_E_NOT_SPD


def test_solve_argument_errors():
    d, L = 256, 1
    state = torch.zeros(B.ridgefill_calib_state_bytes(d, L), dtype=torch.uint8, device="cuda")
    B.ridgefill_calib_reset(state, d, L)
    b = torch.empty((L, d), dtype=torch.float32, device="cuda")
    A = torch.empty((L, d, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.ridgefill_solve_workspace_bytes(d, L), dtype=torch.uint8, device="cuda")
    with pytest.raises(B.RidgeFillError) as e:
        B.ridgefill_solve(state, d, L, -1.0, A, b, None, ws)
    assert e.value.status == B.RF_E_INVALID
    with pytest.raises(B.RidgeFillError) as e:
        B.ridgefill_solve(state, d, L, 0.1, A, b, None, ws[:4096])
    assert e.value.status == B.RF_E_WORKSPACE
    with pytest.raises(B.RidgeFillError) as e:
        B.ridgefill_solve(state, d, L, 0.1, None, b, None, ws)
    assert e.value.status == B.RF_E_INVALID
