"""GPU parity on inputs chosen to break the numerics rather than to stand in for the timing
workloads (section "Ridge map: predict the input, and the original projection runs
unchanged": the closed-form fit on one-pass statistics, the scale-free alpha, and the
predicted input passing through the layer's own normalization and K/V projections).

Calibration and solve:
  * features whose means are 10-50 times their spread (on half of x_S's features and half
    of every layer's outputs): raw fp32 moments would lose the centred part to
    cancellation; the shifted accumulation must match the oracle's float64 accumulation of
    the unshifted rows (A_l and b_l within 5e-3 relative Frobenius);
  * covariance spectra spread over four and six decades (rotated, so the inverse is dense)
    at lambda 1e-4 and 1e-3: the solve of the GPU's own statistics against the oracle's
    float64 Cholesky solve of the same statistics (5e-3), and the normal-equation residual
    (1e-4, or 2.5e-7 kappa_F / d where that is larger: kappa_F / d reaches 7.9e3 here).
Fill, at the 8B layer shape (d = 4096, 8 KV heads x 128), plain and folded layers against
the oracle's plain fill on every filled row: x_S with a few features (0, 1, d - 1 among
them) 50-100 times the others, and maps whose singular values spread over 1e3 and 3e3.
A NaN in one filled row leaves every other row's K and V bit-identical to a clean run.  A calibrate call with sizes other than the reset's marks the state, and a solve on it
reports RF_E_WORKSPACE."""

import numpy as np
import pytest
import torch

import oracle
from ridge_map_kv_amd import binding as B
from ridge_map_kv_amd import synth

from fillcase import Case, build_inputs, check_routing, gpu_rows, oracle_layer, rel_fro, run_fill
from test_gpu_calib import GpuStats, bf16, f64, run_calib

pytestmark = pytest.mark.gpu
TOL = 5e-3


def _gpu_solve(state, d, L, lam):
    A = torch.empty((L, d, d), dtype=torch.float32, device="cuda")
    b = torch.empty((L, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.ridgefill_solve_workspace_bytes(d, L), dtype=torch.uint8, device="cuda")
    B.ridgefill_solve(state, d, L, lam, A, b, None, ws)
    status = B.ridgefill_read_status(ws)
    return A.cpu().numpy().astype(np.float64), b.cpu().numpy().astype(np.float64), status


def _stats_of_state(g: GpuStats, d, L):
    """The GPU's statistics as the oracle's CalibStats (G mirrored from its lower triangle)."""
    st = oracle.calib_new(d, L)
    st.n = g.n
    st.s_S = g.s_S.copy()
    st.s_l = g.s_l.copy()
    low = np.tril(g.G)
    st.G = low + np.tril(low, -1).T
    st.YX = g.YX.copy()
    return st


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_calib_large_means_shifted_and_solved():
    d, L, rows = 512, 2, 8192
    xS, xl = synth.calib_data_hard(d, L, rows, seed=81, mean_lo=10.0, mean_hi=50.0)
    xs_g, xl_g = bf16(xS), [bf16(y) for y in xl]
    cut = 4096
    state = run_calib([xs_g[:cut], xs_g[cut:]], [[y[:cut] for y in xl_g], [y[cut:] for y in xl_g]],
                      d, L)
    g = GpuStats(state, d, L)
    X = f64(xs_g)
    # the shift: the bf16 mean of the first call's rows where it exceeds twice their spread
    m0, s0 = X[:cut].mean(axis=0), X[:cut].std(axis=0)
    want = np.where(np.abs(m0) > 2 * s0, f64(torch.from_numpy(m0.astype(np.float32)).to(torch.bfloat16)),
                    0.0)
    assert np.array_equal(g.shift, want)
    assert np.count_nonzero(g.shift) > d // 4
    # the state holds the moments of bf16(x_S - s), element by element as the GPU forms it
    xsh = f64((xs_g.float() - torch.from_numpy(g.shift.astype(np.float32)).cuda()).to(torch.bfloat16))
    exact = np.mean(xsh == X - g.shift)
    print(f"\nshifted rows exact in bf16: {exact:.4f}", flush=True)
    st = oracle.calib_new(d, L)
    oracle.calib_accumulate(st, xsh, [f64(y) for y in xl_g])
    low = np.tril(np.ones((d, d), dtype=bool))
    assert g.n == rows
    assert _rel(g.G[low], st.G[low]) < 1e-5
    assert _rel(g.YX, st.YX) < 1e-5
    # the fit against the oracle's float64 accumulation of the unshifted rows
    raw = oracle.calib_new(d, L)
    oracle.calib_accumulate(raw, X, [f64(y) for y in xl_g])
    for lam in (1e-4, 0.01, 1.0):
        A, b, status = _gpu_solve(state, d, L, lam)
        assert status == B.RF_OK
        Ao, bo = oracle.solve(raw, lam)
        for l in range(L):
            ea, eb = _rel(A[l], Ao[l]), _rel(b[l], bo[l])
            print(f"  lambda {lam:g} layer {l}: A {ea:.2e} b {eb:.2e}", flush=True)
            assert ea < TOL and eb < TOL


@pytest.mark.parametrize("spread", [1e4, 1e6])
@pytest.mark.parametrize("lam", [1e-4, 1e-3])
def test_solve_ill_conditioned_vs_oracle(spread, lam):
    d, L, rows = 512, 2, 8192
    xS, xl = synth.calib_data_hard(d, L, rows, seed=82, mean_lo=0.0, mean_hi=0.0, spread=spread)
    xs_g, xl_g = bf16(xS), [bf16(y) for y in xl]
    state = run_calib([xs_g], [xl_g], d, L)
    g = GpuStats(state, d, L)
    assert not g.shift.any()
    st = _stats_of_state(g, d, L)
    A, b, status = _gpu_solve(state, d, L, lam)
    assert status == B.RF_OK
    Ao, bo = oracle.solve(st, lam)
    _, _, XtX, YtX = oracle.centred_moments(st)
    alpha = oracle.ridge_alpha(XtX, lam)
    Cp = XtX + alpha * np.eye(d)
    kap = np.linalg.norm(Cp) * np.linalg.norm(np.linalg.inv(Cp))
    for l in range(L):
        ea, eb = _rel(A[l], Ao[l]), _rel(b[l], bo[l])
        res = np.linalg.norm(Cp @ A[l].T - YtX[l].T) / np.linalg.norm(YtX[l])
        print(f"\n  spread {spread:g} lambda {lam:g} kappa_F/d {kap / d:.1e} layer {l}: "
              f"A {ea:.2e} b {eb:.2e} residual {res:.2e}", flush=True)
        assert ea < TOL and eb < TOL
        # the residual of the fp32 map: 1e-4 while kappa_F / d <= 400; beyond, the six-product
        # split's error, about 1e-7 kappa_F / d relative, shows in it (twice that allowed)
        assert res < max(1e-4, 2.5e-7 * kap / d)


def test_calibrate_with_other_sizes_marks_the_state():
    d, L = 256, 3
    xS, xl = synth.calib_data(d, L, 512, seed=83)
    xs_g, xl_g = bf16(xS), [bf16(y) for y in xl]
    state = torch.empty(B.ridgefill_calib_state_bytes(d, L), dtype=torch.uint8, device="cuda")
    B.ridgefill_calib_reset(state, d, L)
    B.ridgefill_calibrate(state, d, L - 1, xs_g, xl_g[:L - 1])      # fewer layers than the reset's
    torch.cuda.synchronize()
    g = GpuStats(state, d, L)
    assert g.n == 0 and not g.G.any() and not g.YX.any() and not g.s_S.any()
    assert g.bad == 1
    A, b, status = _gpu_solve(state, d, L - 1, 0.03)
    assert status == B.RF_E_WORKSPACE
    # a state reset for these sizes solves cleanly
    B.ridgefill_calib_reset(state, d, L)
    B.ridgefill_calibrate(state, d, L, xs_g, xl_g)
    _, _, status = _gpu_solve(state, d, L, 0.03)
    assert status == B.RF_OK


# ------------------------------------------------------------------------ fill, 8B shape

def _hard_case(maps_kind, seed):
    d, n_kv, hd = 4096, 8, 128
    if maps_kind == "spread":
        maps = [(synth.spread_map(d, seed, l, s), synth.rng(seed, 5, l).standard_normal(d).astype(np.float32))
                for l, s in enumerate((1e3, 3e3))]
    else:
        maps = [synth.near_identity_map(d, seed, l) for l in range(2)]
    g = np.random.default_rng(seed)
    N, T = 1300, 100
    exact = np.sort(g.choice(N - T, size=60, replace=False))
    return Case(d=d, n_layers=2, n_kv=n_kv, hd=hd, N=N, T=T, exact=exact, page_size=16, seed=seed,
                map_kind="given", maps=maps)


def _big_features(inp, d, seed):
    g = np.random.default_rng(seed)
    feats = [0, 1, d - 1] + list(g.choice(np.arange(2, d - 1), size=5, replace=False))
    scale = [100.0, 80.0, 100.0] + list(g.uniform(50.0, 100.0, size=5))
    x = inp["xS"].float()
    for f, s in zip(feats, scale):
        x[:, f] *= s
    inp["xS"] = x.to(torch.bfloat16)


@pytest.mark.parametrize("maps_kind", ["near_identity", "spread"])
@pytest.mark.parametrize("folded", [False, True])
def test_fill_hard_inputs_8b_shape(maps_kind, folded):
    case = _hard_case(maps_kind, 84 if maps_kind == "spread" else 85)
    inp = build_inputs(case)
    _big_features(inp, case.d, 86)
    filled, _, _ = oracle.partition(case.N, case.T, case.exact)
    assert run_fill(case, inp, filled, folded=folded) == B.RF_OK
    check_routing(case, inp, filled)
    for l in range(case.n_layers):
        Ko, Vo = oracle_layer(case, inp, l, filled)
        Kg, Vg = gpu_rows(case, inp, l, filled)
        ek, ev = rel_fro(Kg, Ko), rel_fro(Vg, Vo)
        print(f"\n  {maps_kind} {'folded' if folded else 'plain'} layer {l}: K {ek:.2e} V {ev:.2e}",
              flush=True)
        assert ek <= TOL and ev <= TOL


@pytest.mark.parametrize("folded", [False, True])
def test_nan_row_stays_in_its_row(folded):
    case = Case(d=512, n_layers=2, n_kv=2, hd=128, N=700, T=60, exact=np.array([5, 9, 300]),
                page_size=16, seed=87)
    filled, _, _ = oracle.partition(case.N, case.T, case.exact)
    clean = build_inputs(case)
    assert run_fill(case, clean, filled, folded=folded) == B.RF_OK
    dirty = build_inputs(case)
    bad_row = int(filled[200])
    dirty["xS"][bad_row, 17] = float("nan")
    assert run_fill(case, dirty, filled, folded=folded) == B.RF_OK
    others = filled[filled != bad_row]
    for l in range(case.n_layers):
        Kc, Vc = gpu_rows(case, clean, l, others)
        Kd, Vd = gpu_rows(case, dirty, l, others)
        assert np.array_equal(Kc, Kd) and np.array_equal(Vc, Vd), f"layer {l}"
        Kb, Vb = gpu_rows(case, dirty, l, np.array([bad_row]))
        assert np.isnan(Kb).all() and np.isnan(Vb).all()
        # slots of rows that are not filled keep the sentinel
        for key in ("k_pages", "v_pages"):
            a = clean["layers"][l][key].view(torch.int16)
            b = dirty["layers"][l][key].view(torch.int16)
            same = (a == b).flatten(2).all(-1)
            pg, sl = oracle.paged_location(np.array([bad_row]), dirty["table_np"], case.page_size)
            same[int(pg[0]), int(sl[0])] = True
            assert bool(same.all()), f"layer {l} {key}"
