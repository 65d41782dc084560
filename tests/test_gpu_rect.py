"""GPU parity of the calibration and solve for maps whose input width differs from their
output width (x_S rows d_in wide, layer inputs d_out wide), against the oracle; a
rectangular Hadamard design with a closed-form answer; and the fitted rectangular maps
driving the fill."""

import numpy as np
import pytest
import torch

import oracle
from ridge_map_kv_amd import binding as B
from ridge_map_kv_amd import synth

from fillcase import Case, bf16_np, build_inputs, check_routing, check_values, run_fill
from test_gpu_calib import bf16, f64, rel

pytestmark = pytest.mark.gpu
TOL = 5e-3


def _read_state(state, d_in, d_out, L):
    raw = state.cpu().numpy()
    hdr = raw[:24].view(np.int32)
    assert int(hdr[2]) == d_out and int(hdr[3]) == L and int(hdr[5]) == d_in
    off = 256
    n = int(raw[:8].view(np.int64)[0])
    sS = raw[off:off + 8 * d_in].view(np.float64); off += 8 * d_in
    sl = raw[off:off + 8 * d_out * L].view(np.float64).reshape(L, d_out); off += 8 * d_out * L
    G = raw[off:off + 4 * d_in * d_in].view(np.float32).reshape(d_in, d_in); off += 4 * d_in * d_in
    YX = raw[off:off + 4 * d_out * d_in * L].view(np.float32).reshape(L, d_out, d_in)
    return n, sS, sl, G.astype(np.float64), YX.astype(np.float64)


def _calib(chunks_S, chunks_l, d_in, d_out, L):
    state = torch.empty(B.ridgefill_calib_state_bytes(d_in, L, d_out), dtype=torch.uint8,
                        device="cuda")
    B.ridgefill_calib_reset(state, d_in, L, d_out=d_out)
    for xs, xl in zip(chunks_S, chunks_l):
        B.ridgefill_calibrate(state, d_in, L, xs, list(xl), d_out=d_out)
    torch.cuda.synchronize()
    return state


def _solve(state, d_in, d_out, L, lam):
    A = torch.empty((L, d_out, d_in), dtype=torch.float32, device="cuda")
    Ab = torch.empty((L, d_out, d_in), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((L, d_out), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.ridgefill_solve_workspace_bytes(d_in, L, d_out), dtype=torch.uint8,
                     device="cuda")
    B.ridgefill_solve(state, d_in, L, lam, A, b, Ab, ws, d_out=d_out)
    assert B.ridgefill_read_status(ws) == B.RF_OK
    return A, b, Ab


def _data(d_in, d_out, L, rows, seed):
    g = np.random.default_rng(seed)
    xS = (g.standard_normal((rows, d_in)) + 0.25).astype(np.float32)
    xl = []
    for l in range(L):
        W = synth.rect_map(d_out, d_in, seed, l)[0]
        c = g.standard_normal(d_out).astype(np.float32)
        xl.append((xS @ W.T + c + 0.1 * g.standard_t(3.0, size=(rows, d_out))).astype(np.float32))
    return xS, xl


@pytest.mark.parametrize("d_in,d_out,rows", [(512, 256, 1000), (256, 768, 650), (768, 512, 3000)])
def test_rect_calibration_and_solve_match_oracle(d_in, d_out, rows):
    L = 2
    xS, xl = _data(d_in, d_out, L, rows, 81)
    xs_g, xl_g = bf16(xS), [bf16(y) for y in xl]
    cut = rows // 3
    state = _calib([xs_g[:cut], xs_g[cut:]], [[y[:cut] for y in xl_g], [y[cut:] for y in xl_g]],
                   d_in, d_out, L)
    n, sS, sl, G, YX = _read_state(state, d_in, d_out, L)
    st = oracle.calib_new(d_in, L, d_out)
    oracle.calib_accumulate(st, f64(xs_g), [f64(y) for y in xl_g])
    assert n == rows
    low = np.tril(np.ones((d_in, d_in), dtype=bool))
    assert rel(G[low], st.G[low]) < 1e-5
    assert rel(YX, st.YX) < 1e-5
    np.testing.assert_allclose(sS, st.s_S, rtol=1e-6, atol=1e-3)
    np.testing.assert_allclose(sl, st.s_l, rtol=1e-6, atol=1e-3)
    for lam in (1e-3, 0.03):
        A, b, Ab = _solve(state, d_in, d_out, L, lam)
        Ao, bo = oracle.solve(st, lam)
        A64, b64 = A.cpu().numpy().astype(np.float64), b.cpu().numpy().astype(np.float64)
        _, _, XtX, YtX = oracle.centred_moments(st)
        alpha = oracle.ridge_alpha(XtX, lam)
        for l in range(L):
            assert rel(A64[l], Ao[l]) < TOL and rel(b64[l], bo[l]) < TOL
            R = (XtX + alpha * np.eye(d_in)) @ A64[l].T - YtX[l].T
            assert np.linalg.norm(R) / np.linalg.norm(YtX[l]) < 1e-4
        assert torch.equal(Ab.cpu(), A.cpu().to(torch.bfloat16))


@pytest.mark.parametrize("d_out", [512, 256])
def test_rect_hadamard_closed_form(d_out):
    # x_S = columns 1..256 of a 2048-row Hadamard matrix plus a mean shift: centred
    # X^T X = n I, so A = W / (1 + lam) and b = c + lam / (1 + lam) W m exactly
    n, d_in, L = 2048, 256, 2
    H = synth.sylvester_hadamard(n).astype(np.float64)
    m = np.random.default_rng(83).integers(-2, 3, size=d_in) / 2.0
    xS = H[:, 1:d_in + 1] + m
    Ws = [synth.sparse_dyadic_matrix(d_out, d_in, 84 + l).astype(np.float64) for l in range(L)]
    cs = [np.random.default_rng(86 + l).integers(-8, 9, size=d_out) / 4.0 for l in range(L)]
    ys = [xS @ W.T + c for W, c in zip(Ws, cs)]
    state = _calib([bf16(xS)], [[bf16(y) for y in ys]], d_in, d_out, L)
    for lam in (1e-4, 0.03, 1.0):
        A, b, _ = _solve(state, d_in, d_out, L, lam)
        for l in range(L):
            np.testing.assert_allclose(A[l].cpu().numpy(), Ws[l] / (1 + lam), atol=1e-5)
            np.testing.assert_allclose(b[l].cpu().numpy(), cs[l] + lam / (1 + lam) * (Ws[l] @ m),
                                       atol=1e-4)


def test_rect_fit_drives_the_fill():
    # calibrate and solve rectangular maps on the GPU, then fill with them; the reference
    # is the oracle's fill with the same bf16 map bytes
    d_in, d_out, L, rows = 512, 256, 2, 2000
    xS, xl = _data(d_in, d_out, L, rows, 88)
    state = _calib([bf16(xS)], [[bf16(y) for y in xl]], d_in, d_out, L)
    A, b, Ab = _solve(state, d_in, d_out, L, 0.03)
    g = np.random.default_rng(89)
    N, T = 700, 100
    exact = np.sort(g.choice(N - T, size=40, replace=False))
    case = Case(d=d_out, n_layers=L, n_kv=2, hd=128, N=N, T=T, exact=exact, page_size=16, seed=89,
                d_in=d_in, map_kind="given",
                maps=[(bf16_np(Ab[l]).astype(np.float32), b[l].cpu().numpy()) for l in range(L)])
    inp = build_inputs(case)
    f, _, _ = oracle.partition(N, T, exact)
    assert run_fill(case, inp, f) == B.RF_OK
    check_routing(case, inp, f)
    check_values(case, inp, f)


def _random_fits(n, seed):
    """Seeded random fits: widths, layer counts, row counts split into uneven chunks (some
    shorter than one 64-row slice) and lambdas across six decades."""
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d_in = int(g.choice([256, 512, 768]))
        d_out = int(g.choice([256, 512, 768]))
        L = int(g.integers(1, 4))
        rows = int(g.integers(2 * d_in, 4 * d_in))
        cuts = np.sort(g.choice(np.arange(1, rows), size=int(g.integers(0, 4)), replace=False))
        lam = float(g.choice([1e-4, 1e-3, 1e-2, 0.03, 0.1, 1.0]))
        out.append((d_in, d_out, L, rows, [int(c) for c in cuts], lam, int(g.integers(1 << 20))))
    return out


@pytest.mark.parametrize("k", range(12))
def test_seeded_random_fits_match_oracle(k):
    d_in, d_out, L, rows, cuts, lam, seed = _random_fits(12, 77)[k]
    print(f"\nfit {k}: d_in={d_in} d_out={d_out} layers={L} rows={rows} cuts={cuts} "
          f"lambda={lam}", flush=True)
    xS, xl = _data(d_in, d_out, L, rows, seed)
    xs_g, xl_g = bf16(xS), [bf16(y) for y in xl]
    edges = [0] + cuts + [rows]
    state = _calib([xs_g[a:b] for a, b in zip(edges, edges[1:])],
                   [[y[a:b] for y in xl_g] for a, b in zip(edges, edges[1:])], d_in, d_out, L)
    n, sS, sl, G, YX = _read_state(state, d_in, d_out, L)
    st = oracle.calib_new(d_in, L, d_out)
    oracle.calib_accumulate(st, f64(xs_g), [f64(y) for y in xl_g])
    assert n == rows
    low = np.tril(np.ones((d_in, d_in), dtype=bool))
    assert rel(G[low], st.G[low]) < 1e-5 and rel(YX, st.YX) < 1e-5
    np.testing.assert_allclose(sS, st.s_S, rtol=1e-6, atol=1e-3)
    np.testing.assert_allclose(sl, st.s_l, rtol=1e-6, atol=1e-3)
    A, b, _ = _solve(state, d_in, d_out, L, lam)
    Ao, bo = oracle.solve(st, lam)
    A, b = A.cpu().numpy().astype(np.float64), b.cpu().numpy().astype(np.float64)
    _, _, XtX, YtX = oracle.centred_moments(st)
    alpha = oracle.ridge_alpha(XtX, lam)
    for l in range(L):
        assert rel(A[l], Ao[l]) < TOL and rel(b[l], bo[l]) < TOL, (l, rel(A[l], Ao[l]))
        R = (XtX + alpha * np.eye(d_in)) @ A[l].T - YtX[l].T
        assert np.linalg.norm(R) / np.linalg.norm(YtX[l]) < 1e-4
