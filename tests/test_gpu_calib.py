"""GPU parity of ridgefill_calibrate (one-pass sums and moments) against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from ridge_map_kv_amd import binding as B
from ridge_map_kv_amd import synth

pytestmark = pytest.mark.gpu
TOL = 5e-3


def bf16(a, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(torch.bfloat16)


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


class GpuStats:
    """Reads a calibration state back into float64 arrays (layout of include/ridgefill.h)."""

    def __init__(self, state, d, L):
        raw = state.cpu().numpy()
        self.n = int(raw[:8].view(np.int64)[0])
        self.d_hdr = int(raw[8:12].view(np.int32)[0])
        self.L_hdr = int(raw[12:16].view(np.int32)[0])
        off = 256
        self.s_S = raw[off:off + 8 * d].view(np.float64).copy(); off += 8 * d
        self.s_l = raw[off:off + 8 * d * L].view(np.float64).reshape(L, d).copy(); off += 8 * d * L
        self.G = raw[off:off + 4 * d * d].view(np.float32).reshape(d, d).astype(np.float64); off += 4 * d * d
        self.YX = raw[off:off + 4 * d * d * L].view(np.float32).reshape(L, d, d).astype(np.float64)
        off += 4 * d * d * L
        self.shift = raw[off:off + 4 * d].view(np.float32).astype(np.float64)
        self.shift_fixed = int(raw[24:28].view(np.int32)[0])
        self.bad = int(raw[28:32].view(np.int32)[0])


def run_calib(xS_chunks, xl_chunks, d, L):
    nbytes = B.ridgefill_calib_state_bytes(d, L)
    state = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    B.ridgefill_calib_reset(state, d, L)
    for xs, xl in zip(xS_chunks, xl_chunks):
        B.ridgefill_calibrate(state, d, L, xs, list(xl))
    torch.cuda.synchronize()
    return state


def rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


def test_calib_matches_oracle_ragged_chunks():
    d, L, rows = 512, 3, 1000
    xS, xl = synth.calib_data(d, L, rows, seed=31, noise_scale=0.1, noise_dof=3.0, x_shift=0.25)
    xs_g, xl_g = bf16(xS), [bf16(y) for y in xl]
    cuts = [0, 600, 1000]
    state = run_calib([xs_g[a:b] for a, b in zip(cuts, cuts[1:])],
                      [[y[a:b] for y in xl_g] for a, b in zip(cuts, cuts[1:])], d, L)
    g = GpuStats(state, d, L)
    st = oracle.calib_new(d, L)
    oracle.calib_accumulate(st, f64(xs_g), [f64(y) for y in xl_g])
    assert g.n == rows and g.d_hdr == d and g.L_hdr == L
    low = np.tril(np.ones((d, d), dtype=bool))
    assert rel(g.G[low], st.G[low]) < 1e-5
    assert rel(g.YX, st.YX) < 1e-5
    np.testing.assert_allclose(g.s_S, st.s_S, rtol=1e-5, atol=1e-3)
    np.testing.assert_allclose(g.s_l, st.s_l, rtol=1e-5, atol=1e-3)


def _hadamard(n, d, L, seed):
    H = synth.sylvester_hadamard(n).astype(np.float64)
    X = H[:, 1:d + 1]
    Ys, Ws, cs = [], [], []
    for l in range(L):
        W = synth.sparse_dyadic_matrix(d, d, seed + l).astype(np.float64)
        c = np.random.default_rng(seed + l).integers(-8, 9, size=d) / 4.0
        Ys.append(X @ W.T + c)
        Ws.append(W)
        cs.append(c)
    return X, np.stack(Ys), Ws, cs


def test_calib_hadamard_bit_exact_and_chunk_invariant():
    n, d, L = 2048, 256, 2
    X, Y, _, _ = _hadamard(n, d, L, 40)
    xs_g, yl_g = bf16(X), [bf16(y) for y in Y]
    assert np.array_equal(f64(xs_g), X) and all(np.array_equal(f64(a), b) for a, b in zip(yl_g, Y))
    one = GpuStats(run_calib([xs_g], [yl_g], d, L), d, L)
    cuts = [0, 700, 1700, 2048]
    three = GpuStats(run_calib([xs_g[a:b] for a, b in zip(cuts, cuts[1:])],
                               [[y[a:b] for y in yl_g] for a, b in zip(cuts, cuts[1:])], d, L), d, L)
    st = oracle.calib_new(d, L)
    oracle.calib_accumulate(st, X, list(Y))
    low = np.tril(np.ones((d, d), dtype=bool))
    assert np.array_equal(one.G[low], st.G[low])
    assert np.array_equal(one.YX, st.YX)
    assert np.array_equal(one.s_S, st.s_S) and np.array_equal(one.s_l, st.s_l)
    assert np.array_equal(three.G[low], one.G[low]) and np.array_equal(three.YX, one.YX)
    np.testing.assert_array_equal(one.G[low], (n * np.eye(d))[low])


def test_calib_empty_and_one_row_chunks_bit_exact():
    # chunks of 0, 1, 1, 255 and 1,791 rows: the empty call changes nothing, one-row and
    # ragged chunks fill a partial row tile, and on exactly representable data the sums
    # still equal the oracle's bit for bit
    n, d, L = 2048, 256, 2
    X, Y, _, _ = _hadamard(n, d, L, 41)
    xs_g, yl_g = bf16(X), [bf16(y) for y in Y]
    cuts = [0, 0, 1, 2, 257, n]
    g = GpuStats(run_calib([xs_g[a:b] for a, b in zip(cuts, cuts[1:])],
                           [[y[a:b] for y in yl_g] for a, b in zip(cuts, cuts[1:])], d, L), d, L)
    st = oracle.calib_new(d, L)
    oracle.calib_accumulate(st, X, list(Y))
    low = np.tril(np.ones((d, d), dtype=bool))
    assert g.n == n
    assert np.array_equal(g.G[low], st.G[low])
    assert np.array_equal(g.YX, st.YX)
    assert np.array_equal(g.s_S, st.s_S) and np.array_equal(g.s_l, st.s_l)


def test_calib_short_chunks_every_slice_count_bit_exact():
    # chunks of 64, 128, 192 and 256 rows run the moments loop with 1, 2, 3 and 4 row
    # slices (no loop, the first-and-last slice alone, first then last, and one steady slice
    # between), 65 and 130 rows add a ragged tail to the shortest; on exactly representable
    # data every sum equals the oracle's bit for bit.  The first call (64 rows) fixes the
    # shift: the columns whose 64 values are all equal (the Sylvester columns c with
    # c % 64 == 0, +1 in rows 0..63) are accumulated about that value, the balanced ones
    # (mean 0) about zero; the shifted values, 0 and -2, stay exact.
    n, d, L = 2048, 256, 2
    X, Y, _, _ = _hadamard(n, d, L, 42)
    xs_g, yl_g = bf16(X), [bf16(y) for y in Y]
    cuts = [0, 64, 192, 384, 640, 705, 835, n]
    g = GpuStats(run_calib([xs_g[a:b] for a, b in zip(cuts, cuts[1:])],
                           [[y[a:b] for y in yl_g] for a, b in zip(cuts, cuts[1:])], d, L), d, L)
    want = np.where(np.all(X[:64] == X[0], axis=0), X[0], 0.0)
    assert np.count_nonzero(want) == 4 and g.shift_fixed
    assert np.array_equal(g.shift, want)
    st = oracle.calib_new(d, L)
    oracle.calib_accumulate(st, X - want, list(Y))
    low = np.tril(np.ones((d, d), dtype=bool))
    assert g.n == n
    assert np.array_equal(g.G[low], st.G[low])
    assert np.array_equal(g.YX, st.YX)
    assert np.array_equal(g.s_S, st.s_S) and np.array_equal(g.s_l, st.s_l)


def test_reset_clears_state():
    d, L = 256, 1
    state = torch.full((B.ridgefill_calib_state_bytes(d, L),), 7, dtype=torch.uint8, device="cuda")
    B.ridgefill_calib_reset(state, d, L)
    g = GpuStats(state, d, L)
    assert g.n == 0 and not g.G.any() and not g.YX.any() and not g.s_S.any()
    assert not g.shift.any() and g.shift_fixed == 0 and g.bad == 0


def test_calib_argument_errors():
    d, L = 256, 2
    state = torch.empty(B.ridgefill_calib_state_bytes(d, L), dtype=torch.uint8, device="cuda")
    with pytest.raises(B.RidgeFillError) as e:
        B.ridgefill_calib_reset(state[:1024], d, L)
    assert e.value.status == B.RF_E_WORKSPACE
    with pytest.raises(B.RidgeFillError) as e:
        B.ridgefill_calib_reset(state, 300, L)
    assert e.value.status == B.RF_E_SHAPE
