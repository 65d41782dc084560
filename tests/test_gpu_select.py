"""GPU parity of exact-row selection from scores (ridgefill_select_rows) against the
oracle's select_exact: bit-exact masks and filled-row lists, on seeded scores with many
ties, at the workloads' prefix sizes and at the edge cases (k = 0, k = P, P = 1, all scores
equal, signed zeros, negative scores); and selection feeding the fill."""

import numpy as np
import pytest
import torch

import oracle
from ridge_map_kv_amd import binding as B
from ridge_map_kv_amd import synth

pytestmark = pytest.mark.gpu


def _gpu_select(scores_np, k):
    dev = torch.device("cuda")
    P = scores_np.size
    sc = torch.from_numpy(np.ascontiguousarray(scores_np, dtype=np.float32)).to(dev)
    ws = torch.empty(B.ridgefill_select_workspace_bytes(P), dtype=torch.uint8, device=dev)
    mask = torch.full((max(P, 1),), 7, dtype=torch.uint8, device=dev)
    filled = torch.full((max(P - k, 1),), -5, dtype=torch.int32, device=dev)
    B.ridgefill_select_rows(sc, k, filled, ws, exact_mask=mask)
    st = B.ridgefill_read_status(ws)
    return st, mask[:P].cpu().numpy(), filled[:P - k].cpu().numpy(), filled


def _check(scores_np, k):
    st, mask, filled, _ = _gpu_select(scores_np, k)
    assert st == B.RF_OK
    ex = oracle.select_exact(scores_np.astype(np.float64), k)
    want_mask = np.zeros(scores_np.size, dtype=np.uint8)
    want_mask[ex] = 1
    assert np.array_equal(mask, want_mask)
    want_filled, _, _ = oracle.partition(scores_np.size, 0, ex)
    assert np.array_equal(filled, want_filled.astype(np.int32))


@pytest.mark.parametrize("P,frac,seed", [(28672, 0.1, 1), (61440, 0.05, 2), (12288, 0.1, 3),
                                         (1000, 0.5, 4), (1025, 0.1, 5), (7, 0.3, 6)])
def test_select_matches_oracle(P, frac, seed):
    sc = synth.row_scores(P, seed)
    _check(sc, int(round(frac * P)))


@pytest.mark.parametrize("k", [0, 1, 299, 300])
def test_select_edges(k):
    sc = synth.row_scores(300, 7)
    _check(sc, k)


def test_select_all_equal_takes_lowest_rows():
    sc = np.full(5000, 0.25, dtype=np.float32)
    st, mask, filled, _ = _gpu_select(sc, 123)
    assert st == B.RF_OK
    assert mask[:123].all() and not mask[123:].any()
    assert np.array_equal(filled, np.arange(123, 5000, dtype=np.int32))


def test_select_signed_zero_and_negative():
    g = np.random.default_rng(8)
    sc = g.choice(np.array([-2.5, -0.0, 0.0, 1e-30, -1e-30, 3.0], dtype=np.float32), size=4096)
    for k in (1, 500, 2048, 4000):
        _check(sc, k)


def test_select_single_row():
    _check(np.array([1.5], dtype=np.float32), 0)
    _check(np.array([1.5], dtype=np.float32), 1)


def test_select_nan_flagged():
    sc = synth.row_scores(100, 9)
    sc[17] = np.nan
    st, mask, filled, _ = _gpu_select(sc, 10)
    assert st == B.RF_E_INVALID
    assert mask[17] == 0                                 # a NaN ranks lowest


def test_select_argument_errors():
    dev = torch.device("cuda")
    sc = torch.zeros(10, device=dev)
    ws = torch.empty(B.ridgefill_select_workspace_bytes(10), dtype=torch.uint8, device=dev)
    out = torch.empty(10, dtype=torch.int32, device=dev)
    with pytest.raises(B.RidgeFillError) as e:
        B.ridgefill_select_rows(sc, 11, out, ws)
    assert e.value.status == B.RF_E_SHAPE
    with pytest.raises(B.RidgeFillError) as e:
        B.ridgefill_select_rows(sc, 3, out, ws[:64])
    assert e.value.status == B.RF_E_WORKSPACE


def test_selection_feeds_the_fill():
    # the device-selected filled rows drive the fill directly; the result equals a fill
    # over the oracle-selected rows
    from fillcase import Case, build_inputs, check_routing, check_values
    N, T = 900, 100
    P = N - T
    sc = synth.row_scores(P, 10)
    k = int(round(0.1 * P))
    ex = oracle.select_exact(sc.astype(np.float64), k)
    case = Case(d=512, n_layers=2, n_kv=2, hd=128, N=N, T=T, exact=ex, page_size=16, seed=60)
    inp = build_inputs(case)
    _, _, _, filled_dev = _gpu_select(sc, k)
    shape = B.make_shape(512, 2, 128)
    ws = torch.empty(B.ridgefill_fill_workspace_bytes(shape, P - k, 2), dtype=torch.uint8,
                     device="cuda")
    B.ridgefill_fill(shape, inp["xS"], N, T, filled_dev, P - k, inp["layers"], inp["table"], 16,
                     inp["num_pages"], ws)
    assert B.ridgefill_read_status(ws) == B.RF_OK
    f, _, _ = oracle.partition(N, T, ex)
    check_routing(case, inp, f)
    check_values(case, inp, f)
