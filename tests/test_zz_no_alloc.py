"""ridgefill_fill_noalloc (the fill on the library's fixed device scratch, for callers that
cannot allocate) against ridgefill_fill with a workspace, through the C ABI: the K and V
pools must be bit-identical (the per-layer arithmetic does not depend on how many layers
share a launch), on two calls in a row whose second input is smaller, for plain, int8 and
folded layers, and at the 8B shape (25,805 filled rows, 20 folded layers: the scratch then
holds a few layers per launch).  A call whose single layer needs more than the scratch is
refused before anything is enqueued; device status goes to the caller's word."""

import numpy as np
import pytest
import torch

import oracle
from ridge_map_kv_amd import binding as B
from ridge_map_kv_amd import configs, synth

from fillcase import Case, build_inputs, fold_layers, folded_layer_dicts, make_shape, run_fill

pytestmark = pytest.mark.gpu


def _noalloc(case, inp, filled, folded=False):
    shape = make_shape(case)
    idx = torch.from_numpy(np.asarray(filled, dtype=np.int32)).to(inp["xS"].device)
    status = torch.full((1,), -1, dtype=torch.int32, device=inp["xS"].device)
    layers = folded_layer_dicts(inp) if folded else inp["layers"]
    B.ridgefill_fill_noalloc(shape, inp["xS"], case.N, case.T, idx, int(filled.size), layers,
                             inp["table"], case.page_size, inp["num_pages"], status)
    return B.ridgefill_read_status(status)


def _same_pools(a, b):
    for la, lb in zip(a["layers"], b["layers"]):
        for key in ("k_pages", "v_pages"):
            assert torch.equal(la[key].view(torch.int16), lb[key].view(torch.int16)), key


def _case(seed, N, T, ne, n_layers=3, **kw):
    g = np.random.default_rng(seed)
    exact = np.sort(g.choice(N - T, size=ne, replace=False))
    return Case(d=512, n_layers=n_layers, n_kv=2, hd=128, N=N, T=T, exact=exact, page_size=16,
                seed=seed, **kw)


@pytest.mark.parametrize("kind", ["plain", "int8", "folded"])
def test_noalloc_matches_fill_twice_second_smaller(kind):
    folded = kind == "folded"
    for case in (_case(91, 1400, 80, 70, int8=kind == "int8"),
                 _case(92, 600, 40, 11, n_layers=2, int8=kind == "int8")):
        filled, _, _ = oracle.partition(case.N, case.T, case.exact)
        ref = build_inputs(case)
        got = build_inputs(case)
        if folded:
            assert fold_layers(case, ref)[1] == B.RF_OK
            got["folded"] = [t.clone() for t in ref["folded"]]
        assert run_fill(case, ref, filled, folded=folded) == B.RF_OK
        assert _noalloc(case, got, filled, folded=folded) == B.RF_OK
        _same_pools(ref, got)


def test_noalloc_8b_folded_full_size():
    cfg = configs.LLAMA8B
    dev = torch.device("cuda")
    print("\nnoalloc 8B: inputs", flush=True)
    ref = synth.device_fill_inputs(cfg, dev, sentinel=True)
    shape = B.make_shape(cfg.d, cfg.n_kv, cfg.head_dim, cfg.rms_eps, cfg.rope_theta)
    fws = torch.empty(B.ridgefill_fold_workspace_bytes_ex(shape, cfg.n_upper), dtype=torch.uint8,
                      device=dev)
    bufs = [torch.empty(B.ridgefill_fold_bytes(shape), dtype=torch.uint8, device=dev)
            for _ in ref["layers"]]
    B.ridgefill_fold_maps(shape, ref["layers"], bufs, fws)
    assert B.ridgefill_read_status(fws) == B.RF_OK
    del fws
    filled = B.ridgefill_partition(cfg.N, cfg.T, ref["exact_mask"])
    idx = torch.from_numpy(filled).to(dev)
    one_layer = B.ridgefill_fill_workspace_bytes(shape, filled.size, 1, B.RF_MAPS_FOLDED)
    assert 2 * one_layer < B.RIDGEFILL_NOALLOC_SCRATCH_BYTES      # several layers per launch
    pools = lambda: [dict(k_pages=lay["k_pages"].clone(), v_pages=lay["v_pages"].clone())
                     for lay in ref["layers"]]
    want, got = pools(), pools()
    ws = torch.empty(B.ridgefill_fill_workspace_bytes(shape, filled.size, cfg.n_upper,
                                                      B.RF_MAPS_FOLDED), dtype=torch.uint8,
                     device=dev)
    B.ridgefill_fill(shape, ref["xS"], cfg.N, cfg.T, idx, filled.size,
                     [dict(folded=b, **p) for b, p in zip(bufs, want)], ref["table"],
                     cfg.page_size, ref["num_pages"], ws)
    assert B.ridgefill_read_status(ws) == B.RF_OK
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    print("noalloc 8B: fill", flush=True)
    B.ridgefill_fill_noalloc(shape, ref["xS"], cfg.N, cfg.T, idx, filled.size,
                             [dict(folded=b, **p) for b, p in zip(bufs, got)], ref["table"],
                             cfg.page_size, ref["num_pages"], status)
    assert B.ridgefill_read_status(status) == B.RF_OK
    for a, b in zip(want, got):
        for key in ("k_pages", "v_pages"):
            assert torch.equal(a[key].view(torch.int16), b[key].view(torch.int16))


def test_noalloc_refuses_a_layer_larger_than_the_scratch_and_reports_rows():
    # plain layers stage x_hat * w per layer: 70,000 rows of d = 512 need 72 MB for one layer
    case = Case(d=512, n_layers=1, n_kv=2, hd=128, N=70100, T=100, exact=np.zeros(0, np.int64),
                page_size=16, seed=93)
    inp = build_inputs(case)
    filled = np.arange(case.N - case.T, dtype=np.int32)
    assert B.ridgefill_fill_workspace_bytes(make_shape(case), filled.size, 1) > \
        B.RIDGEFILL_NOALLOC_SCRATCH_BYTES
    with pytest.raises(B.RidgeFillError) as e:
        _noalloc(case, inp, filled)
    assert e.value.status == B.RF_E_WORKSPACE
    assert bool((inp["layers"][0]["k_pages"].view(torch.int16) == -1).all())   # nothing written
    # a row list that is not increasing: the bad rows are skipped and the caller's word says so
    small = _case(94, 300, 20, 0, n_layers=1)
    inp = build_inputs(small)
    rows = np.array([5, 4, 9, 10], dtype=np.int32)
    assert _noalloc(small, inp, rows) == B.RF_E_ROWS
