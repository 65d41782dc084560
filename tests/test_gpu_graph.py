"""The fill under HIP graph capture, as a serving loop would run it: the library enqueues
only kernels on the caller's stream (its status word is cleared by a kernel, not a memset),
so a captured fill replays.  Each replay is checked bit for bit against the eager fill,
with the pools reset and other eager work and synchronisations between replays."""

import numpy as np
import pytest
import torch

import oracle
from ridge_map_kv_amd import binding as B

from fillcase import Case, build_inputs, fold_layers, folded_layer_dicts, make_shape

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("folded", [False, True])
def test_captured_fill_replays_bit_identical(folded):
    g = np.random.default_rng(81)
    exact = np.sort(g.choice(600, size=50, replace=False))
    case = Case(d=512, n_layers=3, n_kv=2, hd=128, N=700, T=100, exact=exact, page_size=16,
                seed=81, knorm=True, vscale=True)
    inp = build_inputs(case)
    f, _, _ = oracle.partition(case.N, case.T, case.exact)
    dev = inp["xS"].device
    shape = make_shape(case)
    idx = torch.from_numpy(f.astype(np.int32)).to(dev)
    if folded:
        _, st = fold_layers(case, inp)
        assert st == B.RF_OK
        layers = folded_layer_dicts(inp)
        flags = B.RF_MAPS_FOLDED
    else:
        layers = inp["layers"]
        flags = 0
    ws = torch.empty(B.ridgefill_fill_workspace_bytes(shape, f.size, case.n_layers, flags),
                     dtype=torch.uint8, device=dev)
    pools = [(l["k_pages"], l["v_pages"]) for l in layers]

    def reset():
        for k, v in pools:
            k.view(torch.int16).fill_(-1)
            v.view(torch.int16).fill_(-1)

    def fill():
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, f.size, layers, inp["table"],
                         case.page_size, inp["num_pages"], ws)

    reset()
    fill()
    assert B.ridgefill_read_status(ws) == B.RF_OK
    ref = [(k.clone(), v.clone()) for k, v in pools]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):             # warm the capture stream once
        fill()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        fill()
    torch.cuda.synchronize()

    other = torch.randn(1 << 20, device=dev)
    for rep in range(3):
        reset()
        other.mul_(1.5).add_(0.25)            # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert B.ridgefill_read_status(ws) == B.RF_OK
        for (k, v), (rk, rv) in zip(pools, ref):
            assert torch.equal(k.view(torch.int16), rk.view(torch.int16)), f"replay {rep}: K"
            assert torch.equal(v.view(torch.int16), rv.view(torch.int16)), f"replay {rep}: V"
    del graph
