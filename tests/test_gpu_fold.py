"""GPU parity of folded layers, through the C ABI.

ridgefill_fold_maps against the oracle's fold_map on the same bf16/fp32 values:
  P (one bf16 rounding of a product held to ~2^-17) and R = diag(g) R1 (R1: bf16 of the
  rows of an fp64 Cholesky factor of an fp32-accumulated A^T A over their diagonal
  entries, g that diagonal in fp32): relative Frobenius error <= 2e-3 (a bf16 rounding's
  own error is about 1.1e-3 rms; the fold factors A^T A with its diagonal lifted by a
  relative 2^-16, far below that); R's strict lower triangle exactly zero, R1's diagonal
  exactly one;
  c (fp64 accumulation, fp32 result): 1e-6; r (fp64 substitution on the fp32-accumulated
  Gram): 1e-4; kappa within 1e-4 |b|^2.
The fill of folded layers against the oracle's plain fill_rows (the method's own flow),
the same bar as every fill: bit-exact routing on sentinel-filled caches, K and V within
a relative Frobenius error of 5e-3 per layer."""

import numpy as np
import pytest
import torch

import oracle
from ridge_map_kv_amd import binding as B

from fillcase import (Case, bf16_np, build_inputs, check_routing, check_values, fold_layers,
                      fold_raw, fold_views, folded_layer_dicts, make_shape, rel_fro, run_fill, to_bf16)

pytestmark = pytest.mark.gpu


def _case(d, nl, nkv, hd, N, T, ne, ps, seed, **kw):
    g = np.random.default_rng(seed)
    exact = np.sort(g.choice(N - T, size=ne, replace=False)) if ne else np.zeros(0, np.int64)
    return Case(d=d, n_layers=nl, n_kv=nkv, hd=hd, N=N, T=T, exact=exact, page_size=ps,
                seed=seed, **kw)


def _filled(case):
    f, _, _ = oracle.partition(case.N, case.T, case.exact)
    return f


def _oracle_fold(case, inp, l):
    lay = inp["layers"][l]
    # an int8 map stands for q * scale exactly (float64)
    A = lay["A_ref"] if "A_ref" in lay else bf16_np(lay["A"])
    return oracle.fold_map(A, lay["b"].cpu().numpy().astype(np.float64),
                           bf16_np(lay["norm_w"]), bf16_np(lay["W_K"]), bf16_np(lay["W_V"]))


FOLDS = [
    # d, layers, n_kv, hd, seed, options
    (512, 2, 2, 128, 51, {}),
    (768, 1, 4, 64, 52, dict(d_in=512)),        # tall map: kappa > 0
    (256, 1, 2, 64, 53, dict(map_kind="identity")),
    (512, 3, 2, 128, 54, dict(int8=True)),      # int8 maps: codes and row scales
    (768, 2, 4, 64, 55, dict(d_in=512, int8=True)),
]


@pytest.mark.parametrize("d,nl,nkv,hd,seed,opts", FOLDS)
def test_fold_outputs_vs_oracle(d, nl, nkv, hd, seed, opts):
    case = _case(d, nl, nkv, hd, 300, 20, 0, 16, seed, **opts)
    inp = build_inputs(case)
    print(f"\nfold d={d} d_in={case.width} kv={case.kv} {opts}", flush=True)
    bufs, st = fold_layers(case, inp)
    assert st == B.RF_OK
    for l in range(nl):
        P, R, c, r, kappa = fold_views(case, bufs[l])
        Po, co, Ro, ro, ko = _oracle_fold(case, inp, l)
        b = inp["layers"][l]["b"].cpu().numpy().astype(np.float64)
        eP, eR, ec, er = rel_fro(P, Po), rel_fro(R, Ro), rel_fro(c, co), rel_fro(r, ro)
        print(f"  layer {l}: P {eP:.2e} R {eR:.2e} c {ec:.2e} r {er:.2e} kappa {kappa:.3e} "
              f"(oracle {ko:.3e})", flush=True)
        assert eP <= 2e-3 and eR <= 2e-3 and ec <= 1e-6 and er <= 1e-4
        assert np.all(np.tril(R, -1) == 0.0)
        assert np.all(np.diag(fold_raw(case, bufs[l])[1]) == 1.0)   # unit diagonal, exact
        assert abs(kappa - ko) <= 1e-4 * (b @ b)
        if opts.get("map_kind") == "identity":
            # the Cholesky of I (its diagonal lifted by the relative 2^-16) is exact
            _, R1, _, _, g, _ = fold_raw(case, bufs[l])
            assert np.array_equal(R1, np.eye(case.width))
            assert np.all(g == np.float32(np.sqrt(1.0 + 2.0 ** -16)))
            assert kappa == 0.0


FILLS = [
    # d, layers, n_kv, hd, N, T, n_exact, page, seed, options
    (512, 3, 2, 128, 700, 100, 60, 16, 61, {}),
    (512, 3, 2, 128, 700, 100, 60, 16, 68, dict(int8=True, knorm=True)),   # folded int8 maps
    (512, 2, 2, 128, 700, 100, 60, 16, 62, dict(knorm=True, vscale=True)),
    (768, 2, 4, 64, 333, 33, 17, 8, 63, dict(knorm=True)),
    (768, 2, 4, 64, 600, 40, 25, 16, 64, dict(d_in=512, vscale=True)),     # tall map
    (256, 2, 2, 64, 1100, 60, 300, 16, 65, {}),                           # ragged tiles
    (256, 1, 2, 128, 300, 20, 10, 16, 66, dict(map_kind="identity")),
]


@pytest.mark.parametrize("d,nl,nkv,hd,N,T,ne,ps,seed,opts", FILLS)
def test_folded_fill_parity(d, nl, nkv, hd, N, T, ne, ps, seed, opts):
    case = _case(d, nl, nkv, hd, N, T, ne, ps, seed, **opts)
    inp = build_inputs(case)
    f = _filled(case)
    print(f"\nfolded fill d={d} d_in={case.width} hd={hd} rows={f.size} {opts}", flush=True)
    assert run_fill(case, inp, f, folded=True) == B.RF_OK
    check_routing(case, inp, f)
    worst = check_values(case, inp, f)
    print(f"  worst rel {worst:.2e}", flush=True)


def test_folded_and_plain_fills_agree():
    # the two GPU paths on the same inputs: both are within 5e-3 of the oracle, and
    # their difference is of the order of one bf16 rounding
    case = _case(512, 2, 2, 128, 700, 100, 60, 16, 67, knorm=True)
    f = _filled(case)
    a = build_inputs(case)
    b = build_inputs(case)
    assert run_fill(case, a, f) == B.RF_OK
    assert run_fill(case, b, f, folded=True) == B.RF_OK
    for l in range(case.n_layers):
        for key in ("k_pages", "v_pages"):
            x = a["layers"][l][key].float()
            y = b["layers"][l][key].float()
            written = a["layers"][l][key].view(torch.int16) != -1
            assert torch.equal(written, b["layers"][l][key].view(torch.int16) != -1)
            e = float(torch.linalg.norm((x - y)[written]) / torch.linalg.norm(x[written]))
            print(f"layer {l} {key}: plain vs folded {e:.2e}", flush=True)
            assert e <= 5e-3


def test_folded_empty_filled_list_leaves_cache_untouched():
    # T = N: no prefix rows, nothing filled; the folded fill writes no page
    case = _case(256, 2, 2, 64, 40, 40, 0, 4, 74)
    inp = build_inputs(case)
    before = [(l["k_pages"].clone(), l["v_pages"].clone()) for l in inp["layers"]]
    assert run_fill(case, inp, np.zeros(0, np.int32), folded=True) == B.RF_OK
    torch.cuda.synchronize()
    for l, (k, v) in zip(inp["layers"], before):
        assert torch.equal(l["k_pages"].view(torch.int16), k.view(torch.int16))
        assert torch.equal(l["v_pages"].view(torch.int16), v.view(torch.int16))


@pytest.mark.parametrize("int8", [False, True])
def test_fold_group_size_does_not_change_the_buffers(int8):
    # layers folded one at a time and four side by side (one batched Cholesky; int8 maps:
    # GEMM launches of two layers): the per-layer arithmetic is the same, so the folded
    # buffers agree bit for bit
    case = _case(768, 4, 4, 64, 300, 20, 0, 16, 71, d_in=512, int8=int8)
    inp = build_inputs(case)
    one, st1 = fold_layers(case, inp, layers_at_once=1)
    one = [t.clone() for t in one]
    four, st4 = fold_layers(case, inp, layers_at_once=4)
    assert st1 == B.RF_OK and st4 == B.RF_OK
    three, st3 = fold_layers(case, inp, layers_at_once=3)   # groups of 3 and 1
    assert st3 == B.RF_OK
    for l in range(case.n_layers):
        ref = fold_raw(case, one[l])           # the fields; padding between them is unset
        for other, tag in ((four[l], "4"), (three[l], "3")):
            got = fold_raw(case, other)
            for name, x, y in zip(("P", "R1", "c", "r1", "g", "kappa"), ref, got):
                assert np.array_equal(np.asarray(x), np.asarray(y)), \
                    f"layer {l} {name}: 1 vs {tag} at once"


def test_fold_flags_rank_deficient_map_in_a_group():
    # one singular layer among three folded side by side: the status says so
    case = _case(256, 3, 2, 64, 300, 20, 0, 16, 72)
    inp = build_inputs(case)
    A = inp["layers"][1]["A"].clone()
    A[:, 9] = 0
    inp["layers"][1]["A"] = A
    _, st = fold_layers(case, inp)
    assert st == B.RF_E_NOT_SPD


def test_fold_flags_rank_deficient_map():
    # a zero column of A makes A^T A singular: the pivot is exactly 0 and the status says so
    case = _case(256, 1, 2, 64, 300, 20, 0, 16, 68)
    inp = build_inputs(case)
    A = inp["layers"][0]["A"].clone()
    A[:, 5] = 0
    inp["layers"][0]["A"] = A
    _, st = fold_layers(case, inp)
    assert st == B.RF_E_NOT_SPD


def test_folded_argument_errors():
    case = _case(256, 2, 2, 64, 300, 20, 0, 16, 69)
    inp = build_inputs(case)
    fold_layers(case, inp)
    f = _filled(case)
    dev = inp["xS"].device
    shape = make_shape(case)
    idx = torch.from_numpy(f.astype(np.int32)).to(dev)
    ws = torch.empty(B.ridgefill_fill_workspace_bytes(shape, f.size, 2, B.RF_MAPS_FOLDED),
                     dtype=torch.uint8, device=dev)
    lays = folded_layer_dicts(inp)
    mixed = [lays[0], inp["layers"][1]]
    with pytest.raises(RuntimeError, match="folded"):
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, f.size, mixed, inp["table"],
                         case.page_size, inp["num_pages"], ws)
    # the streamed fill needs landing slots: a workspace sized for the resident fill is short
    with pytest.raises(RuntimeError, match="workspace"):
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, f.size, lays, inp["table"],
                         case.page_size, inp["num_pages"], ws, copy_stream=torch.cuda.Stream())
    small = torch.empty(4096, dtype=torch.uint8, device=dev)
    with pytest.raises(RuntimeError, match="workspace"):
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, f.size, lays, inp["table"],
                         case.page_size, inp["num_pages"], small)
    int8 = dict(inp["layers"][0])
    int8.pop("A")
    int8["A_q"] = torch.zeros((case.d, case.d), dtype=torch.int8, device=dev)
    int8["A_scale"] = torch.ones(case.d, dtype=torch.float32, device=dev)
    # int8 maps take a second operand slot: the bf16 maps' one-layer workspace is short
    fws = torch.empty(B.ridgefill_fold_workspace_bytes(shape), dtype=torch.uint8, device=dev)
    assert B.ridgefill_fold_workspace_bytes_maps(shape, 1, B.RF_MAPS_INT8) > fws.numel()
    with pytest.raises(RuntimeError, match="workspace"):
        B.ridgefill_fold_maps(shape, [int8], [inp["folded"][0]], fws)
    # one map kind per call
    fws = torch.empty(B.ridgefill_fold_workspace_bytes_maps(shape, 2, B.RF_MAPS_INT8),
                      dtype=torch.uint8, device=dev)
    with pytest.raises(RuntimeError, match="int8 maps or none"):
        B.ridgefill_fold_maps(shape, [int8, inp["layers"][1]], inp["folded"], fws)
    both = dict(int8, A=inp["layers"][0]["A"])
    with pytest.raises(RuntimeError, match="exactly one map"):
        B.ridgefill_fold_maps(shape, [both], [inp["folded"][0]], fws)


def test_folded_group_split_is_bit_identical():
    # one launch per layer (a one-layer workspace) against all layers in one launch: the
    # per-layer arithmetic is the same, so the caches agree bit for bit
    case = _case(512, 3, 2, 128, 700, 100, 60, 16, 70, knorm=True, vscale=True)
    f = _filled(case)
    a = build_inputs(case)
    b = build_inputs(case)
    assert run_fill(case, a, f, folded=True) == B.RF_OK
    b["folded"] = a["folded"]
    assert run_fill(case, b, f, folded=True, ws_layers=1) == B.RF_OK
    for l in range(case.n_layers):
        for key in ("k_pages", "v_pages"):
            assert torch.equal(a["layers"][l][key].view(torch.int16),
                               b["layers"][l][key].view(torch.int16)), f"layer {l} {key}"


def test_streamed_folded_layers_bit_identical():
    # folded buffers in page-locked host memory, 5 layers through a workspace that holds 2:
    # groups of 1, 2, 2, so both landing slots are reused; the caches match the resident
    # folded fill bit for bit.  Only R's upper block triangle is copied: with the workspace
    # filled with 0xFF bytes (NaN as bf16 and fp32) beforehand, a read of the rest of a
    # landing slot would show as NaNs
    case = _case(512, 5, 2, 128, 700, 100, 60, 16, 73, knorm=True, vscale=True)
    f = _filled(case)
    a = build_inputs(case)
    b = build_inputs(case)
    assert run_fill(case, a, f, folded=True, ws_byte=0xFF) == B.RF_OK
    b["folded"] = a["folded"]
    assert run_fill(case, b, f, folded=True, streamed=True, ws_layers=2, ws_byte=0xFF) == B.RF_OK
    torch.cuda.synchronize()
    for l in range(case.n_layers):
        for key in ("k_pages", "v_pages"):
            assert torch.equal(a["layers"][l][key].view(torch.int16),
                               b["layers"][l][key].view(torch.int16)), f"layer {l} {key}"
    check_routing(case, b, f)

