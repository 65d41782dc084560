"""GPU parity of the fill's variants against the oracle, through the C ABI: per-head key
norm, value-rescale factors (computed and applied), rectangular maps (d_in != d), int8
maps, and maps streamed from host memory (bit-identical to the resident fill).

Routing is checked bit-exactly on sentinel-filled caches; K and V against the float64
oracle on the same inputs to a relative Frobenius error of 5e-3 per layer.  Value-rescale
factors: relative error 2e-3 per factor (the norms come from one bf16 rounding of the
normalised input and fp32 projections; 2e-3 is about twice the rounding's 2^-9 bound)."""

import numpy as np
import pytest
import torch

import oracle
from ridge_map_kv_amd import binding as B
from ridge_map_kv_amd import synth

from fillcase import (Case, bf16_np, build_inputs, check_routing, check_values, fold_layers,
                      host_maps, make_shape, run_fill, to_bf16)

pytestmark = pytest.mark.gpu


def _case(d, nl, nkv, hd, N, T, ne, ps, seed, **kw):
    g = np.random.default_rng(seed)
    exact = np.sort(g.choice(N - T, size=ne, replace=False)) if ne else np.zeros(0, np.int64)
    return Case(d=d, n_layers=nl, n_kv=nkv, hd=hd, N=N, T=T, exact=exact, page_size=ps,
                seed=seed, **kw)


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _filled(case):
    f, _, _ = oracle.partition(case.N, case.T, case.exact)
    return f


def _run_and_check(case, **kw):
    inp = build_inputs(case)
    f = _filled(case)
    print(f"\ncase d={case.d} d_in={case.width} hd={case.hd} rows={f.size} knorm={case.knorm} "
          f"vscale={case.vscale} int8={case.int8} {kw}", flush=True)
    assert run_fill(case, inp, f, **kw) == B.RF_OK
    check_routing(case, inp, f)
    worst = check_values(case, inp, f)
    print(f"  worst rel {worst:.2e}", flush=True)
    return inp, f


VARIANTS = [
    # d, layers, n_kv, hd, N, T, n_exact, page, seed, options
    (512, 2, 2, 128, 700, 100, 60, 16, 31, dict(knorm=True)),
    (768, 2, 4, 64, 333, 33, 17, 8, 32, dict(knorm=True)),
    (512, 2, 2, 128, 700, 100, 60, 16, 33, dict(vscale=True)),
    (768, 2, 4, 64, 333, 33, 17, 8, 34, dict(vscale=True, knorm=True)),
    (256, 2, 2, 64, 600, 80, 40, 16, 35, dict(d_in=1024)),
    (512, 2, 8, 128, 300, 0, 0, 16, 36, dict(d_in=320)),              # d_in not a tile multiple
    (512, 3, 2, 128, 700, 100, 60, 16, 37, dict(int8=True)),
    (256, 2, 2, 128, 520, 8, 5, 16, 38, dict(int8=True, d_in=1024, knorm=True, vscale=True)),
]


@pytest.mark.parametrize("d,nl,nkv,hd,N,T,ne,ps,seed,opts", VARIANTS)
def test_variant_parity(d, nl, nkv, hd, N, T, ne, ps, seed, opts):
    _run_and_check(_case(d, nl, nkv, hd, N, T, ne, ps, seed, **opts))


def test_rectangular_identity_block_copies_x():
    # A = [I | 0], b = 0: x_hat is the first d features of x_S exactly, so the fill equals
    # the identity fill of those features
    case = _case(256, 1, 2, 128, 300, 20, 10, 16, 39, d_in=512, map_kind="identity")
    inp, f = _run_and_check(case)
    sq = Case(d=256, n_layers=1, n_kv=2, hd=128, N=300, T=20, exact=case.exact, page_size=16,
              seed=39, map_kind="identity")
    inp2 = build_inputs(sq)
    inp2["xS"] = inp["xS"][:, :256].contiguous()
    for k in ("norm_w", "W_K", "W_V", "b"):
        inp2["layers"][0][k] = inp["layers"][0][k]
    assert run_fill(sq, inp2, f) == B.RF_OK
    assert _same_bits(inp2["layers"][0]["k_pages"], inp["layers"][0]["k_pages"])
    assert _same_bits(inp2["layers"][0]["v_pages"], inp["layers"][0]["v_pages"])


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("nl,ws_layers", [(5, 2), (9, 3)])
def test_streamed_maps_bit_identical(int8, nl, ws_layers):
    # group sizes ramp up to what the workspace holds: 5 layers through 2 run as groups of
    # 1, 2, 2 and 9 through 3 as 1, 2, 3, 3, so landing slots are reused, also by groups of
    # another size than the one that used them before
    case = _case(512, nl, 2, 128, 700, 100, 60, 16, 40, int8=int8)
    inp = build_inputs(case)
    f = _filled(case)
    assert run_fill(case, inp, f) == B.RF_OK
    ref = [(l["k_pages"].clone(), l["v_pages"].clone()) for l in inp["layers"]]
    for l in inp["layers"]:
        l["k_pages"].view(torch.int16).fill_(-1)
        l["v_pages"].view(torch.int16).fill_(-1)
    assert run_fill(case, inp, f, ws_layers=ws_layers, streamed=True) == B.RF_OK
    torch.cuda.synchronize()
    for (k, v), l in zip(ref, inp["layers"]):
        assert _same_bits(k, l["k_pages"]) and _same_bits(v, l["v_pages"])
    check_routing(case, inp, f)


def test_streamed_calls_back_to_back_on_one_workspace():
    # two streamed fills enqueued without a sync between them, sharing the workspace and
    # the streams, each into its own page pools: the second call's copies must not
    # overwrite landing slots that the first call's last groups still read
    case = _case(512, 5, 2, 128, 700, 100, 60, 16, 42)
    inp = build_inputs(case)
    f = _filled(case)
    assert run_fill(case, inp, f) == B.RF_OK
    ref = [(l["k_pages"].clone(), l["v_pages"].clone()) for l in inp["layers"]]
    shape = make_shape(case)
    idx = torch.from_numpy(np.asarray(f, dtype=np.int32)).to(inp["xS"].device)
    ws = torch.empty(B.ridgefill_fill_workspace_bytes(shape, f.size, 2, B.RF_MAPS_STREAMED),
                     dtype=torch.uint8, device=inp["xS"].device)
    copy = torch.cuda.Stream()
    calls = []
    for _ in range(2):
        layers = host_maps(inp["layers"])
        for l in layers:
            l["k_pages"] = torch.full_like(l["k_pages"], -1, dtype=torch.int16).view(torch.bfloat16)
            l["v_pages"] = torch.full_like(l["v_pages"], -1, dtype=torch.int16).view(torch.bfloat16)
        calls.append(layers)
    torch.cuda.synchronize()
    for layers in calls:
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, f.size, layers, inp["table"],
                         case.page_size, inp["num_pages"], ws, copy_stream=copy)
    assert B.ridgefill_read_status(ws) == B.RF_OK
    torch.cuda.synchronize()
    for layers in calls:
        for (k, v), l in zip(ref, layers):
            assert _same_bits(k, l["k_pages"]) and _same_bits(v, l["v_pages"])


def test_group_split_bit_identical_with_variants():
    # one layer per launch vs all layers in one launch: same bytes
    case = _case(512, 3, 2, 128, 700, 100, 60, 16, 41, knorm=True, vscale=True, int8=True)
    inp = build_inputs(case)
    f = _filled(case)
    assert run_fill(case, inp, f) == B.RF_OK
    ref = [(l["k_pages"].clone(), l["v_pages"].clone()) for l in inp["layers"]]
    assert run_fill(case, inp, f, ws_layers=1) == B.RF_OK
    for (k, v), l in zip(ref, inp["layers"]):
        assert _same_bits(k, l["k_pages"]) and _same_bits(v, l["v_pages"])


def _vs_inputs(case, c, dev="cuda"):
    inp = build_inputs(case)
    xS_tail = to_bf16(synth.x_split((c, case.width), seed=case.seed + 1000), dev)
    xt = bf16_np(xS_tail).astype(np.float32)
    if case.width >= case.d:
        xin = xt[:, :case.d]
    else:                        # a tall map: the exact inputs are d wide, x_S narrower
        xin = np.concatenate([xt, np.zeros((c, case.d - case.width), np.float32)], axis=1)
    exact = [to_bf16(synth.exact_tail_inputs(xin, case.d, case.seed, l), dev)
             for l in range(case.n_layers)]
    return inp, xS_tail, exact


def _gpu_factors(case, inp, xS_tail, exact):
    shape = make_shape(case)
    c = xS_tail.shape[0]
    ws = torch.empty(B.ridgefill_value_scale_workspace_bytes(shape, c, case.n_layers,
                                                             case.map_flags),
                     dtype=torch.uint8, device="cuda")
    out = torch.full((case.n_layers, case.n_kv), float("nan"), device="cuda")
    B.ridgefill_value_scale(shape, xS_tail, exact, inp["layers"], out, ws)
    assert B.ridgefill_read_status(ws) == B.RF_OK
    return out


def _oracle_factors(case, inp, xS_tail, exact):
    res = []
    for l, lay in enumerate(inp["layers"]):
        A = lay["A_ref"] if "A_ref" in lay else bf16_np(lay["A"])
        res.append(oracle.value_scale(bf16_np(xS_tail), bf16_np(exact[l]), A,
                                      lay["b"].cpu().numpy().astype(np.float64),
                                      bf16_np(lay["norm_w"]), bf16_np(lay["W_V"]),
                                      eps=case.eps, n_kv=case.n_kv, hd=case.hd))
    return np.stack(res)


VS = [
    # d, layers, n_kv, hd, c, seed, options
    (512, 3, 2, 128, 300, 51, {}),
    (768, 2, 4, 64, 512, 52, {}),
    (256, 2, 2, 128, 77, 53, dict(int8=True)),
    (256, 2, 2, 64, 256, 54, dict(d_in=1024)),
]


@pytest.mark.parametrize("d,nl,nkv,hd,c,seed,opts", VS)
def test_value_scale_factors_parity(d, nl, nkv, hd, c, seed, opts):
    case = _case(d, nl, nkv, hd, 600, 64, 0, 16, seed, **opts)
    inp, xS_tail, exact = _vs_inputs(case, c)
    got = _gpu_factors(case, inp, xS_tail, exact).cpu().numpy().astype(np.float64)
    want = _oracle_factors(case, inp, xS_tail, exact)
    print(f"\nfactors {got.ravel()[:4]} ... max rel {np.max(np.abs(got / want - 1)):.2e}", flush=True)
    np.testing.assert_allclose(got, want, rtol=2e-3)


VS_FOLDED = [
    # d, layers, n_kv, hd, c, seed, options
    (512, 3, 2, 128, 300, 58, {}),
    (768, 2, 4, 64, 512, 59, dict(d_in=512)),        # tall map
    (256, 2, 2, 128, 77, 60, {}),                    # c short of one tile
]


@pytest.mark.parametrize("d,nl,nkv,hd,c,seed,opts", VS_FOLDED)
def test_value_scale_factors_folded_layers(d, nl, nkv, hd, c, seed, opts):
    # folded layers: the predicted values from P, c, R, r, kappa, the exact ones from the
    # layer's own W_V and norm weight; against the oracle (plain fields) and the plain GPU path
    case = _case(d, nl, nkv, hd, 600, 64, 0, 16, seed, **opts)
    inp, xS_tail, exact = _vs_inputs(case, c)
    plain = _gpu_factors(case, inp, xS_tail, exact).cpu().numpy().astype(np.float64)
    bufs, st = fold_layers(case, inp)
    assert st == B.RF_OK
    layers = [dict(folded=bufs[l], norm_w=lay["norm_w"], W_V=lay["W_V"])
              for l, lay in enumerate(inp["layers"])]
    shape = make_shape(case)
    ws = torch.empty(B.ridgefill_value_scale_workspace_bytes(shape, c, nl, B.RF_MAPS_FOLDED),
                     dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    out = torch.full((nl, nkv), float("nan"), device="cuda")
    B.ridgefill_value_scale(shape, xS_tail, exact, layers, out, ws)
    assert B.ridgefill_read_status(ws) == B.RF_OK
    got = out.cpu().numpy().astype(np.float64)
    want = _oracle_factors(case, inp, xS_tail, exact)
    print(f"\nfolded factors max rel {np.max(np.abs(got / want - 1)):.2e} "
          f"(plain path {np.max(np.abs(plain / want - 1)):.2e})", flush=True)
    np.testing.assert_allclose(got, want, rtol=2e-3)
    np.testing.assert_allclose(got, plain, rtol=3e-3)


@pytest.mark.parametrize("folded", [False, True])
def test_value_scale_many_layers_and_uneven_groups(folded):
    # 40 layers in one group, more than the kernel arguments hold (the layer pointers then
    # come from a table in the workspace), against the oracle; then through a workspace that
    # holds 3 layers (groups of 3, the last of 1, whose exact-row blocks and norms sit at
    # other offsets), which must give the same bits; W_K is not passed (it is not read)
    nl, c = 40, 300
    case = _case(256, nl, 2, 128, 600, 64, 0, 16, 62)
    inp, xS_tail, exact = _vs_inputs(case, c)
    shape = make_shape(case)
    flags = 0
    layers = [{k: v for k, v in lay.items() if k != "W_K"} for lay in inp["layers"]]
    if folded:
        bufs, st = fold_layers(case, inp)
        assert st == B.RF_OK
        layers = [dict(folded=bufs[l], norm_w=lay["norm_w"], W_V=lay["W_V"])
                  for l, lay in enumerate(inp["layers"])]
        flags = B.RF_MAPS_FOLDED
    outs = []
    for ws_layers in (nl, 3):
        ws = torch.empty(B.ridgefill_value_scale_workspace_bytes(shape, c, ws_layers, flags),
                         dtype=torch.uint8, device="cuda")
        ws.fill_(0xFF)
        out = torch.full((nl, case.n_kv), float("nan"), device="cuda")
        B.ridgefill_value_scale(shape, xS_tail, exact, layers, out, ws)
        assert B.ridgefill_read_status(ws) == B.RF_OK
        outs.append(out.cpu())
    assert torch.equal(outs[0], outs[1])
    got = outs[0].numpy().astype(np.float64)
    want = _oracle_factors(case, inp, xS_tail, exact)
    print(f"\n{nl} layers {'folded' if folded else 'plain'}: max rel "
          f"{np.max(np.abs(got / want - 1)):.2e}", flush=True)
    np.testing.assert_allclose(got, want, rtol=2e-3)


def test_value_scale_folded_argument_errors():
    case = _case(256, 2, 2, 128, 600, 64, 0, 16, 61)
    inp, xS_tail, exact = _vs_inputs(case, 100)
    bufs, _ = fold_layers(case, inp)
    shape = make_shape(case)
    ws = torch.empty(B.ridgefill_value_scale_workspace_bytes(shape, 100, 2, B.RF_MAPS_FOLDED),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((2, case.n_kv), device="cuda")
    no_wv = [dict(folded=bufs[l], norm_w=lay["norm_w"]) for l, lay in enumerate(inp["layers"])]
    with pytest.raises(RuntimeError, match="W_V"):
        B.ridgefill_value_scale(shape, xS_tail, exact, no_wv, out, ws)
    mixed = [dict(folded=bufs[0], norm_w=inp["layers"][0]["norm_w"], W_V=inp["layers"][0]["W_V"]),
             inp["layers"][1]]
    with pytest.raises(RuntimeError, match="folded"):
        B.ridgefill_value_scale(shape, xS_tail, exact, mixed, out, ws)
    assert B.ridgefill_value_scale_workspace_bytes(shape, 100, 2,
                                                   B.RF_MAPS_FOLDED | B.RF_MAPS_INT8) == 0


def test_value_scale_is_one_when_exact_rows_equal_prediction():
    case = _case(512, 2, 2, 128, 600, 64, 0, 16, 55)
    inp, xS_tail, _ = _vs_inputs(case, 200)
    xs = bf16_np(xS_tail)
    exact = []
    for lay in inp["layers"]:
        pred = oracle.predict_input(xs, bf16_np(lay["A"]), lay["b"].cpu().numpy())
        exact.append(to_bf16(pred, "cuda"))
    got = _gpu_factors(case, inp, xS_tail, exact).cpu().numpy()
    np.testing.assert_allclose(got, 1.0, rtol=3e-3)


def test_value_scale_then_fill_end_to_end():
    # factors from the GPU feed the fill; the reference uses the oracle's factors
    case = _case(512, 2, 2, 128, 700, 100, 60, 16, 56)
    inp, xS_tail, exact = _vs_inputs(case, 256)
    out = _gpu_factors(case, inp, xS_tail, exact)
    want = _oracle_factors(case, inp, xS_tail, exact)
    for l, lay in enumerate(inp["layers"]):
        lay["v_scale"] = out[l].contiguous()
    f = _filled(case)
    assert run_fill(case, inp, f) == B.RF_OK
    check_routing(case, inp, f)
    for l, lay in enumerate(inp["layers"]):
        lay["v_scale"] = torch.from_numpy(want[l].astype(np.float32)).cuda()
    check_values(case, inp, f)


def test_variant_argument_errors():
    case = _case(256, 2, 2, 128, 300, 20, 0, 16, 57, int8=True)
    inp = build_inputs(case)
    f = _filled(case)
    shape = make_shape(case)
    idx = torch.from_numpy(f.astype(np.int32)).cuda()
    # int8 maps are read as codes by the map GEMM: they need no more workspace than bf16 maps
    assert B.ridgefill_fill_workspace_bytes(shape, f.size, 2, B.RF_MAPS_INT8) == \
        B.ridgefill_fill_workspace_bytes(shape, f.size, 2)
    # a workspace short of one layer's block is refused before anything is enqueued
    ws_small = torch.empty(B.ridgefill_fill_workspace_bytes(shape, f.size, 1) - 256,
                           dtype=torch.uint8, device="cuda")
    with pytest.raises(B.RidgeFillError) as e:
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, f.size, inp["layers"],
                         inp["table"], 16, inp["num_pages"], ws_small)
    assert e.value.status == B.RF_E_WORKSPACE
    ws = torch.empty(B.ridgefill_fill_workspace_bytes(shape, f.size, 2, B.RF_MAPS_INT8),
                     dtype=torch.uint8, device="cuda")
    mixed = [dict(inp["layers"][0]), dict(inp["layers"][1])]
    mixed[1]["A"] = torch.zeros((256, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.RidgeFillError) as e:     # both A and A_q on one layer
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, f.size, mixed, inp["table"], 16,
                         inp["num_pages"], ws)
    assert e.value.status == B.RF_E_INVALID
    kn = [dict(inp["layers"][0]), dict(inp["layers"][1])]
    kn[0]["k_norm_w"] = torch.ones(128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.RidgeFillError) as e:     # key norm on one layer only
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, f.size, kn, inp["table"], 16,
                         inp["num_pages"], ws)
    assert e.value.status == B.RF_E_INVALID
    bad = B.make_shape(256, 2, 128, d_in=100)
    with pytest.raises(B.RidgeFillError) as e:
        B.ridgefill_fill(bad, inp["xS"], case.N, case.T, idx, f.size, inp["layers"], inp["table"],
                         16, inp["num_pages"], ws)
    assert e.value.status == B.RF_E_SHAPE


@pytest.mark.parametrize("rows,cols,seed", [(256, 4096, 61), (37, 1000, 62), (5120, 5120, 63)])
def test_quantize_map_bit_exact(rows, cols, seed):
    # integer codes decided in fp32 on both sides: bit-exact codes and scales
    g = np.random.default_rng(seed)
    A = (g.standard_normal((rows, cols)) * np.exp(0.5 * g.standard_normal((rows, 1)))).astype(np.float32)
    A[rows // 2] = 0.0
    A[0, :8] = [0.5, -0.5, 1.5, -2.5, 127.0, 0.0, -0.0, 3.0]     # half-way cases for row 0
    q, sc = oracle.quantize_map_int8(A, np.float32)
    At = torch.from_numpy(A).cuda()
    qg = torch.empty((rows, cols), dtype=torch.int8, device="cuda")
    sg = torch.empty(rows, dtype=torch.float32, device="cuda")
    B.ridgefill_quantize_map(At, qg, sg)
    assert np.array_equal(qg.cpu().numpy(), q)
    assert np.array_equal(sg.cpu().numpy().view(np.uint32), sc.astype(np.float32).view(np.uint32))
