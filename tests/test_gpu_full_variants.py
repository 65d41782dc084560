"""Parity of the fill's variants at the workloads' full sizes, in the launch configurations
the benchmark times: the 27B-shaped fill with int8 maps streamed from pinned host memory in
4-layer groups, the Qwen3-8B-shaped fill with key norm, the 8B-shaped fill with a split
state twice as wide as the layers, the value-rescale factors over c = 512 tail rows of
the 27B shape, and the folded 8B, 27B (resident, and streamed from pinned host memory in
groups of up to 4 layers) and Qwen3-8B (key norm) fills against the plain oracle.

Fills: routing bit-exact on every byte of every layer's pools (sentinel-filled), K and V
against the oracle on 512 sampled rows of every layer (first and last filled row, rows
next to exact rows, page edges, the rest seeded) and on every filled row of the first
and last upper layer, relative Frobenius error <= 5e-3.
Value-rescale factors: relative error <= 2e-3 on four layers.  The int8 codes come from the
oracle's float32 quantizer; the oracle uses q * scale exactly."""

import numpy as np
import pytest
import torch

import oracle
from ridge_map_kv_amd import binding as B
from ridge_map_kv_amd import configs, synth

from test_gpu_full import _all_rows_layer, _np64, _rel, _sample_rows

pytestmark = pytest.mark.gpu
TOL = 5e-3


def _routing(cfg, inp, filled):
    dev = inp["xS"].device
    pg, sl = oracle.paged_location(filled, inp["table_np"], cfg.page_size)
    expect = torch.zeros((inp["num_pages"], cfg.page_size), dtype=torch.bool, device=dev)
    expect[torch.from_numpy(pg).to(dev), torch.from_numpy(sl).to(dev)] = True
    for l, lay in enumerate(inp["layers"]):
        for key in ("k_pages", "v_pages"):
            sent = lay[key].view(torch.int16) == -1
            assert torch.equal((~sent).flatten(2).all(-1), expect), f"layer {l} {key}: row not fully written"
            assert torch.equal(sent.flatten(2).all(-1), ~expect), f"layer {l} {key}: write outside filled rows"
            del sent
    return pg, sl


def _values(cfg, inp, filled, exact, pg, sl, A_of=None, kn_of=None):
    """Sampled rows of every layer, then every filled row of the first and last layer."""
    n, worst = _values_sampled(cfg, inp, filled, exact, pg, sl, A_of, kn_of)
    for l in (0, len(inp["layers"]) - 1):
        ek, ev = _all_rows_layer(cfg, inp, filled, pg, sl, l, A_of, kn_of)
        print(f"  layer {l}, all {filled.size} filled rows: K {ek:.2e} V {ev:.2e}", flush=True)
        worst = max(worst, ek, ev)
        assert ek <= TOL and ev <= TOL, f"layer {l} all rows: K {ek:.3e} V {ev:.3e}"
    return n, worst


def _values_sampled(cfg, inp, filled, exact, pg, sl, A_of=None, kn_of=None):
    dev = inp["xS"].device
    rows = _sample_rows(filled, exact, cfg.page_size)
    xs = _np64(inp["xS"][torch.from_numpy(rows).to(dev)])
    sel = np.searchsorted(filled, rows)
    rpg = torch.from_numpy(pg[sel]).to(dev)
    rsl = torch.from_numpy(sl[sel]).to(dev)
    worst = 0.0
    for l, lay in enumerate(inp["layers"]):
        A = A_of(l) if A_of else _np64(lay["A"])
        Ko, Vo = oracle.fill_rows(xs, rows, A, lay["b"].cpu().numpy().astype(np.float64),
                                  _np64(lay["norm_w"]), _np64(lay["W_K"]), _np64(lay["W_V"]),
                                  eps=cfg.rms_eps, theta=cfg.rope_theta, n_kv=cfg.n_kv,
                                  hd=cfg.head_dim, k_norm_w=kn_of(l) if kn_of else None)
        ek = _rel(_np64(lay["k_pages"][rpg, rsl]), Ko)
        ev = _rel(_np64(lay["v_pages"][rpg, rsl]), Vo)
        worst = max(worst, ek, ev)
        assert ek <= TOL and ev <= TOL, f"layer {l}: K {ek:.3e} V {ev:.3e}"
    return rows.size, worst


def _run(cfg, inp, flags=0, ws_layers=None, copy=None, layers=None, ws_byte=None):
    dev = inp["xS"].device
    filled = B.ridgefill_partition(cfg.N, cfg.T, inp["exact_mask"])
    shape = B.make_shape(cfg.d, cfg.n_kv, cfg.head_dim, cfg.rms_eps, cfg.rope_theta, d_in=cfg.d_in)
    idx = torch.from_numpy(filled).to(dev)
    ws = torch.empty(B.ridgefill_fill_workspace_bytes(shape, filled.size, ws_layers or cfg.n_upper,
                                                      flags), dtype=torch.uint8, device=dev)
    if ws_byte is not None:             # poison: reads of bytes the call never wrote show up
        ws.fill_(ws_byte)
    B.ridgefill_fill(shape, inp["xS"], cfg.N, cfg.T, idx, filled.size, layers or inp["layers"],
                     inp["table"], cfg.page_size, inp["num_pages"], ws, copy_stream=copy)
    assert B.ridgefill_read_status(ws) == B.RF_OK
    del ws
    return filled


def test_27b_int8_maps_streamed_full_size():
    cfg = configs.QWEN27B
    dev = torch.device("cuda")
    print("\n27B int8 streamed: inputs and oracle quantization", flush=True)
    inp = synth.device_fill_inputs(cfg, dev, sentinel=True)
    codes, host = [], []
    for l, lay in enumerate(inp["layers"]):
        q, sc = oracle.quantize_map_int8(lay["A"].float().cpu().numpy(), np.float32)
        codes.append((q, sc))
        h = dict(lay)
        del h["A"]
        pinned = torch.empty(q.shape, dtype=torch.int8, pin_memory=True)
        pinned.copy_(torch.from_numpy(q))
        h["A_q"] = pinned
        h["A_scale"] = torch.from_numpy(sc.astype(np.float32)).to(dev)
        host.append(h)
        del lay["A"]
        if l % 12 == 11:
            print(f"  quantized {l + 1} maps", flush=True)
    torch.cuda.empty_cache()
    print("27B int8 streamed: fill", flush=True)
    filled = _run(cfg, inp, B.RF_MAPS_INT8 | B.RF_MAPS_STREAMED, ws_layers=4,
                  copy=torch.cuda.Stream(), layers=host)
    _, exact, _ = oracle.partition(cfg.N, cfg.T, synth.exact_rows(cfg))
    print("27B int8 streamed: routing", flush=True)
    pg, sl = _routing(cfg, inp, filled)
    print("27B int8 streamed: values", flush=True)
    n, worst = _values(cfg, inp, filled, exact, pg, sl,
                       A_of=lambda l: oracle.dequantize_map_int8(*codes[l]))
    print(f"27B int8 streamed: {n} rows x {cfg.n_upper} layers, worst rel {worst:.2e}", flush=True)


def test_qwen3_8b_key_norm_full_size():
    cfg = configs.QWEN3_8B
    dev = torch.device("cuda")
    print("\nQwen3-8B key norm: inputs", flush=True)
    inp = synth.device_fill_inputs(cfg, dev, sentinel=True)
    kn = [synth.key_norm_weight(cfg.head_dim, cfg.seed, l) for l in range(cfg.n_upper)]
    for l, lay in enumerate(inp["layers"]):
        lay["k_norm_w"] = torch.from_numpy(kn[l]).to(dev).to(torch.bfloat16)
    filled = _run(cfg, inp)
    _, exact, _ = oracle.partition(cfg.N, cfg.T, synth.exact_rows(cfg))
    pg, sl = _routing(cfg, inp, filled)
    n, worst = _values(cfg, inp, filled, exact, pg, sl,
                       kn_of=lambda l: _np64(inp["layers"][l]["k_norm_w"]))
    print(f"Qwen3-8B key norm: {n} rows x {cfg.n_upper} layers, worst rel {worst:.2e}", flush=True)


def test_wide_split_state_full_size():
    cfg = configs.WIDE8B
    dev = torch.device("cuda")
    print("\nwide split state: inputs", flush=True)
    inp = synth.device_fill_inputs(cfg, dev, sentinel=True)
    filled = _run(cfg, inp)
    _, exact, _ = oracle.partition(cfg.N, cfg.T, synth.exact_rows(cfg))
    pg, sl = _routing(cfg, inp, filled)
    n, worst = _values(cfg, inp, filled, exact, pg, sl)
    print(f"wide split state: {n} rows x {cfg.n_upper} layers, worst rel {worst:.2e}", flush=True)


def test_value_scale_27b_shape():
    cfg = configs.QWEN27B
    dev = torch.device("cuda")
    c = 512
    print("\nvalue scale 27B shape: inputs", flush=True)
    inp = synth.device_fill_inputs(cfg, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(7070)
    xt = torch.randn((c, cfg.d), generator=g, device=dev).to(torch.bfloat16)
    # exact inputs near the prediction: A x + b plus noise of a tenth of its scale
    exact = []
    for lay in inp["layers"]:
        pred = xt.float() @ lay["A"].float().T + lay["b"]
        exact.append((pred + 0.1 * pred.std() * torch.randn(pred.shape, generator=g, device=dev))
                     .to(torch.bfloat16).contiguous())
        del pred
    shape = B.make_shape(cfg.d, cfg.n_kv, cfg.head_dim, cfg.rms_eps, cfg.rope_theta)
    ws = torch.empty(B.ridgefill_value_scale_workspace_bytes(shape, c, cfg.n_upper),
                     dtype=torch.uint8, device=dev)
    out = torch.full((cfg.n_upper, cfg.n_kv), float("nan"), device=dev)
    B.ridgefill_value_scale(shape, xt, exact, inp["layers"], out, ws)
    assert B.ridgefill_read_status(ws) == B.RF_OK
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    print("value scale 27B shape: oracle on 4 layers", flush=True)
    for l in (0, 17, 30, cfg.n_upper - 1):
        lay = inp["layers"][l]
        want = oracle.value_scale(_np64(xt), _np64(exact[l]), _np64(lay["A"]),
                                  lay["b"].cpu().numpy().astype(np.float64), _np64(lay["norm_w"]),
                                  _np64(lay["W_V"]), eps=cfg.rms_eps, n_kv=cfg.n_kv,
                                  hd=cfg.head_dim)
        np.testing.assert_allclose(got[l], want, rtol=2e-3)
        print(f"  layer {l}: max rel {np.max(np.abs(got[l] / want - 1)):.2e}", flush=True)


def test_8b_folded_full_size():
    # the 8B-shaped fill through folded layers (fold once, then the fill), every layer in
    # one launch as the benchmark runs it; the fold of two layers checked against the
    # oracle's fold_map as well
    cfg = configs.LLAMA8B
    dev = torch.device("cuda")
    print("\n8B folded: inputs", flush=True)
    inp = synth.device_fill_inputs(cfg, dev, sentinel=True)
    shape = B.make_shape(cfg.d, cfg.n_kv, cfg.head_dim, cfg.rms_eps, cfg.rope_theta)
    fb = B.ridgefill_fold_bytes(shape)
    fws = torch.empty(B.ridgefill_fold_workspace_bytes_ex(shape, len(inp["layers"])),
                      dtype=torch.uint8, device=dev)
    bufs = [torch.empty(fb, dtype=torch.uint8, device=dev) for _ in inp["layers"]]
    print("8B folded: fold", flush=True)
    B.ridgefill_fold_maps(shape, inp["layers"], bufs, fws)
    assert B.ridgefill_read_status(fws) == B.RF_OK
    del fws
    kv = cfg.n_kv * cfg.head_dim
    a = lambda x: (x + 255) // 256 * 256
    oR = a(2 * kv * cfg.d * 2)
    oc = oR + a(cfg.d * cfg.d * 2)
    for l in (0, cfg.n_upper - 1):
        print(f"8B folded: oracle fold of layer {l}", flush=True)
        lay = inp["layers"][l]
        Po, co, Ro, ro, ko = oracle.fold_map(_np64(lay["A"]), lay["b"].cpu().numpy().astype(np.float64),
                                             _np64(lay["norm_w"]), _np64(lay["W_K"]), _np64(lay["W_V"]))
        buf = bufs[l].cpu()
        og = oc + a(2 * kv * 4) + a(cfg.d * 4)
        P = buf[:2 * kv * cfg.d * 2].view(torch.bfloat16).double().numpy().reshape(2 * kv, cfg.d)
        R1 = buf[oR:oR + cfg.d * cfg.d * 2].view(torch.bfloat16).double().numpy().reshape(cfg.d, cfg.d)
        c = buf[oc:oc + 2 * kv * 4].view(torch.float32).double().numpy()
        g = buf[og:og + cfg.d * 4].view(torch.float32).double().numpy()
        R = R1 * g[:, None]                  # R = diag(g) R1, R1 with a unit diagonal
        eP, eR, ec = _rel(P, Po), _rel(R, Ro), _rel(c, co)
        print(f"  P {eP:.2e} R {eR:.2e} c {ec:.2e}", flush=True)
        assert eP <= 2e-3 and eR <= 2e-3 and ec <= 1e-6 and np.all(np.tril(R, -1) == 0.0)
        assert np.all(np.diag(R1) == 1.0)
    folded = [dict(folded=bufs[l], k_pages=lay["k_pages"], v_pages=lay["v_pages"])
              for l, lay in enumerate(inp["layers"])]
    print("8B folded: fill", flush=True)
    filled = _run(cfg, inp, B.RF_MAPS_FOLDED, layers=folded)
    _, exact, _ = oracle.partition(cfg.N, cfg.T, synth.exact_rows(cfg))
    pg, sl = _routing(cfg, inp, filled)
    n, worst = _values(cfg, inp, filled, exact, pg, sl)
    print(f"8B folded: {n} rows x {cfg.n_upper} layers, worst rel {worst:.2e}", flush=True)


def _folded_full(cfg, knorm=False, streamed=False, int8=False):
    dev = torch.device("cuda")
    print(f"\n{cfg.name} folded: inputs", flush=True)
    inp = synth.device_fill_inputs(cfg, dev, sentinel=True)
    if knorm:
        for l, lay in enumerate(inp["layers"]):
            lay["k_norm_w"] = torch.from_numpy(synth.key_norm_weight(cfg.head_dim, cfg.seed, l)).to(
                dev).to(torch.bfloat16)
    codes = []
    if int8:                           # int8 maps from the oracle's quantizer, folded as codes
        for l, lay in enumerate(inp["layers"]):
            q, sc = oracle.quantize_map_int8(lay["A"].float().cpu().numpy(), np.float32)
            codes.append((q, sc))
            del lay["A"]
            lay["A_q"] = torch.from_numpy(q).to(dev)
            lay["A_scale"] = torch.from_numpy(sc.astype(np.float32)).to(dev)
            if l % 12 == 11:
                print(f"  quantized {l + 1} maps", flush=True)
    shape = B.make_shape(cfg.d, cfg.n_kv, cfg.head_dim, cfg.rms_eps, cfg.rope_theta)
    fws = torch.empty(B.ridgefill_fold_workspace_bytes_maps(shape, len(inp["layers"]),
                                                            B.RF_MAPS_INT8 if int8 else 0),
                      dtype=torch.uint8, device=dev)
    bufs = [torch.empty(B.ridgefill_fold_bytes(shape), dtype=torch.uint8, device=dev)
            for _ in inp["layers"]]
    print(f"{cfg.name} folded: fold of {cfg.n_upper} layers", flush=True)
    B.ridgefill_fold_maps(shape, inp["layers"], bufs, fws)
    assert B.ridgefill_read_status(fws) == B.RF_OK
    del fws
    if streamed:                       # folded buffers to page-locked host memory
        host = []
        for b in bufs:
            h = torch.empty(b.shape, dtype=b.dtype, pin_memory=True)
            h.copy_(b.cpu())
            host.append(h)
        bufs = host
        torch.cuda.empty_cache()
    folded = [dict(folded=bufs[l], k_pages=lay["k_pages"], v_pages=lay["v_pages"],
                   **({"k_norm_w": lay["k_norm_w"]} if knorm else {}))
              for l, lay in enumerate(inp["layers"])]
    print(f"{cfg.name} folded: fill{' streamed from host memory' if streamed else ''}", flush=True)
    if streamed:
        filled = _run(cfg, inp, B.RF_MAPS_FOLDED | B.RF_MAPS_STREAMED, ws_layers=4,
                      copy=torch.cuda.Stream(), layers=folded, ws_byte=0xFF)
    else:
        filled = _run(cfg, inp, B.RF_MAPS_FOLDED, layers=folded)
    _, exact, _ = oracle.partition(cfg.N, cfg.T, synth.exact_rows(cfg))
    pg, sl = _routing(cfg, inp, filled)
    n, worst = _values(cfg, inp, filled, exact, pg, sl,
                       kn_of=(lambda l: _np64(inp["layers"][l]["k_norm_w"])) if knorm else None,
                       A_of=(lambda l: oracle.dequantize_map_int8(*codes[l])) if int8 else None)
    print(f"{cfg.name} folded: {n} rows x {cfg.n_upper} layers, worst rel {worst:.2e}", flush=True)


def test_27b_folded_full_size():
    # 48 folded layers in two 24-layer launches, as the benchmark runs them
    _folded_full(configs.QWEN27B)


def test_qwen3_8b_key_norm_folded_full_size():
    _folded_full(configs.QWEN3_8B, knorm=True)


def test_27b_folded_from_int8_maps_full_size():
    # the 48 maps quantized to int8, folded through their codes, against the oracle's fill
    # with the dequantized maps
    _folded_full(configs.QWEN27B, int8=True)


def test_27b_folded_streamed_full_size():
    # the 48 folded buffers in page-locked host memory, through a workspace of 4 layers
    # (groups of 1, 2, 3, then 4), as the benchmark runs it; only the upper block triangle
    # of each R is copied, and the workspace starts as 0xFF bytes
    _folded_full(configs.QWEN27B, streamed=True)
