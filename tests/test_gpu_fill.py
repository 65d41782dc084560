"""GPU parity of ridgefill_fill against the oracle, through the C ABI.

Routing is checked bit-exactly (sentinel-filled caches: every byte outside the filled rows
of every layer is unchanged); K and V are checked against the float64 oracle on the same
bf16/fp32 inputs to a relative Frobenius error of 5e-3 per layer.  Sizes span several
256-row and 256-feature tiles with ragged row tails."""

import numpy as np
import pytest
import torch

import oracle
from ridge_map_kv_amd import binding as B
from ridge_map_kv_amd import configs, synth

from fillcase import Case, build_inputs, check_routing, check_values, run_fill

pytestmark = pytest.mark.gpu


def _filled(case):
    f, _, _ = oracle.partition(case.N, case.T, case.exact)
    return f


def _tiny_case():
    cfg = configs.TINY
    # maps: the oracle's ridge fit (lambda = 0.03) on 2048 seeded synthetic calibration rows
    xS, xl = synth.calib_data(cfg.d, cfg.n_upper, cfg.calib_rows, seed=cfg.seed)
    st = oracle.calib_new(cfg.d, cfg.n_upper)
    oracle.calib_accumulate(st, xS.astype(np.float64), [y.astype(np.float64) for y in xl])
    A, b = oracle.solve(st, cfg.lam)
    maps = [(A[l].astype(np.float32), b[l].astype(np.float32)) for l in range(cfg.n_upper)]
    return Case(d=cfg.d, n_layers=cfg.n_upper, n_kv=cfg.n_kv, hd=cfg.head_dim, N=cfg.N, T=cfg.T,
                exact=synth.exact_rows(cfg), page_size=cfg.page_size, seed=cfg.seed,
                eps=cfg.rms_eps, theta=cfg.rope_theta, map_kind="given", maps=maps)


def test_tiny_config_full_parity():
    case = _tiny_case()
    inp = build_inputs(case)
    f = _filled(case)
    assert len(f) == 7
    assert run_fill(case, inp, f) == B.RF_OK
    check_routing(case, inp, f)
    check_values(case, inp, f)


MULTI = [
    # d, layers, n_kv, hd, N, T, n_exact, page, seed
    (512, 3, 2, 128, 700, 100, 60, 16, 11),      # 540 filled: 3 row tiles, ragged
    (768, 2, 4, 64, 333, 33, 17, 8, 12),         # hd = 64, 3 map feature tiles
    (1024, 2, 8, 128, 1100, 64, 0, 16, 13),      # no exact rows, 5 row tiles, kv = 1024
    (256, 5, 1, 128, 257, 0, 1, 1, 14),          # T = 0, page size 1, 256 filled rows
]


@pytest.mark.parametrize("d,nl,nkv,hd,N,T,ne,ps,seed", MULTI)
def test_multi_tile_parity(d, nl, nkv, hd, N, T, ne, ps, seed):
    g = np.random.default_rng(seed)
    exact = np.sort(g.choice(N - T, size=ne, replace=False)) if ne else np.zeros(0, np.int64)
    case = Case(d=d, n_layers=nl, n_kv=nkv, hd=hd, N=N, T=T, exact=exact, page_size=ps, seed=seed)
    inp = build_inputs(case)
    f = _filled(case)
    assert run_fill(case, inp, f) == B.RF_OK
    check_routing(case, inp, f)
    check_values(case, inp, f)


def test_identity_map_equals_identity_fill():
    # Table 3's identity arm: with A = I, b = 0 the fill is POP's identity fill.
    case = Case(d=512, n_layers=2, n_kv=2, hd=128, N=400, T=50, exact=np.array([3, 200]),
                page_size=16, seed=21, map_kind="identity")
    inp = build_inputs(case)
    f = _filled(case)
    assert run_fill(case, inp, f) == B.RF_OK
    check_routing(case, inp, f)
    check_values(case, inp, f)


def test_empty_filled_list_leaves_cache_byte_identical():
    case = Case(d=256, n_layers=2, n_kv=1, hd=128, N=40, T=40, exact=np.zeros(0, np.int64),
                page_size=4, seed=22)
    inp = build_inputs(case)
    before = [l["k_pages"].clone() for l in inp["layers"]]
    assert run_fill(case, inp, np.zeros(0, np.int32)) == B.RF_OK
    for l, b in zip(inp["layers"], before):
        assert torch.equal(l["k_pages"].view(torch.int16), b.view(torch.int16))
        assert bool((l["v_pages"].view(torch.int16) == -1).all())


def test_deterministic_and_group_and_split_invariant():
    case = Case(d=512, n_layers=3, n_kv=2, hd=128, N=900, T=100, exact=np.arange(10, 80, 7),
                page_size=16, seed=23)
    f = _filled(case)
    inp1 = build_inputs(case)
    assert run_fill(case, inp1, f) == B.RF_OK                 # all layers in one launch
    inp2 = build_inputs(case)
    assert run_fill(case, inp2, f, ws_layers=1) == B.RF_OK    # one layer per launch
    inp3 = build_inputs(case)
    cut = len(f) // 3
    assert run_fill(case, inp3, f[:cut]) == B.RF_OK           # rows split over two calls
    assert run_fill(case, inp3, f[cut:]) == B.RF_OK
    for l in range(case.n_layers):
        for key in ("k_pages", "v_pages"):
            a = inp1["layers"][l][key].view(torch.int16)
            assert torch.equal(a, inp2["layers"][l][key].view(torch.int16))
            assert torch.equal(a, inp3["layers"][l][key].view(torch.int16))


def test_host_argument_errors():
    case = Case(d=256, n_layers=1, n_kv=1, hd=128, N=20, T=4, exact=np.zeros(0, np.int64),
                page_size=4, seed=24)
    inp = build_inputs(case)
    f = _filled(case)
    idx = torch.from_numpy(f.astype(np.int32)).cuda()
    shape = B.make_shape(256, 1, 128)
    ws = torch.empty(B.ridgefill_fill_workspace_bytes(shape, len(f), 1), dtype=torch.uint8,
                     device="cuda")
    with pytest.raises(B.RidgeFillError) as e:       # more filled rows than the prefix
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, 17, inp["layers"], inp["table"],
                         4, inp["num_pages"], ws)
    assert e.value.status == B.RF_E_SHAPE
    with pytest.raises(B.RidgeFillError) as e:       # workspace too small
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, len(f), inp["layers"],
                         inp["table"], 4, inp["num_pages"], ws[:1024])
    assert e.value.status == B.RF_E_WORKSPACE
    bad = B.make_shape(256, 1, 96)
    with pytest.raises(B.RidgeFillError) as e:
        B.ridgefill_fill(bad, inp["xS"], case.N, case.T, idx, len(f), inp["layers"], inp["table"],
                         4, inp["num_pages"], ws)
    assert e.value.status == B.RF_E_SHAPE
    # nothing was written
    for l in inp["layers"]:
        assert bool((l["k_pages"].view(torch.int16) == -1).all())


def test_device_flags_bad_rows_and_skips_them():
    # In-range but repeated and out-of-prefix indices: the device guard flags them; the
    # out-of-prefix row is skipped (tail rows never receive a filled entry).
    case = Case(d=256, n_layers=1, n_kv=1, hd=128, N=20, T=4, exact=np.zeros(0, np.int64),
                page_size=4, seed=25)
    inp = build_inputs(case)
    idx = np.array([0, 1, 1, 5, 17], dtype=np.int32)        # repeat, and 17 >= N - T = 16
    assert run_fill(case, inp, idx) == B.RF_E_ROWS
    pg, sl = oracle.paged_location(np.array([17]), inp["table_np"], 4)
    k = inp["layers"][0]["k_pages"].view(torch.int16)
    assert bool((k[int(pg[0]), int(sl[0])] == -1).all())


def _random_cases(n, seed):
    """Seeded random small workloads over the options the ABI allows: model widths, head
    shapes, prompt and tail lengths (T = 0 and all-exact prefixes included), page sizes,
    rectangular and int8 maps, key norm, value rescale and folded layers."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        d = int(g.choice([256, 512, 768, 1024]))
        hd = int(g.choice([64, 128]))
        n_kv = int(g.choice([h for h in (1, 2, 4, 8) if (h * hd) % 128 == 0]))
        N = int(g.integers(2, 900))
        T = int(g.integers(0, N)) if g.random() < 0.8 else 0
        P = N - T
        ne = int(g.integers(0, P + 1)) if g.random() < 0.3 else int(g.integers(0, max(P // 10, 1)))
        exact = np.sort(g.choice(P, size=ne, replace=False)) if ne else np.zeros(0, np.int64)
        kind = g.choice(["plain", "rect", "int8", "folded"])
        d_in = 0
        if kind == "rect":
            d_in = int(g.choice([w for w in (256, 320, 512, 1024, 1280) if w != d]))
        if kind == "folded" and g.random() < 0.5 and d >= 512:
            d_in = int(g.choice([w for w in (256, 512, 768) if w < d]))   # a tall folded map
        out.append(dict(case=Case(d=d, n_layers=int(g.integers(1, 4)), n_kv=n_kv, hd=hd, N=N, T=T,
                                  exact=exact, page_size=int(g.choice([1, 3, 8, 16, 32])),
                                  seed=int(g.integers(1 << 20)), d_in=d_in,
                                  knorm=bool(g.random() < 0.3), vscale=bool(g.random() < 0.3),
                                  int8=kind == "int8"),
                        folded=kind == "folded"))
    return out


@pytest.mark.parametrize("k", range(32))
def test_seeded_random_workloads(k):
    # cases from 12 on also start from a workspace of 0xFF bytes, and every third of them,
    # every folded one and every one with 3 layers streams its maps (or folded buffers) from
    # page-locked host memory through a one-layer workspace (landing slots are reused from
    # the third layer on)
    spec = _random_cases(32, 2024)[k]
    case, folded = spec["case"], spec["folded"]
    streamed = k >= 12 and (k % 3 == 0 or folded or case.n_layers == 3)
    print(f"\ncase {k}: d={case.d} d_in={case.width} layers={case.n_layers} kv={case.n_kv}x"
          f"{case.hd} N={case.N} T={case.T} exact={len(case.exact)} page={case.page_size} "
          f"knorm={case.knorm} vscale={case.vscale} int8={case.int8} folded={folded} "
          f"streamed={streamed}", flush=True)
    inp = build_inputs(case)
    f = _filled(case)
    assert run_fill(case, inp, f, folded=folded, streamed=streamed,
                    ws_layers=1 if streamed else None,
                    ws_byte=0xFF if k >= 12 else None) == B.RF_OK
    check_routing(case, inp, f)
    if len(f):
        check_values(case, inp, f)
