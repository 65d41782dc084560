"""Parity at the workloads' full sizes, in the launch configuration the benchmark times
(all upper layers in one call, workspace for all of them).

Fill (8B, Qwen3-8B and 27B shapes): routing is checked bit-exactly on every byte of every
layer's K and V pools (sentinel-filled before the call); K and V are checked against the
oracle on 512 seeded filled rows of every layer (first and last filled row, rows next to
exact rows, rows on page edges, the rest uniform), and on every filled row of the first
and the last upper layer.

Calibration (8B shape, 131,072 rows in 16,384-row chunks): 256 seeded columns of the
Gram matrix, 256 seeded rows of every Y_l^T X and the matching sums against the oracle's
float64 accumulation of the same bf16 rows.  Solve at full size: the oracle's float64
solve of the statistics the GPU accumulated, for every layer at all six lambdas, with the
normal-equation residual; and a Hadamard design whose answer is known in closed form."""

import numpy as np
import pytest
import torch

import oracle
from ridge_map_kv_amd import binding as B
from ridge_map_kv_amd import configs, synth

pytestmark = pytest.mark.gpu
TOL = 5e-3


def _np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def _all_rows_layer(cfg, inp, filled, pg, sl, l, A_of=None, kn_of=None, block=4096):
    """Relative Frobenius errors of K and V over every filled row of layer l against the
    oracle's plain fill, accumulated over blocks of rows (the oracle is row-wise)."""
    dev = inp["xS"].device
    lay = inp["layers"][l]
    A = A_of(l) if A_of else _np64(lay["A"])
    b = lay["b"].cpu().numpy().astype(np.float64)
    w, WK, WV = _np64(lay["norm_w"]), _np64(lay["W_K"]), _np64(lay["W_V"])
    kn = kn_of(l) if kn_of else None
    num = np.zeros(2)
    den = np.zeros(2)
    for r0 in range(0, filled.size, block):
        rows = filled[r0:r0 + block]
        xs = _np64(inp["xS"][torch.from_numpy(rows).to(dev)])
        Ko, Vo = oracle.fill_rows(xs, rows, A, b, w, WK, WV, eps=cfg.rms_eps,
                                  theta=cfg.rope_theta, n_kv=cfg.n_kv, hd=cfg.head_dim,
                                  k_norm_w=kn)
        tpg = torch.from_numpy(pg[r0:r0 + block]).to(dev)
        tsl = torch.from_numpy(sl[r0:r0 + block]).to(dev)
        for j, (key, want) in enumerate((("k_pages", Ko), ("v_pages", Vo))):
            got = _np64(lay[key][tpg, tsl])
            num[j] += np.sum((got - want) ** 2)
            den[j] += np.sum(want ** 2)
    return float(np.sqrt(num[0] / den[0])), float(np.sqrt(num[1] / den[1]))


def _sample_rows(filled, exact, page_size, n=512, seed=7):
    g = np.random.default_rng(seed)
    ex = np.zeros(int(filled[-1]) + 2, dtype=bool)
    ex[exact[exact < ex.size]] = True
    f = filled.astype(np.int64)
    adj = f[ex[np.maximum(f - 1, 0)] | ex[f + 1]]
    edge = f[(f % page_size == 0) | (f % page_size == page_size - 1)]
    pick = [f[:1], f[-1:]]
    if adj.size:
        pick.append(g.choice(adj, size=min(64, adj.size), replace=False))
    pick.append(g.choice(edge, size=min(64, edge.size), replace=False))
    rest = n - sum(p.size for p in pick)
    pick.append(g.choice(f, size=rest, replace=False))
    return np.unique(np.concatenate(pick))


@pytest.mark.parametrize("name", ["llama3.1-8b", "qwen3-8b", "27b-long"])
def test_full_size_fill(name):
    cfg = configs.FILL_CONFIGS[name]
    dev = torch.device("cuda")
    print(f"\nfull fill {name}: generating inputs", flush=True)
    inp = synth.device_fill_inputs(cfg, dev, sentinel=True)
    filled = B.ridgefill_partition(cfg.N, cfg.T, inp["exact_mask"])
    want, exact, tail = oracle.partition(cfg.N, cfg.T, synth.exact_rows(cfg))
    assert np.array_equal(filled, want) and filled.size == cfg.n_filled

    shape = B.make_shape(cfg.d, cfg.n_kv, cfg.head_dim, cfg.rms_eps, cfg.rope_theta)
    idx = torch.from_numpy(filled).to(dev)
    ws = torch.empty(B.ridgefill_fill_workspace_bytes(shape, filled.size, cfg.n_upper),
                     dtype=torch.uint8, device=dev)
    B.ridgefill_fill(shape, inp["xS"], cfg.N, cfg.T, idx, filled.size, inp["layers"], inp["table"],
                     cfg.page_size, inp["num_pages"], ws)
    assert B.ridgefill_read_status(ws) == B.RF_OK
    print(f"full fill {name}: routing", flush=True)

    pg, sl = oracle.paged_location(filled, inp["table_np"], cfg.page_size)
    expect = torch.zeros((inp["num_pages"], cfg.page_size), dtype=torch.bool, device=dev)
    expect[torch.from_numpy(pg).to(dev), torch.from_numpy(sl).to(dev)] = True
    for l, lay in enumerate(inp["layers"]):
        for key in ("k_pages", "v_pages"):
            sent = lay[key].view(torch.int16) == -1
            untouched = sent.flatten(2).all(-1)
            written = (~sent).flatten(2).all(-1)
            assert torch.equal(written, expect), f"layer {l} {key}: a filled row not fully written"
            assert torch.equal(untouched, ~expect), f"layer {l} {key}: write outside filled rows"
            del sent, untouched, written

    print(f"full fill {name}: numerics", flush=True)
    rows = _sample_rows(filled, exact, cfg.page_size)
    xs = _np64(inp["xS"][torch.from_numpy(rows).to(dev)])
    rpg = torch.from_numpy(pg[np.searchsorted(filled, rows)]).to(dev)
    rsl = torch.from_numpy(sl[np.searchsorted(filled, rows)]).to(dev)
    worst = 0.0
    for l, lay in enumerate(inp["layers"]):
        Ko, Vo = oracle.fill_rows(xs, rows, _np64(lay["A"]), lay["b"].cpu().numpy().astype(np.float64),
                                  _np64(lay["norm_w"]), _np64(lay["W_K"]), _np64(lay["W_V"]),
                                  eps=cfg.rms_eps, theta=cfg.rope_theta, n_kv=cfg.n_kv,
                                  hd=cfg.head_dim)
        Kg = _np64(lay["k_pages"][rpg, rsl])
        Vg = _np64(lay["v_pages"][rpg, rsl])
        ek, ev = _rel(Kg, Ko), _rel(Vg, Vo)
        worst = max(worst, ek, ev)
        assert ek <= TOL and ev <= TOL, f"layer {l}: K {ek:.3e} V {ev:.3e}"
    print(f"full fill {name}: {rows.size} rows x {cfg.n_upper} layers, worst rel {worst:.2e}",
          flush=True)
    for l in (0, cfg.n_upper - 1):
        ek, ev = _all_rows_layer(cfg, inp, filled, pg, sl, l)
        print(f"full fill {name}: layer {l}, all {filled.size} rows: K {ek:.2e} V {ev:.2e}",
              flush=True)
        assert ek <= TOL and ev <= TOL, f"layer {l} all rows: K {ek:.3e} V {ev:.3e}"


def _state_arrays(state, d, L):
    raw = state.cpu().numpy()
    off = 256
    n = int(raw[:8].view(np.int64)[0])
    sS = raw[off:off + 8 * d].view(np.float64); off += 8 * d
    sl = raw[off:off + 8 * d * L].view(np.float64).reshape(L, d); off += 8 * d * L
    G = raw[off:off + 4 * d * d].view(np.float32).reshape(d, d); off += 4 * d * d
    YX = raw[off:off + 4 * d * d * L].view(np.float32).reshape(L, d, d); off += 4 * d * d * L
    shift = raw[off:off + 4 * d].view(np.float32).astype(np.float64)
    return n, sS, sl, G, YX, shift


def test_full_size_calibration_sampled():
    ccfg = configs.CALIB8B
    d, L = ccfg.d, ccfg.n_layers
    dev = torch.device("cuda")
    print("\nfull calibration: generating rows", flush=True)
    chunks = synth.device_calib_chunks(ccfg, dev)
    state = torch.empty(B.ridgefill_calib_state_bytes(d, L), dtype=torch.uint8, device=dev)
    B.ridgefill_calib_reset(state, d, L)
    for xs, xl in chunks:
        B.ridgefill_calibrate(state, d, L, xs, xl)
    torch.cuda.synchronize()
    n, sS, sl, G, YX, shift = _state_arrays(state, d, L)
    assert n == ccfg.rows
    assert not shift.any()              # zero-mean rows: the moments are the raw ones

    print("full calibration: oracle on sampled entries", flush=True)
    g = np.random.default_rng(11)
    cols = np.sort(g.choice(d, size=256, replace=False))
    outs = np.sort(g.choice(d, size=256, replace=False))
    Gc = np.zeros((d, cols.size))
    Yr = np.zeros((L, outs.size, d))
    sS_o = np.zeros(d)
    sl_o = np.zeros((L, outs.size))
    ci = torch.from_numpy(cols).to(dev)
    oi = torch.from_numpy(outs).to(dev)
    for xs, xl in chunks:
        X = _np64(xs)
        Gc += X.T @ X[:, cols]
        sS_o += X.sum(axis=0)
        for l in range(L):
            Yo = _np64(xl[l][:, oi])
            Yr[l] += Yo.T @ X
            sl_o[l] += Yo.sum(axis=0)
    low = np.arange(d)[:, None] >= cols[None, :]           # valid lower-triangle entries
    assert _rel(G[:, cols][low].astype(np.float64), Gc[low]) < 1e-5
    assert _rel(YX[:, outs, :].astype(np.float64), Yr) < 1e-5
    np.testing.assert_allclose(sS, sS_o, rtol=1e-6, atol=1e-2)
    np.testing.assert_allclose(sl[:, outs], sl_o, rtol=1e-6, atol=1e-2)


@pytest.fixture(scope="module")
def calib8b():
    """The 8B-shaped calibration (131,072 rows in 16,384-row calls) on the GPU, and the
    statistics it accumulated read back as the oracle's CalibStats in float64."""
    ccfg = configs.CALIB8B
    d, L = ccfg.d, ccfg.n_layers
    dev = torch.device("cuda")
    print("\nfull solve: calibrating 131,072 rows", flush=True)
    chunks = synth.device_calib_chunks(ccfg, dev)
    state = torch.empty(B.ridgefill_calib_state_bytes(d, L), dtype=torch.uint8, device=dev)
    B.ridgefill_calib_reset(state, d, L)
    for xs, xl in chunks:
        B.ridgefill_calibrate(state, d, L, xs, xl)
    torch.cuda.synchronize()
    del chunks
    torch.cuda.empty_cache()
    n, sS, sl, G, YX, shift = _state_arrays(state, d, L)
    st = oracle.calib_new(d, L)
    st.n = n
    st.s_S = sS.astype(np.float64)
    st.s_l = sl.astype(np.float64)
    low = np.tril(G.astype(np.float64))
    st.G = low + np.tril(low, -1).T
    st.YX = YX.astype(np.float64)
    return state, st, shift


@pytest.mark.parametrize("lam", [1e-4, 1e-3, 0.01, 0.03, 0.1, 1.0])
def test_full_size_solve_vs_oracle(calib8b, lam):
    # the oracle's float64 Cholesky solve of the very statistics the GPU accumulated, for
    # all 20 layers; the GPU's shift (zero here) enters only b = mu_l - A (mu' + s)
    state, st, shift = calib8b
    d, L = st.d, st.n_layers
    dev = torch.device("cuda")
    A = torch.empty((L, d, d), dtype=torch.float32, device=dev)
    b = torch.empty((L, d), dtype=torch.float32, device=dev)
    ws = torch.empty(B.ridgefill_solve_workspace_bytes(d, L), dtype=torch.uint8, device=dev)
    B.ridgefill_solve(state, d, L, lam, A, b, None, ws)
    assert B.ridgefill_read_status(ws) == B.RF_OK
    print(f"\nfull solve lambda {lam}: oracle", flush=True)
    Ao, bo = oracle.solve(st, lam)
    bo = bo - Ao @ shift
    _, _, XtX, YtX = oracle.centred_moments(st)
    Cp = torch.from_numpy(XtX + oracle.ridge_alpha(XtX, lam) * np.eye(d)).to(dev)
    worst_a = worst_b = worst_r = 0.0
    for l in range(L):
        Al = A[l].cpu().numpy().astype(np.float64)
        ea, eb = _rel(Al, Ao[l]), _rel(b[l].cpu().numpy().astype(np.float64), bo[l])
        Yt = torch.from_numpy(YtX[l]).to(dev)
        res = float(torch.linalg.norm(Cp @ A[l].double().T - Yt.T) / torch.linalg.norm(Yt))
        worst_a, worst_b, worst_r = max(worst_a, ea), max(worst_b, eb), max(worst_r, res)
        assert ea < TOL and eb < TOL, f"layer {l}: A {ea:.2e} b {eb:.2e}"
        assert res < 1e-4, f"layer {l}: residual {res:.2e}"
    print(f"full solve lambda {lam}: {L} layers, worst A {worst_a:.2e} b {worst_b:.2e} "
          f"residual {worst_r:.2e}", flush=True)


def test_full_size_solve_hadamard_closed_form():
    ccfg = configs.CALIB8B
    n, d, L = ccfg.rows, ccfg.d, ccfg.n_layers
    dev = torch.device("cuda")
    print("\nfull solve: Hadamard design", flush=True)
    g = np.random.default_rng(21)
    m = g.integers(-2, 3, size=d) / 2.0
    X = synth.device_hadamard_columns(n, d, dev)
    xS = (X + torch.from_numpy(m).float().to(dev)).to(torch.bfloat16)
    del X
    Ws, cs, ys = [], [], []
    for l in range(L):
        W = synth.sparse_dyadic_matrix(d, d, 300 + l)
        c = g.integers(-8, 9, size=d) / 4.0
        nz = [np.nonzero(W[o])[0] for o in range(d)]
        j0 = torch.from_numpy(np.array([z[0] for z in nz])).to(dev)
        j1 = torch.from_numpy(np.array([z[1] for z in nz])).to(dev)
        w0 = torch.from_numpy(W[np.arange(d), [z[0] for z in nz]]).to(dev)
        w1 = torch.from_numpy(W[np.arange(d), [z[1] for z in nz]]).to(dev)
        xf = xS.float()
        y = xf[:, j0] * w0 + xf[:, j1] * w1 + torch.from_numpy(c).float().to(dev)
        ys.append(y.to(torch.bfloat16))
        assert torch.equal(ys[-1].float(), y)               # exact in bf16
        del xf, y
        Ws.append(W.astype(np.float64))
        cs.append(c)
    state = torch.empty(B.ridgefill_calib_state_bytes(d, L), dtype=torch.uint8, device=dev)
    B.ridgefill_calib_reset(state, d, L)
    for r0 in range(0, n, ccfg.chunk):
        B.ridgefill_calibrate(state, d, L, xS[r0:r0 + ccfg.chunk], [y[r0:r0 + ccfg.chunk] for y in ys])
    A = torch.empty((L, d, d), dtype=torch.float32, device=dev)
    b = torch.empty((L, d), dtype=torch.float32, device=dev)
    ws = torch.empty(B.ridgefill_solve_workspace_bytes(d, L), dtype=torch.uint8, device=dev)
    for lam in (1e-4, 0.03, 1.0):
        B.ridgefill_solve(state, d, L, lam, A, b, None, ws)
        assert B.ridgefill_read_status(ws) == B.RF_OK
        for l in (0, L // 2, L - 1):
            Al = A[l].cpu().numpy().astype(np.float64)
            np.testing.assert_allclose(Al, Ws[l] / (1 + lam), atol=2e-5)
            np.testing.assert_allclose(b[l].cpu().numpy(), cs[l] + lam / (1 + lam) * (Ws[l] @ m),
                                       atol=2e-4)
        print(f"full solve: lambda {lam} closed form ok", flush=True)


def test_largest_prefix_accepted_one_more_refused():
    # The fill addresses gathered rows of x_S with 32-bit byte offsets; the host admits a
    # prefix whose last row ends within 4 GiB.  At d_in = x_stride = 256 that is
    # P = 8,388,607 rows (a 4.29 GB x_S): rows at both ends of the largest prefix are filled
    # correctly, and one more prefix row is refused before anything is enqueued.
    dev = torch.device("cuda")
    d, n_kv, hd, T, page = 256, 1, 128, 64, 256
    P = (0xFFFFFFFF - 2 * d) // (2 * d) + 1
    assert (P - 1) * 2 * d + 2 * d <= 0xFFFFFFFF < P * 2 * d + 2 * d
    N = P + T
    print(f"\nlargest prefix: P = {P:,} rows, x_S of {(N + 1) * d * 2 / 1e9:.2f} GB", flush=True)
    g = torch.Generator(device=dev).manual_seed(11)
    x_S = torch.empty((N + 1, d), dtype=torch.bfloat16, device=dev)
    for r0 in range(0, N + 1, 1 << 20):
        r1 = min(r0 + (1 << 20), N + 1)
        x_S[r0:r1] = torch.randn((r1 - r0, d), generator=g, device=dev).to(torch.bfloat16)
    A = torch.eye(d, device=dev) + 0.05 * torch.randn(d, d, generator=g, device=dev)
    A = A.to(torch.bfloat16)
    b = 0.1 * torch.randn(d, generator=g, device=dev)
    w = (1 + 0.1 * torch.randn(d, generator=g, device=dev)).to(torch.bfloat16)
    WK = (torch.randn(n_kv * hd, d, generator=g, device=dev) / d ** 0.5).to(torch.bfloat16)
    WV = (torch.randn(n_kv * hd, d, generator=g, device=dev) / d ** 0.5).to(torch.bfloat16)
    num_pages = (N + 1 + page - 1) // page
    table_np = np.random.default_rng(12).permutation(num_pages).astype(np.int32)
    table = torch.from_numpy(table_np).to(dev)
    pool = lambda: torch.full((num_pages, page, n_kv, hd), -1, dtype=torch.int16,
                              device=dev).view(torch.bfloat16)
    kp, vp = pool(), pool()
    rows = np.concatenate([np.arange(0, 50), np.arange(P - 250, P)]).astype(np.int32)
    idx = torch.from_numpy(rows).to(dev)
    shape = B.make_shape(d, n_kv, hd, 1e-5, 5e5)
    layer = [dict(A=A, b=b, norm_w=w, W_K=WK, W_V=WV, k_pages=kp, v_pages=vp)]
    ws = torch.empty(B.ridgefill_fill_workspace_bytes(shape, rows.size, 1), dtype=torch.uint8,
                     device=dev)
    B.ridgefill_fill(shape, x_S, N, T, idx, rows.size, layer, table, page, num_pages, ws)
    assert B.ridgefill_read_status(ws) == B.RF_OK
    pg, sl = oracle.paged_location(rows, table_np, page)
    written = kp.view(torch.int16) != -1
    expect = torch.zeros((num_pages, page), dtype=torch.bool, device=dev)
    expect[torch.from_numpy(pg).to(dev), torch.from_numpy(sl).to(dev)] = True
    assert torch.equal(written.flatten(2).all(-1), expect)
    assert torch.equal(written.flatten(2).any(-1), expect)
    Ko, Vo = oracle.fill_rows(_np64(x_S[idx.long()]), rows, _np64(A),
                              b.cpu().numpy().astype(np.float64), _np64(w), _np64(WK), _np64(WV),
                              eps=1e-5, theta=5e5, n_kv=n_kv, hd=hd)
    tpg, tsl = torch.from_numpy(pg).to(dev), torch.from_numpy(sl).to(dev)
    ek, ev = _rel(_np64(kp[tpg, tsl]), Ko), _rel(_np64(vp[tpg, tsl]), Vo)
    print(f"  rows 0..49 and {P - 250:,}..{P - 1:,}: K {ek:.2e} V {ev:.2e}", flush=True)
    assert ek <= 5e-3 and ev <= 5e-3
    # one more prefix row: the same call with T one smaller is refused on the host
    with pytest.raises(RuntimeError, match="4 GiB"):
        B.ridgefill_fill(shape, x_S, N + 1, T, idx, rows.size, layer, table, page,
                         num_pages, ws)
