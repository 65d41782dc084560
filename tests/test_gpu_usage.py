"""The library used end to end through the binding, as README.md shows it: calibrate, solve
one lambda, fill plain layers, fold them, fill the folded layers; the two fills agree to
bf16 rounding and write the same cache slots."""

import numpy as np
import pytest
import torch

from ridge_map_kv_amd import binding as B

pytestmark = pytest.mark.gpu


def test_calibrate_solve_fold_fill():
    dev = "cuda"
    d, L, n_kv, hd = 256, 2, 2, 128                 # hidden size, upper layers, KV heads
    N, T, page = 300, 20, 16                        # prompt rows, tail rows, page size
    g = torch.Generator(device=dev).manual_seed(7)
    bf = lambda *s, scale=1.0: (torch.randn(*s, generator=g, device=dev) * scale).to(torch.bfloat16)

    # one-pass calibration over chunks of (x_S, [x_l for each upper layer])
    W_true = [torch.eye(d, device=dev) + 0.05 * torch.randn(d, d, generator=g, device=dev)
              for _ in range(L)]
    state = torch.empty(B.ridgefill_calib_state_bytes(d, L), dtype=torch.uint8, device=dev)
    B.ridgefill_calib_reset(state, d, L)
    for rows in (1000, 1000, 500):
        xs = torch.randn(rows, d, generator=g, device=dev)
        xl = [(xs @ W.T + 0.1 * torch.randn(rows, d, generator=g, device=dev)).to(torch.bfloat16)
              for W in W_true]
        B.ridgefill_calibrate(state, d, L, xs.to(torch.bfloat16), xl)

    # the closed-form ridge solve for one lambda
    A = torch.empty(L, d, d, dtype=torch.float32, device=dev)
    b = torch.empty(L, d, dtype=torch.float32, device=dev)
    A16 = torch.empty(L, d, d, dtype=torch.bfloat16, device=dev)
    sws = torch.empty(B.ridgefill_solve_workspace_bytes(d, L), dtype=torch.uint8, device=dev)
    B.ridgefill_solve(state, d, L, 0.03, A, b, A16, sws)
    assert B.ridgefill_read_status(sws) == B.RF_OK

    # the prompt: split-layer states, exact rows, a paged cache per layer
    x_S = bf(N, d)
    exact_mask = np.zeros(N - T, np.uint8)
    exact_mask[::10] = 1
    filled = B.ridgefill_partition(N, T, exact_mask)           # ascending int32 rows
    idx = torch.from_numpy(filled).to(dev)
    num_pages = (N + page - 1) // page
    block_table = torch.randperm(num_pages, generator=g, device=dev).to(torch.int32)
    pools = lambda: torch.full((num_pages, page, n_kv, hd), -1, dtype=torch.int16,
                               device=dev).view(torch.bfloat16)
    w = [(1 + 0.1 * torch.randn(d, generator=g, device=dev)).to(torch.bfloat16) for _ in range(L)]
    WK = [bf(n_kv * hd, d, scale=d ** -0.5) for _ in range(L)]
    WV = [bf(n_kv * hd, d, scale=d ** -0.5) for _ in range(L)]
    shape = B.make_shape(d, n_kv, hd, rms_eps=1e-5, rope_theta=5e5)

    # fill with the maps as they are
    layers = [dict(A=A16[l], b=b[l], norm_w=w[l], W_K=WK[l], W_V=WV[l], k_pages=pools(),
                   v_pages=pools()) for l in range(L)]
    ws = torch.empty(B.ridgefill_fill_workspace_bytes(shape, len(filled), L), dtype=torch.uint8,
                     device=dev)
    B.ridgefill_fill(shape, x_S, N, T, idx, len(filled), layers, block_table, page, num_pages, ws)
    assert B.ridgefill_read_status(ws) == B.RF_OK

    # fold once per model (and lambda), then fill the folded layers
    fws = torch.empty(B.ridgefill_fold_workspace_bytes_ex(shape, L), dtype=torch.uint8, device=dev)
    bufs = [torch.empty(B.ridgefill_fold_bytes(shape), dtype=torch.uint8, device=dev)
            for _ in range(L)]
    B.ridgefill_fold_maps(shape, layers, bufs, fws)
    assert B.ridgefill_read_status(fws) == B.RF_OK
    folded = [dict(folded=bufs[l], k_pages=pools(), v_pages=pools()) for l in range(L)]
    fws2 = torch.empty(B.ridgefill_fill_workspace_bytes(shape, len(filled), L, B.RF_MAPS_FOLDED),
                       dtype=torch.uint8, device=dev)
    B.ridgefill_fill(shape, x_S, N, T, idx, len(filled), folded, block_table, page, num_pages,
                     fws2)
    assert B.ridgefill_read_status(fws2) == B.RF_OK

    for a, f in zip(layers, folded):
        for key in ("k_pages", "v_pages"):
            written = a[key].view(torch.int16) != -1
            assert torch.equal(written, f[key].view(torch.int16) != -1)
            assert int(written.flatten(2).all(-1).sum()) == len(filled)
            x, y = a[key].float()[written], f[key].float()[written]
            assert float(torch.linalg.norm(x - y) / torch.linalg.norm(x)) <= 5e-3
