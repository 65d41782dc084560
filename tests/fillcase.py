"""Builds one fill case: seeded inputs on the GPU, the HIP fill through the C ABI, and the
oracle's float64 reference from the very same bf16/fp32 values."""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import oracle
from ridge_map_kv_amd import binding as B
from ridge_map_kv_amd import synth

SENTINEL = 0xFFFF          # bf16 bit pattern the fill never produces from finite inputs
TOL = 5e-3                 # relative Frobenius bound on K and V


def to_bf16(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(torch.bfloat16)


def bf16_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


@dataclass
class Case:
    d: int
    n_layers: int
    n_kv: int
    hd: int
    N: int
    T: int
    exact: np.ndarray
    page_size: int
    seed: int
    eps: float = 1e-5
    theta: float = 500000.0
    map_kind: str = "near_identity"      # or "identity", or "given"
    maps: list | None = None             # [(A float32 [d,d], b float32 [d])] for "given"

    @property
    def kv(self):
        return self.n_kv * self.hd


def build_inputs(case: Case, dev="cuda"):
    d, kv = case.d, case.kv
    xS = synth.x_split((case.N, d), seed=case.seed)
    table, num_pages = synth.block_table(case.N, case.page_size, case.seed)
    layers = []
    for l in range(case.n_layers):
        w, WK, WV = synth.layer_weights(d, kv, case.seed, l)
        if case.map_kind == "identity":
            A, b = np.eye(d, dtype=np.float32), np.zeros(d, dtype=np.float32)
        elif case.map_kind == "given":
            A, b = case.maps[l]
        else:
            A, b = synth.near_identity_map(d, case.seed, l)
        layers.append(dict(A=to_bf16(A, dev), b=torch.from_numpy(np.asarray(b, np.float32)).to(dev),
                           norm_w=to_bf16(w, dev), W_K=to_bf16(WK, dev), W_V=to_bf16(WV, dev)))
    for lay in layers:
        shape = (num_pages, case.page_size, case.n_kv, case.hd)
        lay["k_pages"] = _sentinel(shape, dev)
        lay["v_pages"] = _sentinel(shape, dev)
    return dict(xS=to_bf16(xS, dev), table=torch.from_numpy(table).to(dev), num_pages=num_pages,
                table_np=table, layers=layers)


def _sentinel(shape, dev):
    t = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    t.view(torch.int16).fill_(-1)            # 0xFFFF
    return t


def run_fill(case: Case, inp, filled: np.ndarray, ws_layers: int | None = None, stream=None):
    dev = inp["xS"].device
    shape = B.make_shape(case.d, case.n_kv, case.hd, case.eps, case.theta)
    nf = int(filled.size)
    idx = torch.from_numpy(np.asarray(filled, dtype=np.int32)).to(dev)
    nbytes = B.ridgefill_fill_workspace_bytes(shape, max(nf, 1),
                                              ws_layers if ws_layers else case.n_layers)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, nf, inp["layers"], inp["table"],
                     case.page_size, inp["num_pages"], ws, stream=stream)
    status = B.ridgefill_read_status(ws, stream)
    return status


def oracle_layer(case: Case, inp, l: int, filled: np.ndarray, rows: np.ndarray | None = None):
    """float64 K, V [len(rows), n_kv, hd] for the filled rows `rows` (default all)."""
    lay = inp["layers"][l]
    sel = filled if rows is None else rows
    xs = bf16_np(inp["xS"][torch.from_numpy(np.asarray(sel, np.int64)).to(inp["xS"].device)])
    return oracle.fill_rows(xs, sel, bf16_np(lay["A"]), lay["b"].cpu().numpy().astype(np.float64),
                            bf16_np(lay["norm_w"]), bf16_np(lay["W_K"]), bf16_np(lay["W_V"]),
                            eps=case.eps, theta=case.theta, n_kv=case.n_kv, hd=case.hd)


def gpu_rows(case: Case, inp, l: int, rows: np.ndarray):
    """GPU K, V of prompt rows `rows` read back through the block table (float64)."""
    pg, sl = oracle.paged_location(rows, inp["table_np"], case.page_size)
    pg = torch.from_numpy(pg).to(inp["xS"].device)
    sl = torch.from_numpy(sl).to(inp["xS"].device)
    lay = inp["layers"][l]
    return bf16_np(lay["k_pages"][pg, sl]), bf16_np(lay["v_pages"][pg, sl])


def written_mask(case: Case, inp, l: int) -> np.ndarray:
    """[num_pages, page_size] bool: slots whose K or V differs from the sentinel anywhere,
    and [num_pages, page_size] bool: slots that are entirely sentinel."""
    lay = inp["layers"][l]
    k = lay["k_pages"].view(torch.int16) != -1
    v = lay["v_pages"].view(torch.int16) != -1
    any_w = (k.flatten(2).any(-1) | v.flatten(2).any(-1)).cpu().numpy()
    all_w = (k.flatten(2).all(-1) & v.flatten(2).all(-1)).cpu().numpy()
    return any_w, all_w


def check_routing(case: Case, inp, filled: np.ndarray):
    """Bit-exact routing: every slot of a filled row is fully written; every other slot of
    every layer still holds the sentinel in all its bytes."""
    pg, sl = oracle.paged_location(filled, inp["table_np"], case.page_size)
    expect = np.zeros((inp["num_pages"], case.page_size), dtype=bool)
    expect[pg, sl] = True
    for l in range(case.n_layers):
        any_w, all_w = written_mask(case, inp, l)
        assert np.array_equal(any_w, expect), f"layer {l}: writes outside the filled rows"
        assert np.all(all_w[expect]), f"layer {l}: a filled row was not fully written"


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_values(case: Case, inp, filled: np.ndarray, rows: np.ndarray | None = None,
                 layers=None, tol: float = TOL):
    worst = 0.0
    sel = filled if rows is None else rows
    for l in (range(case.n_layers) if layers is None else layers):
        Ko, Vo = oracle_layer(case, inp, l, filled, sel)
        Kg, Vg = gpu_rows(case, inp, l, sel)
        ek, ev = rel_fro(Kg, Ko), rel_fro(Vg, Vo)
        worst = max(worst, ek, ev)
        assert ek <= tol and ev <= tol, f"layer {l}: rel Frobenius K {ek:.3e} V {ev:.3e}"
    return worst
