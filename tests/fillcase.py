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
    d_in: int = 0                        # width of x_S (0: d); != d gives a rectangular map
    knorm: bool = False                  # per-head key norm
    vscale: bool = False                 # value-rescale factors
    int8: bool = False                   # int8 maps (codes + row scales)

    @property
    def kv(self):
        return self.n_kv * self.hd

    @property
    def width(self):
        return self.d_in or self.d

    @property
    def map_flags(self):
        return B.RF_MAPS_INT8 if self.int8 else 0


def build_inputs(case: Case, dev="cuda"):
    d, kv = case.d, case.kv
    xS = synth.x_split((case.N, case.width), seed=case.seed)
    table, num_pages = synth.block_table(case.N, case.page_size, case.seed)
    layers = []
    for l in range(case.n_layers):
        w, WK, WV = synth.layer_weights(d, kv, case.seed, l)
        if case.map_kind == "identity":
            A, b = np.eye(d, case.width, dtype=np.float32), np.zeros(d, dtype=np.float32)
        elif case.map_kind == "given":
            A, b = case.maps[l]
        elif case.width != d:
            A, b = synth.rect_map(d, case.width, case.seed, l)
        else:
            A, b = synth.near_identity_map(d, case.seed, l)
        lay = dict(b=torch.from_numpy(np.asarray(b, np.float32)).to(dev), norm_w=to_bf16(w, dev),
                   W_K=to_bf16(WK, dev), W_V=to_bf16(WV, dev))
        if case.int8:
            # codes from the oracle's float32 quantizer; the reference uses q * scale exactly
            q, sc = oracle.quantize_map_int8(A.astype(np.float32), np.float32)
            lay["A_q"] = torch.from_numpy(q).to(dev)
            lay["A_scale"] = torch.from_numpy(sc.astype(np.float32)).to(dev)
            lay["A_ref"] = oracle.dequantize_map_int8(q, sc)
        else:
            lay["A"] = to_bf16(A, dev)
        if case.knorm:
            lay["k_norm_w"] = to_bf16(synth.key_norm_weight(case.hd, case.seed, l), dev)
        if case.vscale:
            lay["v_scale"] = torch.from_numpy(synth.value_factors(case.n_kv, case.seed, l)).to(dev)
        layers.append(lay)
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


def make_shape(case: Case):
    return B.make_shape(case.d, case.n_kv, case.hd, case.eps, case.theta,
                        d_in=case.d_in if case.width != case.d else 0)


def host_maps(layers: list[dict]) -> list[dict]:
    """The same layers with their maps (A or A_q, or the folded buffer) copied to
    page-locked host tensors."""
    out = []
    for lay in layers:
        h = dict(lay)
        key = "folded" if "folded" in lay else "A_q" if "A_q" in lay else "A"
        pinned = torch.empty(lay[key].shape, dtype=lay[key].dtype, pin_memory=True)
        pinned.copy_(lay[key].cpu())
        h[key] = pinned
        out.append(h)
    return out


def fold_offsets(case: Case):
    """Byte offsets of P, R1, c, r1, g and kappa in one layer's folded buffer: the sections
    in that order, each starting on a 256-byte boundary."""
    a = lambda x: (x + 255) // 256 * 256
    kv2, din = 2 * case.kv, case.width
    R = a(kv2 * din * 2)
    c = R + a(din * din * 2)
    r = c + a(kv2 * 4)
    g = r + a(din * 4)
    return 0, R, c, r, g, g + a(din * 4)


def fold_layers(case: Case, inp, stream=None, layers_at_once=None):
    """Folded buffers of every layer (cached in inp["folded"]) and the fold's status.  The
    workspace folds layers_at_once layers side by side (default: all of them)."""
    dev = inp["xS"].device
    shape = make_shape(case)
    nb = B.ridgefill_fold_bytes(shape)
    assert nb > 0
    g = layers_at_once or len(inp["layers"])
    ws = torch.empty(B.ridgefill_fold_workspace_bytes_maps(shape, g, case.map_flags),
                     dtype=torch.uint8, device=dev)
    bufs = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in inp["layers"]]
    B.ridgefill_fold_maps(shape, inp["layers"], bufs, ws, stream)
    status = B.ridgefill_read_status(ws, stream)
    inp["folded"] = bufs
    return bufs, status


def fold_raw(case: Case, buf: torch.Tensor):
    """(P, R1, c, r1, g, kappa) of a folded buffer as stored, float64 numpy values."""
    oP, oR, oc, orr, og, ok = fold_offsets(case)
    kv2, din = 2 * case.kv, case.width
    b = buf.cpu()
    P = b[oP:oP + kv2 * din * 2].view(torch.bfloat16).float().numpy().reshape(kv2, din)
    R1 = b[oR:oR + din * din * 2].view(torch.bfloat16).float().numpy().reshape(din, din)
    c = b[oc:oc + kv2 * 4].view(torch.float32).numpy()
    r1 = b[orr:orr + din * 4].view(torch.float32).numpy()
    g = b[og:og + din * 4].view(torch.float32).numpy()
    kappa = float(b[ok:ok + 4].view(torch.float32).item())
    return (P.astype(np.float64), R1.astype(np.float64), c.astype(np.float64),
            r1.astype(np.float64), g.astype(np.float64), kappa)


def fold_views(case: Case, buf: torch.Tensor):
    """(P, R, c, r, kappa) of a folded buffer, as float64 numpy values, with R = diag(g) R1
    and r = g r1 (the buffer holds R's rows over their diagonal entries, and the diagonal
    apart)."""
    P, R1, c, r1, g, kappa = fold_raw(case, buf)
    return P, R1 * g[:, None], c, r1 * g, kappa


def folded_layer_dicts(inp):
    keep = ("k_pages", "v_pages", "k_norm_w", "v_scale")
    return [dict({k: lay[k] for k in keep if k in lay}, folded=buf)
            for lay, buf in zip(inp["layers"], inp["folded"])]


def run_fill(case: Case, inp, filled: np.ndarray, ws_layers: int | None = None, stream=None,
             streamed: bool = False, folded: bool = False, ws_byte: int | None = None):
    dev = inp["xS"].device
    shape = make_shape(case)
    nf = int(filled.size)
    idx = torch.from_numpy(np.asarray(filled, dtype=np.int32)).to(dev)
    flags = case.map_flags | (B.RF_MAPS_STREAMED if streamed else 0)
    if folded:
        flags = B.RF_MAPS_FOLDED | (B.RF_MAPS_STREAMED if streamed else 0)
        if "folded" not in inp:
            _, st = fold_layers(case, inp, stream)
            assert st == B.RF_OK, f"fold status {st}"
    nbytes = B.ridgefill_fill_workspace_bytes(shape, max(nf, 1),
                                              ws_layers if ws_layers else case.n_layers, flags)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if ws_byte is not None:          # poison: a read of workspace bytes the call never wrote
        ws.fill_(ws_byte)            # then shows in the results
    if folded and streamed:
        layers = host_maps(folded_layer_dicts(inp))
        copy = torch.cuda.Stream()
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, nf, layers, inp["table"],
                         case.page_size, inp["num_pages"], ws, stream=stream, copy_stream=copy)
    elif folded:
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, nf, folded_layer_dicts(inp),
                         inp["table"], case.page_size, inp["num_pages"], ws, stream=stream)
    elif streamed:
        layers = host_maps(inp["layers"])
        copy = torch.cuda.Stream()
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, nf, layers, inp["table"],
                         case.page_size, inp["num_pages"], ws, stream=stream, copy_stream=copy)
    else:
        B.ridgefill_fill(shape, inp["xS"], case.N, case.T, idx, nf, inp["layers"], inp["table"],
                         case.page_size, inp["num_pages"], ws, stream=stream)
    status = B.ridgefill_read_status(ws, stream)
    return status


def oracle_layer(case: Case, inp, l: int, filled: np.ndarray, rows: np.ndarray | None = None):
    """float64 K, V [len(rows), n_kv, hd] for the filled rows `rows` (default all)."""
    lay = inp["layers"][l]
    sel = filled if rows is None else rows
    xs = bf16_np(inp["xS"][torch.from_numpy(np.asarray(sel, np.int64)).to(inp["xS"].device)])
    A = lay["A_ref"] if "A_ref" in lay else bf16_np(lay["A"])
    kn = bf16_np(lay["k_norm_w"]) if "k_norm_w" in lay else None
    vs = lay["v_scale"].cpu().numpy().astype(np.float64) if "v_scale" in lay else None
    return oracle.fill_rows(xs, sel, A, lay["b"].cpu().numpy().astype(np.float64),
                            bf16_np(lay["norm_w"]), bf16_np(lay["W_K"]), bf16_np(lay["W_V"]),
                            eps=case.eps, theta=case.theta, n_kv=case.n_kv, hd=case.hd,
                            k_norm_w=kn, v_scale=vs)


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
