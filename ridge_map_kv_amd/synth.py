"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and builds input structures (row masks, block
tables, synthetic linear "model" data).  It contains none of the method's arithmetic:
no map prediction, normalisation, projection, rotation, moment accumulation or solve.

Recipes (the shapes and value distributions of the workloads):
  * x_S ~ N(0, 1), drawn in float32 and rounded to bfloat16 where the library takes it.
  * norm weights w = 1 + 0.1 N(0, 1); key/value projections W_K, W_V ~ N(0, 1/d).
  * Synthetic layer inputs for calibration follow a near-identity linear model:
    x_l = W_true,l x_S + c_l + s * e, with W_true,l = I + U_l diag(0.5) V_l^T (rank 64,
    U, V ~ N(0, 1/d)), c_l ~ N(0, 1) and e either N(0, 1) or Student-t with 3 degrees
    of freedom (the heavy-tailed case).
  * Where a workload is too large for a CPU-side fit, a fill input map is drawn as
    A = I + U diag(0.5) V^T, b ~ N(0, 1): the same near-identity family.  The fill
    computes the same function of whatever map bytes it is given.
  * Exact prefix rows: a seeded uniform draw without replacement ("count"), none, or
    seeded contiguous blocks with lengths U[16, 80] covering half of the budget plus
    uniformly drawn singletons for the other half ("blocks").
  * Block tables: a seeded permutation of the physical pages.
  * Rectangular maps (input width d_in != output width d):
    A = [I | 0] + U V^T / 2 with U ~ N(0, 1/d) [d, 64], V ~ N(0, 1/d_in) [d_in, 64]
    (the identity block on the first d inputs), b ~ N(0, 1).
  * Key-norm weights 1 + 0.1 N(0, 1) [head_dim]; value-rescale factors U[0.5, 1.5].
  * Exact tail inputs for the value rescale: the near-identity model's x_l on the tail
    rows (x_l = W_true x_S + c + 0.1 e, e ~ N(0, 1)).
  * Attention-like row scores: Exp(1) draws, rounded to multiples of 1/64 so that ties
    occur.
"""

from __future__ import annotations

import numpy as np

TRUE_MAP_RANK = 64
TRUE_MAP_GAIN = 0.5


def rng(seed: int, *tags: int) -> np.random.Generator:
    """Independent stream for (seed, tags...), via SeedSequence spawn keys."""
    return np.random.default_rng(np.random.SeedSequence(entropy=int(seed),
                                                        spawn_key=tuple(int(t) for t in tags)))


# Stream tags, so every tensor has its own stream.
TAG_XS, TAG_EXACT, TAG_TABLE, TAG_NORM, TAG_WK, TAG_WV, TAG_MAPU, TAG_MAPV, TAG_MAPB, \
    TAG_CAL_X, TAG_CAL_NOISE, TAG_CAL_C, TAG_KNORM, TAG_VSCALE, TAG_SCORES = range(1, 16)
TAG_SPREAD, TAG_HARD = 16, 17


def exact_rows(cfg) -> np.ndarray:
    """Seeded exact prefix rows of a fill workload (ascending int64)."""
    P = cfg.prefix
    g = rng(cfg.seed, TAG_EXACT)
    if cfg.exact == "none" or cfg.exact_count == 0:
        return np.zeros(0, dtype=np.int64)
    if cfg.exact == "count":
        return np.sort(g.choice(P, size=cfg.exact_count, replace=False)).astype(np.int64)
    if cfg.exact == "blocks":
        return blocks_and_singletons(P, cfg.exact_count, g)
    raise ValueError(cfg.exact)


def blocks_and_singletons(P: int, count: int, g: np.random.Generator,
                          lo: int = 16, hi: int = 80) -> np.ndarray:
    taken = np.zeros(P, dtype=bool)
    block_budget = count // 2
    placed = 0
    while placed < block_budget:
        length = int(g.integers(lo, hi + 1))
        length = min(length, block_budget - placed)
        start = int(g.integers(0, P - length + 1))
        if taken[start:start + length].any():
            continue
        taken[start:start + length] = True
        placed += length
    free = np.flatnonzero(~taken)
    singles = g.choice(free, size=count - placed, replace=False)
    taken[singles] = True
    out = np.flatnonzero(taken).astype(np.int64)
    assert out.size == count
    return out


def exact_mask(cfg) -> np.ndarray:
    """uint8 mask over the prefix: 1 where the row is exact."""
    m = np.zeros(cfg.prefix, dtype=np.uint8)
    m[exact_rows(cfg)] = 1
    return m


def n_pages(N: int, page_size: int) -> int:
    return (N + page_size - 1) // page_size


def block_table(N: int, page_size: int, seed: int, spare: int = 3) -> tuple[np.ndarray, int]:
    """Permuted block table for one prompt.  Returns (table int32, number of physical
    pages); the pool has a few spare pages that no row maps to."""
    n_log = n_pages(N, page_size)
    num = n_log + spare
    perm = rng(seed, TAG_TABLE).permutation(num)[:n_log]
    return perm.astype(np.int32), num


def x_split(cfg_or_shape, seed: int | None = None) -> np.ndarray:
    """x_S ~ N(0, 1) float32 [N, d]."""
    if seed is None:
        N, d, seed = cfg_or_shape.N, cfg_or_shape.d, cfg_or_shape.seed
    else:
        N, d = cfg_or_shape
    return rng(seed, TAG_XS).standard_normal((N, d), dtype=np.float32)


def layer_weights(d: int, kv: int, seed: int, layer: int):
    """(norm_w, W_K, W_V) float32 for one layer: 1 + 0.1 N(0,1), N(0, 1/d), N(0, 1/d)."""
    s = 1.0 / np.sqrt(d)
    w = 1.0 + 0.1 * rng(seed, TAG_NORM, layer).standard_normal(d, dtype=np.float32)
    WK = s * rng(seed, TAG_WK, layer).standard_normal((kv, d), dtype=np.float32)
    WV = s * rng(seed, TAG_WV, layer).standard_normal((kv, d), dtype=np.float32)
    return w.astype(np.float32), WK.astype(np.float32), WV.astype(np.float32)


def true_map_factors(d: int, seed: int, layer: int, rank: int = TRUE_MAP_RANK):
    """U, V ~ N(0, 1/d) [d, rank] of W_true = I + U diag(0.5) V^T."""
    s = 1.0 / np.sqrt(d)
    U = s * rng(seed, TAG_MAPU, layer).standard_normal((d, rank), dtype=np.float32)
    V = s * rng(seed, TAG_MAPV, layer).standard_normal((d, rank), dtype=np.float32)
    return U.astype(np.float32), V.astype(np.float32)


def near_identity_map(d: int, seed: int, layer: int):
    """A = I + U diag(0.5) V^T (float32 [d, d]) and b ~ N(0, 1) (float32 [d])."""
    U, V = true_map_factors(d, seed, layer)
    A = np.eye(d, dtype=np.float32) + TRUE_MAP_GAIN * (U @ V.T)
    b = rng(seed, TAG_MAPB, layer).standard_normal(d, dtype=np.float32)
    return A.astype(np.float32), b.astype(np.float32)


def calib_data(d: int, n_layers: int, rows: int, seed: int, *, noise_scale: float = 0.1,
               noise_dof: float | None = None, x_shift: float = 0.0):
    """Synthetic calibration rows: x_S [rows, d] and x_l [n_layers, rows, d] (float32),
    x_l = W_true,l x_S + c_l + noise_scale * e; e is N(0,1), or Student-t(noise_dof)."""
    xS = rng(seed, TAG_CAL_X).standard_normal((rows, d), dtype=np.float32) + np.float32(x_shift)
    xl = np.empty((n_layers, rows, d), dtype=np.float32)
    for l in range(n_layers):
        U, V = true_map_factors(d, seed, l)
        c = rng(seed, TAG_CAL_C, l).standard_normal(d, dtype=np.float32)
        gn = rng(seed, TAG_CAL_NOISE, l)
        e = (gn.standard_t(noise_dof, size=(rows, d)) if noise_dof
             else gn.standard_normal((rows, d)))
        xl[l] = xS + TRUE_MAP_GAIN * ((xS @ V) @ U.T) + c[None, :] + noise_scale * e
    return xS, xl


def sylvester_hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), entries +-1 (int8)."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    H = np.ones((1, 1), dtype=np.int8)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def sparse_dyadic_matrix(d_out: int, d_in: int, seed: int, per_row: int = 2) -> np.ndarray:
    """d_out x d_in matrix with at most `per_row` nonzeros per row, each in
    {+-1, +-1/2}: every product and sum with +-1 data is exact in bf16/fp32."""
    g = rng(seed, 99)
    W = np.zeros((d_out, d_in), dtype=np.float32)
    vals = np.array([1.0, -1.0, 0.5, -0.5], dtype=np.float32)
    for o in range(d_out):
        cols = g.choice(d_in, size=per_row, replace=False)
        W[o, cols] = g.choice(vals, size=per_row)
    return W


# --------------------------------------------------------------------------- on the GPU
# Large workloads are drawn on the device with torch's seeded generator (same recipes).

def device_fill_inputs(cfg, dev, maps=None, sentinel: bool = False):
    """Seeded fill inputs on `dev` for a FillConfig: x_S bf16 [N, d_in]; per upper layer A
    (bf16 [d, d_in], near-identity, [I | 0] plus the low-rank term when d_in > d, unless
    `maps` gives (A bf16, b fp32) pairs), b fp32, norm_w, W_K,
    W_V (bf16) and K/V page pools (zeros, or 0xFFFF everywhere when `sentinel`); the block
    table; the exact-row mask."""
    import torch

    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    d, kv = cfg.d, cfg.kv
    width = getattr(cfg, "width", d)
    xS = torch.randn((cfg.N, width), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    table_np, num_pages = block_table(cfg.N, cfg.page_size, cfg.seed)
    s = 1.0 / np.sqrt(d)
    layers = []
    for l in range(cfg.n_upper):
        if maps is not None:
            A, b = maps[l]
        else:
            U = torch.randn((d, TRUE_MAP_RANK), generator=g, device=dev) * s
            V = torch.randn((width, TRUE_MAP_RANK), generator=g, device=dev) / np.sqrt(width)
            A = (torch.eye(d, width, device=dev) + TRUE_MAP_GAIN * (U @ V.T)).to(torch.bfloat16)
            b = torch.randn(d, generator=g, device=dev)
            del U, V
        w = (1.0 + 0.1 * torch.randn(d, generator=g, device=dev)).to(torch.bfloat16)
        WK = (torch.randn((kv, d), generator=g, device=dev) * s).to(torch.bfloat16)
        WV = (torch.randn((kv, d), generator=g, device=dev) * s).to(torch.bfloat16)
        shape = (num_pages, cfg.page_size, cfg.n_kv, cfg.head_dim)
        pools = []
        for _ in range(2):
            t = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
            if sentinel:
                t.view(torch.int16).fill_(-1)
            pools.append(t)
        layers.append(dict(A=A.contiguous(), b=b.float().contiguous(), norm_w=w, W_K=WK, W_V=WV,
                           k_pages=pools[0], v_pages=pools[1]))
    return dict(xS=xS, table=torch.from_numpy(table_np).to(dev), table_np=table_np,
                num_pages=num_pages, layers=layers, exact_mask=exact_mask(cfg))


def device_calib_chunks(ccfg, dev):
    """Seeded calibration rows on `dev`, chunk by chunk: x_l = W_true,l x_S + c_l + s * e with
    W_true,l = I + U_l diag(0.5) V_l^T (rank 64) and e Student-t(dof) built from normals
    (z / sqrt(chi^2_dof / dof)).  Returns [(x_S bf16 [n, d], [x_l bf16 [n, d]] * L)]."""
    import torch

    g = torch.Generator(device=dev)
    g.manual_seed(ccfg.seed)
    d, L = ccfg.d, ccfg.n_layers
    s = 1.0 / np.sqrt(d)
    dof = int(ccfg.noise_dof)
    U = [torch.randn((d, TRUE_MAP_RANK), generator=g, device=dev) * s for _ in range(L)]
    V = [torch.randn((d, TRUE_MAP_RANK), generator=g, device=dev) * s for _ in range(L)]
    c = [torch.randn(d, generator=g, device=dev) for _ in range(L)]
    chunks = []
    for r0 in range(0, ccfg.rows, ccfg.chunk):
        n = min(ccfg.chunk, ccfg.rows - r0)
        xs = torch.randn((n, d), generator=g, device=dev)
        xl = []
        for l in range(L):
            z = torch.randn((n, d), generator=g, device=dev)
            chi = sum(torch.randn((n, d), generator=g, device=dev) ** 2 for _ in range(dof))
            e = z / torch.sqrt(chi / dof)
            y = xs + TRUE_MAP_GAIN * ((xs @ V[l]) @ U[l].T) + c[l] + ccfg.noise_scale * e
            xl.append(y.to(torch.bfloat16))
            del z, chi, e, y
        chunks.append((xs.to(torch.bfloat16), xl))
    return chunks


def device_hadamard_columns(rows: int, cols: int, dev, first_col: int = 1):
    """Columns first_col .. first_col + cols - 1 of the Sylvester Hadamard matrix of order
    2^k >= rows (entry (r, c) = (-1)^popcount(r & c)), rows 0 .. rows-1, float32 on `dev`."""
    import torch

    r = torch.arange(rows, device=dev, dtype=torch.int64)[:, None]
    c = torch.arange(first_col, first_col + cols, device=dev, dtype=torch.int64)[None, :]
    v = r & c
    par = torch.zeros_like(v)
    while bool((v != 0).any()):
        par ^= v & 1
        v = v >> 1
    return (1 - 2 * par).to(torch.float32)


def rect_map(d_out: int, d_in: int, seed: int, layer: int):
    """A = [I | 0] + U V^T / 2 (float32 [d_out, d_in]) and b ~ N(0, 1) (float32 [d_out])."""
    U = rng(seed, TAG_MAPU, layer).standard_normal((d_out, TRUE_MAP_RANK), dtype=np.float32)
    V = rng(seed, TAG_MAPV, layer).standard_normal((d_in, TRUE_MAP_RANK), dtype=np.float32)
    A = (U / np.sqrt(d_out)) @ (V / np.sqrt(d_in)).T * np.float32(TRUE_MAP_GAIN)
    A[:, :min(d_out, d_in)] += np.eye(d_out, min(d_out, d_in), dtype=np.float32)
    b = rng(seed, TAG_MAPB, layer).standard_normal(d_out, dtype=np.float32)
    return A.astype(np.float32), b.astype(np.float32)


def key_norm_weight(hd: int, seed: int, layer: int) -> np.ndarray:
    """1 + 0.1 N(0, 1), float32 [hd]."""
    return (1.0 + 0.1 * rng(seed, TAG_KNORM, layer).standard_normal(hd)).astype(np.float32)


def value_factors(n_kv: int, seed: int, layer: int) -> np.ndarray:
    """U[0.5, 1.5], float32 [n_kv]."""
    return rng(seed, TAG_VSCALE, layer).uniform(0.5, 1.5, n_kv).astype(np.float32)


def exact_tail_inputs(xS_tail: np.ndarray, d: int, seed: int, layer: int) -> np.ndarray:
    """x_l of the near-identity model on the given split-layer rows (float32 [c, d])."""
    U, V = true_map_factors(d, seed, layer)
    c = rng(seed, TAG_CAL_C, layer).standard_normal(d, dtype=np.float32)
    e = rng(seed, TAG_CAL_NOISE, layer).standard_normal(xS_tail.shape, dtype=np.float32)
    return (xS_tail + TRUE_MAP_GAIN * ((xS_tail @ V) @ U.T) + c[None, :] + 0.1 * e).astype(np.float32)


def row_scores(P: int, seed: int) -> np.ndarray:
    """Exp(1) draws rounded to multiples of 1/64 (ties occur), float32 [P]."""
    s = rng(seed, TAG_SCORES).exponential(1.0, P)
    return (np.round(s * 64.0) / 64.0).astype(np.float32)



# --------------------------------------------------------------------- harder inputs
# Inputs that stress the numerics rather than stand in for the timing workloads: feature
# magnitudes far apart, feature means far larger than the spread, spectra spread over
# several decades.

def spread_map(d: int, seed: int, layer: int, spread: float) -> np.ndarray:
    """A = (D1 H) diag(s) (H D2) / d (float32 [d, d]): H the Sylvester Hadamard matrix of
    order d (a power of two), D1, D2 seeded random signs, so the singular values are
    exactly s, log-spaced from 1 down to 1/spread and scaled to a root-mean-square of 1."""
    H = sylvester_hadamard(d).astype(np.float32)
    g = rng(seed, TAG_SPREAD, layer)
    s = np.logspace(0.0, -np.log10(spread), d).astype(np.float32)
    s /= np.sqrt(np.mean(s.astype(np.float64) ** 2)).astype(np.float32)
    d1 = g.choice(np.array([-1.0, 1.0], dtype=np.float32), size=d)
    d2 = g.choice(np.array([-1.0, 1.0], dtype=np.float32), size=d)
    left = (d1[:, None] * H) * s[None, :]
    return ((left @ (H * d2[None, :])) / np.float32(d)).astype(np.float32)


def calib_data_hard(d: int, n_layers: int, rows: int, seed: int, *, mean_lo: float = 10.0,
                    mean_hi: float = 50.0, spread: float = 1.0, noise_scale: float = 0.1):
    """Calibration rows whose statistics are hard to keep in fp32 or to invert:
    x_S = z diag(sd) Q^T + m, z ~ N(0,1), Q a seeded orthogonal matrix (when spread > 1),
    sd log-spaced so that the covariance's eigenvalues span `spread`, and on a seeded half
    of the features a mean m of magnitude U[mean_lo, mean_hi] times the unit spread with a
    random sign; x_l = W_true,l x_S + c_l + noise_scale e with c_l of the same magnitudes
    on a seeded half of the outputs.  float32 x_S [rows, d], x_l [n_layers, rows, d]."""
    g = rng(seed, TAG_HARD)
    z = g.standard_normal((rows, d))
    if spread > 1.0:
        sd = np.logspace(0.0, 0.5 * np.log10(spread), d)
        Q, _ = np.linalg.qr(g.standard_normal((d, d)))
        z = (z * sd[None, :]) @ Q.T
    m = np.where(g.random(d) < 0.5, g.uniform(mean_lo, mean_hi, d) * g.choice([-1.0, 1.0], d), 0.0)
    xS = (z + m[None, :]).astype(np.float32)
    xl = np.empty((n_layers, rows, d), dtype=np.float32)
    for l in range(n_layers):
        U, V = true_map_factors(d, seed, l)
        gl = rng(seed, TAG_HARD, 1 + l)
        c = np.where(gl.random(d) < 0.5, gl.uniform(mean_lo, mean_hi, d) * gl.choice([-1.0, 1.0], d),
                     gl.standard_normal(d))
        e = gl.standard_normal((rows, d))
        xl[l] = xS + TRUE_MAP_GAIN * ((xS @ V) @ U.T) + c[None, :].astype(np.float32) + noise_scale * e
    return xS, xl
