"""Plain, slow, float64 CPU oracle for RidgeFill's upper-layer KV fill, its one-pass
calibration and its closed-form ridge solve.

TEST INFRASTRUCTURE ONLY.  The test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (the HIP library and its
Python binding) never imports or runs anything here, and nothing here imports or
runs the product path.  This module shares no code, tables or constants with it.

Every step is written from the method's definition, in the order and notation of the
English RidgeFill review (jaehun.me, "paper-2611-09709v1", English edition), and cited
by its section:

  [split]  "Method: predict the late layers' inputs ..." -> "Two numbers set the skip range"
  [map]    "Ridge map: predict the input, and the original projection runs unchanged",
           the prediction equation  x_hat_l = A_l x_S + b_l
  [obj]    same section, the ridge objective
  [closed] same section, the closed-form solution after subtracting the means
  [alpha]  same section, alpha = lambda * tr(X^T X) / d_in and the one-pass statistics
  [own]    same section, the paragraph on feeding the predicted input to the
           layer's norm and K/V projections, and Fig. 2
  [arms]   "Tables from the paper", Table 3 (exact / no fill / identity / RidgeFill)
  [notation] "Tables from the paper", Table 2
  [size]   same section as [map], the paragraph on map size (int8 maps, maps whose input
           width differs from their output width, resident or streamed maps)
  [rescale] "Hybrid layers and two corrections", the value-rescale paragraph
  [qknorm] same paragraph (the Qwen models apply a norm to the keys) and "Experiments",
           the error attribution paragraph on key normalization
  [select] "Which rows to compute exactly", attention selection
  [fold]   [map] and [own] taken together: the folded form of one layer (the norm weight
           and the K/V projections multiplied into the map, the prediction's sum of
           squares as a triangular quadratic form).  This is an exact rearrangement of
           the same arithmetic, not a step the page describes; fill_rows_folded must
           agree with fill_rows to float64 rounding.

Readings of points the page leaves open (each is listed with its reason in the design
notes of the repository):
  * x_S is the input to layer S; the upper layers are l = S .. L-1 and each has its own
    map, the one at l = S included.
  * the layer's normalization, whose type the page does not name, is RMSNorm with a multiplicative weight w and an
    epsilon eps:  y = x / sqrt(mean(x^2) + eps) * w.
  * The key/value projections have no bias; head h owns columns [h*hd, (h+1)*hd).
  * RoPE is applied to the keys only, rotate-half pairing (j, j + hd/2), inverse
    frequency theta^(-2j/hd), position = absolute prompt index t (0-based), angles in
    float64.
  * The calibration accumulates raw sums and raw second moments in one pass and centres
    them at solve time; the trace in alpha is that of the centred X^T X; d_in = d.
  * The statistic kept per layer is Y_l^T X (d_out x d_in), the factor that appears in
    the closed form.
  * Key normalization (Qwen-style layers) is an RMSNorm over each key head's hd entries
    with its own weight [hd], after the key projection and before RoPE; it uses the
    same eps as the layer norm.
  * Value rescale: "magnitude" is the Euclidean norm of one KV head's value vector; the
    exact and predicted values both go through the layer's RMSNorm and W_V; the scale
    of head h is the plain mean over the c rows of |v_exact| / |v_pred|, and it
    multiplies head h of every filled row's value.
  * int8 maps: symmetric, one scale per output row (max |A| / 127, round half to
    even, clip to [-127, 127]); the map used is q * scale.
  * Selection from scores: the k prefix rows with the largest score, ties to the lower
    index; the attention-selected arm uses k = round(0.1 * P).

Parity status: every function below is pinned by the CPU tests in tests/test_oracle_*.py
(closed forms, library routines that solve the same problem another way, invariants,
special cases and brute force).  No function is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "upper_layers",
    "partition",
    "predict_input",
    "rms_norm",
    "rope_inv_freq",
    "rope_keys",
    "project_kv",
    "fill_rows",
    "key_norm",
    "value_scale",
    "quantize_map_int8",
    "dequantize_map_int8",
    "select_exact",
    "fold_map",
    "fill_rows_folded",
    "paged_location",
    "fill_paged_cache",
    "CalibStats",
    "calib_new",
    "calib_accumulate",
    "centred_moments",
    "ridge_alpha",
    "solve",
    "fit_direct",
    "ridge_objective",
    "prefill_compute_fraction",
]


# --------------------------------------------------------------------------- [split]

def upper_layers(S: int, L: int) -> list[int]:
    """Layers whose cache a filled row receives from its map: l = S, ..., L-1.

    [split]: every row runs the layers below S as usual; the map predicts the input of
    every upper layer l >= S from x_S (one map per upper layer, [map]).
    """
    if not (0 <= S <= L):
        raise ValueError(f"need 0 <= S <= L, got S={S}, L={L}")
    return list(range(S, L))


def partition(N: int, T: int, exact_rows):
    """Split a prompt of N rows into (filled, exact, tail), each an ascending int64 array.

    [split]: the last T rows are the tail and run every layer; the N - T rows before
    them form the prefix, and above the split each prefix row is exact (computed as
    usual) or filled (its cache comes from the map).  Exact rows must lie in the prefix and must
    not repeat.
    """
    N = int(N)
    T = int(T)
    if N < 0 or T < 0 or T > N:
        raise ValueError(f"need 0 <= T <= N, got N={N}, T={T}")
    P = N - T
    exact_list = [int(e) for e in exact_rows]
    exact_set = set(exact_list)
    if len(exact_set) != len(exact_list):
        raise ValueError("exact rows repeat")
    for e in exact_list:
        if e < 0 or e >= P:
            raise ValueError(f"exact row {e} is not in the prefix [0, {P})")
    filled = [t for t in range(P) if t not in exact_set]
    exact = sorted(exact_set)
    tail = list(range(P, N))
    assert len(filled) + len(exact) + len(tail) == N
    return (np.asarray(filled, dtype=np.int64),
            np.asarray(exact, dtype=np.int64),
            np.asarray(tail, dtype=np.int64))


def prefill_compute_fraction(S: int, L: int, N: int, T: int) -> float:
    """Share r of exact-prefill layer passes that remain: prefix rows pass S layers,
    tail rows pass L layers, so r = (S (N-T) + L T) / (L N).

    Section "Results: speed" -> "The compute bound and measured values differ".  Used
    by a test to pin the prefix/tail counting of `partition` against the bounds the
    page prints for its second deployment.
    """
    _, _, tail = partition(N, T, [])
    prefix = N - len(tail)
    return (S * prefix + L * len(tail)) / (L * N)


# --------------------------------------------------------------------------- [map]

def predict_input(x_S: np.ndarray, A: np.ndarray, b: np.ndarray) -> np.ndarray:
    """x_hat = A x_S + b for every row of x_S ([map]); A is d_out x d_in, rows are tokens."""
    x_S = np.asarray(x_S, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return x_S @ A.T + b[None, :]


# --------------------------------------------------------------------------- [own]

def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Each row divided by its root mean square (with eps inside the root), then scaled
    elementwise by the layer's norm weight w ([own]: the layer's own normalization)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * w


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Inverse frequency of pair j: theta^(-2j/head_dim), j = 0 .. head_dim/2 - 1."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * j / head_dim)


def rope_keys(k: np.ndarray, positions, theta: float) -> np.ndarray:
    """Rotate each key head: pair (j, j + hd/2) of row t turns by angle t * inv_freq_j.

    k has shape [rows, heads, hd]; positions has one absolute prompt index per row.
    """
    k = np.asarray(k, dtype=np.float64)
    hd = k.shape[-1]
    half = hd // 2
    pos = np.asarray(positions, dtype=np.float64)
    ang = pos[:, None] * rope_inv_freq(hd, theta)[None, :]      # [rows, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    lo = k[..., :half]
    hi = k[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def project_kv(h: np.ndarray, W_K: np.ndarray, W_V: np.ndarray, n_kv: int, hd: int):
    """The layer's unchanged key and value projections ([own]); no bias.
    Returns K, V with shape [rows, n_kv, hd]."""
    h = np.asarray(h, dtype=np.float64)
    K = h @ np.asarray(W_K, dtype=np.float64).T
    V = h @ np.asarray(W_V, dtype=np.float64).T
    rows = h.shape[0]
    return K.reshape(rows, n_kv, hd), V.reshape(rows, n_kv, hd)


def key_norm(K: np.ndarray, k_norm_w: np.ndarray, eps: float) -> np.ndarray:
    """Per-head key normalization ([qknorm]): each key head's hd entries divided by their
    root mean square (eps inside the root), then scaled by the head weight k_norm_w [hd].
    K has shape [rows, heads, hd]."""
    return rms_norm(K, k_norm_w, eps)


def fill_rows(x_S_rows, positions, A, b, norm_w, W_K, W_V, *, eps, theta, n_kv, hd,
              k_norm_w=None, v_scale=None):
    """Cache entries of one upper layer for the given filled rows (Fig. 2 flow):
    predicted input -> the layer's RMSNorm -> K and V projections -> (key norm) -> RoPE
    on K; V times the per-head value-rescale factors when given ([rescale]).

    x_S_rows: [rows, d_in] split-layer states of the filled rows; positions: their prompt
    indices; A is d_out x d_in.  Returns (K, V), each [rows, n_kv, hd] in float64.
    """
    x_hat = predict_input(x_S_rows, A, b)
    h = rms_norm(x_hat, norm_w, eps)
    K, V = project_kv(h, W_K, W_V, n_kv, hd)
    if k_norm_w is not None:
        K = key_norm(K, k_norm_w, eps)
    K = rope_keys(K, positions, theta)
    if v_scale is not None:
        V = V * np.asarray(v_scale, dtype=np.float64)[None, :, None]
    return K, V


# --------------------------------------------------------------------------- [rescale]

def value_scale(x_S_tail, x_l_exact_tail, A, b, norm_w, W_V, *, eps, n_kv, hd):
    """Per-KV-head value-rescale factors of one upper layer ([rescale]).

    The values of the first c tail rows are computed twice: from their true layer input
    x_l (x_l_exact_tail, [c, d_out]) and from the map's prediction out of their
    split-layer state (x_S_tail, [c, d_in]).  For head h the factor is the
    mean over the c rows of |v_exact[h]| / |v_pred[h]|.  Returns [n_kv] float64.
    """
    W_V = np.asarray(W_V, dtype=np.float64)
    v_ex = (rms_norm(x_l_exact_tail, norm_w, eps) @ W_V.T).reshape(-1, n_kv, hd)
    x_hat = predict_input(x_S_tail, A, b)
    v_pr = (rms_norm(x_hat, norm_w, eps) @ W_V.T).reshape(-1, n_kv, hd)
    ratio = np.linalg.norm(v_ex, axis=-1) / np.linalg.norm(v_pr, axis=-1)
    return ratio.mean(axis=0)


# --------------------------------------------------------------------------- [size]

def quantize_map_int8(A: np.ndarray, dtype=np.float64):
    """Symmetric int8 map with one scale per output row: scale = max_k |A[o, k]| / 127,
    q = round-half-even(A / scale) clipped to [-127, 127] (an all-zero row gets scale 0
    and q = 0).  The arithmetic runs in `dtype` (float32 to take the same rounding
    decisions as a float32 quantizer).  Returns (q int8 [d_out, d_in], scale [d_out])."""
    A = np.asarray(A).astype(dtype)
    amax = np.max(np.abs(A), axis=1)
    scale = (amax / dtype(127.0)).astype(dtype)
    safe = np.where(scale > 0, scale, dtype(1.0)).astype(dtype)
    q = np.clip(np.rint((A / safe[:, None]).astype(dtype)), -127, 127)
    q[scale == 0] = 0
    return q.astype(np.int8), scale


def dequantize_map_int8(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """The map an int8 map stands for: q[o, k] * scale[o], in float64."""
    return np.asarray(q, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[:, None]


# --------------------------------------------------------------------------- [fold]

def fold_map(A, b, norm_w, W_K, W_V):
    """Folded form of one upper layer ([fold]).  In the plain flow x_hat = A x + b,
    h = x_hat / sqrt(mean(x_hat^2) + eps) * w, k = W_K h, v = W_V h ([map], [own]), the
    weight w and the projections are linear and the only non-linear quantity is the
    scalar |x_hat|^2.  With

        P     = [W_K; W_V] diag(w) A                         [2 kv, d_in]
        c     = [W_K; W_V] (w * b)                           [2 kv]
        R     = the upper-triangular factor of A^T A with a positive diagonal
                (R^T R = A^T A: the transpose of its Cholesky factor)
        r     = R^-T A^T b                                   [d_in]
        kappa = |b|^2 - |r|^2

    every x has [W_K; W_V] diag(w) x_hat = P x + c, and |x_hat|^2 = |R x + r|^2 + kappa,
    because |R x + r|^2 = x^T A^T A x + 2 b^T A x + |r|^2.  kappa is the squared distance
    from b to the column space of A (zero when A is square and invertible).  A^T A must
    be positive definite (A of full column rank: d_in <= d_out); otherwise numpy's
    Cholesky raises LinAlgError.  Returns (P, c, R, r, kappa) in float64.
    """
    A = np.asarray(A, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    w = np.asarray(norm_w, dtype=np.float64)
    W = np.concatenate([np.asarray(W_K, dtype=np.float64), np.asarray(W_V, dtype=np.float64)])
    Ww = W * w[None, :]
    P = Ww @ A
    c = Ww @ b
    L = np.linalg.cholesky(A.T @ A)          # lower, A^T A = L L^T
    R = L.T
    r = np.linalg.solve(L, A.T @ b)          # R^T r = A^T b, R^T = L
    kappa = float(b @ b - r @ r)
    return P, c, R, r, kappa


def fill_rows_folded(x_S_rows, positions, P, c, R, r, kappa, d, *, eps, theta, n_kv, hd,
                     k_norm_w=None, v_scale=None):
    """The cache entries of fill_rows computed from the folded form of fold_map ([fold]):
    mean(x_hat^2) = (|R x + r|^2 + kappa) / d with d the map's output width, then
    [k; v] = (P x + c) / sqrt(mean(x_hat^2) + eps), followed by the same key norm, RoPE
    and value rescale as fill_rows.  Returns (K, V), each [rows, n_kv, hd] in float64."""
    x = np.asarray(x_S_rows, dtype=np.float64)
    u = x @ np.asarray(R, dtype=np.float64).T + np.asarray(r, dtype=np.float64)[None, :]
    ms = (np.sum(u * u, axis=1) + float(kappa)) / float(d)
    kvp = (x @ np.asarray(P, dtype=np.float64).T + np.asarray(c, dtype=np.float64)[None, :])
    kvp = kvp / np.sqrt(ms + float(eps))[:, None]
    kv = n_kv * hd
    rows = x.shape[0]
    K = kvp[:, :kv].reshape(rows, n_kv, hd)
    V = kvp[:, kv:].reshape(rows, n_kv, hd)
    if k_norm_w is not None:
        K = key_norm(K, k_norm_w, eps)
    K = rope_keys(K, positions, theta)
    if v_scale is not None:
        V = V * np.asarray(v_scale, dtype=np.float64)[None, :, None]
    return K, V


# --------------------------------------------------------------------------- [select]

def select_exact(scores, k: int) -> np.ndarray:
    """The k prefix rows with the largest score, ties broken toward the lower row index
    ([select]); returned in ascending row order.  scores: one value per prefix row."""
    sc = np.asarray(scores, dtype=np.float64)
    P = sc.shape[0]
    if not 0 <= k <= P:
        raise ValueError("need 0 <= k <= P")
    order = sorted(range(P), key=lambda i: (-sc[i], i))
    return np.sort(np.asarray(order[:k], dtype=np.int64))


def paged_location(t, block_table, page_size: int):
    """(physical page, slot) that holds prompt row t in a paged cache: logical page
    t // page_size is looked up in the block table; the slot is t % page_size."""
    t = np.asarray(t, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    return bt[t // page_size], t % page_size


def fill_paged_cache(k_cache, v_cache, x_S, filled, layer, *, block_table, page_size,
                     eps, theta, n_kv, hd):
    """Write one upper layer's filled rows into its paged K and V caches, in place.

    k_cache, v_cache: float arrays [num_pages, page_size, n_kv, hd]; every entry that is
    not a filled row is left untouched ([arms]: exact rows and the tail get their cache
    elsewhere, and with no filled rows the cache is unchanged).
    layer: dict with keys A, b, norm_w, W_K, W_V.
    """
    filled = np.asarray(filled, dtype=np.int64)
    if filled.size == 0:
        return k_cache, v_cache
    xs = np.asarray(x_S, dtype=np.float64)[filled]
    K, V = fill_rows(xs, filled, layer["A"], layer["b"], layer["norm_w"],
                     layer["W_K"], layer["W_V"], eps=eps, theta=theta, n_kv=n_kv, hd=hd)
    page, slot = paged_location(filled, block_table, page_size)
    k_cache[page, slot] = K
    v_cache[page, slot] = V
    return k_cache, v_cache


# --------------------------------------------------------------------------- [alpha]

class CalibStats:
    """One-pass sufficient statistics for one split ([alpha]): the row count n, the sums
    of x_S and of every x_l, the raw second moment sum_t x_S x_S^T and, per upper layer,
    the raw cross moment sum_t x_l x_S^T (= Y_l^T X before centring, d_out x d_in)."""

    def __init__(self, d: int, n_layers: int, d_out: int | None = None):
        self.d = int(d)                          # d_in: width of x_S
        self.d_out = int(d_out) if d_out else self.d
        self.n_layers = int(n_layers)
        self.n = 0
        self.s_S = np.zeros(self.d, dtype=np.float64)
        self.s_l = np.zeros((n_layers, self.d_out), dtype=np.float64)
        self.G = np.zeros((self.d, self.d), dtype=np.float64)
        self.YX = np.zeros((n_layers, self.d_out, self.d), dtype=np.float64)


def calib_new(d: int, n_layers: int, d_out: int | None = None) -> CalibStats:
    """Empty statistics for x_S of width d (= d_in) and layer inputs of width d_out
    (default d; [size]: a map's input width may differ from its output width)."""
    return CalibStats(d, n_layers, d_out)


def calib_accumulate(st: CalibStats, x_S_chunk, x_l_chunks) -> CalibStats:
    """Add one chunk of calibration rows: x_S_chunk [n_c, d_in] and one [n_c, d_out] array
    per upper layer.  Only sums and moments are kept, so a new lambda needs no re-read."""
    X = np.asarray(x_S_chunk, dtype=np.float64)
    if len(x_l_chunks) != st.n_layers:
        raise ValueError("one chunk per upper layer is required")
    st.n += X.shape[0]
    st.s_S += X.sum(axis=0)
    st.G += X.T @ X
    for l, Y in enumerate(x_l_chunks):
        Y = np.asarray(Y, dtype=np.float64)
        if Y.shape != (X.shape[0], st.d_out):
            raise ValueError("x_l chunk must be [rows of x_S, d_out]")
        st.s_l[l] += Y.sum(axis=0)
        st.YX[l] += Y.T @ X
    return st


def centred_moments(st: CalibStats):
    """Means and the centred X^T X and Y_l^T X ([closed]: X and Y_l are stacked after
    subtracting mu_S and mu_l), from the raw one-pass sums."""
    n = float(st.n)
    if n <= 0:
        raise ValueError("no calibration rows")
    mu_S = st.s_S / n
    mu_l = st.s_l / n
    XtX = st.G - n * np.outer(mu_S, mu_S)
    YtX = st.YX - n * mu_l[:, :, None] * mu_S[None, None, :]
    return mu_S, mu_l, XtX, YtX


def ridge_alpha(XtX: np.ndarray, lam: float) -> float:
    """alpha = lambda * tr(X^T X) / d_in ([alpha])."""
    return float(lam) * float(np.trace(XtX)) / XtX.shape[0]


def solve(st: CalibStats, lam: float):
    """Closed-form ridge maps for every upper layer ([closed], [alpha]):
    A_l = Y_l^T X (X^T X + alpha I)^-1,  b_l = mu_l - A_l mu_S.

    (X^T X + alpha I) is factored by Cholesky; A_l^T is found from
    (X^T X + alpha I) A_l^T = (Y_l^T X)^T by two triangular solves.
    Returns (A [n_layers, d_out, d_in], b [n_layers, d_out]) in float64.
    """
    import scipy.linalg as sla

    if lam < 0:
        raise ValueError("lambda must be >= 0")
    mu_S, mu_l, XtX, YtX = centred_moments(st)
    d = XtX.shape[0]
    alpha = ridge_alpha(XtX, lam)
    M = XtX + alpha * np.eye(d)
    c_low = sla.cho_factor(M, lower=True)
    A = np.empty_like(YtX)
    for l in range(st.n_layers):
        A[l] = sla.cho_solve(c_low, YtX[l].T).T
    b = mu_l - np.einsum("lij,j->li", A, mu_S)
    return A, b


def fit_direct(x_S, x_l, lam: float):
    """The same fit written straight from its definition for one layer: subtract the
    means, stack the rows as X and Y, and apply the closed form ([closed], [alpha])."""
    Xr = np.asarray(x_S, dtype=np.float64)
    Yr = np.asarray(x_l, dtype=np.float64)
    mu_S = Xr.mean(axis=0)
    mu_l = Yr.mean(axis=0)
    X = Xr - mu_S
    Y = Yr - mu_l
    XtX = X.T @ X
    alpha = ridge_alpha(XtX, lam)
    A = (Y.T @ X) @ np.linalg.inv(XtX + alpha * np.eye(XtX.shape[0]))
    b = mu_l - A @ mu_S
    return A, b


def ridge_objective(x_S, x_l, A, b, alpha: float) -> float:
    """sum_t ||x_l,t - (A x_S,t + b)||^2 + alpha ||A||_F^2 ([obj])."""
    R = np.asarray(x_l, dtype=np.float64) - predict_input(x_S, A, b)
    return float(np.sum(R * R) + alpha * np.sum(np.asarray(A, dtype=np.float64) ** 2))
