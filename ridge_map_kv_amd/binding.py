"""Thin ctypes binding of libridgefill.so (C ABI in include/ridgefill.h).

Argument marshalling only: every step of the fill, calibration and solve runs in the
HIP library.  torch tensors supply device memory and the current stream.  There is no
fallback: if the library is missing, `lib()` raises.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libridgefill.so")

RF_OK, RF_E_INVALID, RF_E_SHAPE, RF_E_WORKSPACE, RF_E_HIP, RF_E_NOT_SPD, RF_E_ROWS, \
    RF_E_UNSUPPORTED = range(8)

EXPORTED = [
    "ridgefill_partition",
    "ridgefill_fill_workspace_bytes",
    "ridgefill_fill_workspace_bytes_ex",
    "ridgefill_fill",
    "ridgefill_fill_streamed",
    "ridgefill_fill_noalloc",
    "ridgefill_value_scale_workspace_bytes",
    "ridgefill_value_scale",
    "ridgefill_quantize_map",
    "ridgefill_fold_bytes",
    "ridgefill_fold_workspace_bytes",
    "ridgefill_fold_workspace_bytes_ex",
    "ridgefill_fold_workspace_bytes_maps",
    "ridgefill_fold_maps",
    "ridgefill_select_workspace_bytes",
    "ridgefill_select_rows",
    "ridgefill_calib_state_bytes",
    "ridgefill_calib_reset",
    "ridgefill_calibrate",
    "ridgefill_calib_state_bytes_ex",
    "ridgefill_calib_reset_ex",
    "ridgefill_calibrate_ex",
    "ridgefill_solve_workspace_bytes",
    "ridgefill_solve",
    "ridgefill_solve_workspace_bytes_ex",
    "ridgefill_solve_ex",
    "ridgefill_read_status",
    "ridgefill_solve_info",
    "ridgefill_profile_enable",
    "ridgefill_profile_read",
    "ridgefill_profile_reset",
    "ridgefill_status_string",
    "ridgefill_last_error",
]


class RidgeFillError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"ridgefill status {status}: {msg}")
        self.status = status


RF_MAPS_INT8 = 1
RF_MAPS_STREAMED = 2
RF_MAPS_FOLDED = 4


class rf_shape(C.Structure):
    _fields_ = [("d", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("rms_eps", C.c_float), ("rope_theta", C.c_double), ("d_in", C.c_int32),
                ("reserved", C.c_int32)]


class rf_layer(C.Structure):
    _fields_ = [("A", C.c_void_p), ("b", C.c_void_p), ("norm_w", C.c_void_p),
                ("W_K", C.c_void_p), ("W_V", C.c_void_p), ("k_pages", C.c_void_p),
                ("v_pages", C.c_void_p), ("k_norm_w", C.c_void_p), ("v_scale", C.c_void_p),
                ("A_q", C.c_void_p), ("A_scale", C.c_void_p), ("folded", C.c_void_p)]


class rf_paged_kv(C.Structure):
    _fields_ = [("block_table", C.c_void_p), ("n_logical", C.c_int64),
                ("page_size", C.c_int32), ("num_pages", C.c_int32)]


_lib = None


def lib() -> C.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m ridge_map_kv_amd.build` (there is no CPU fallback)")
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    st = C.c_int
    sig = {
        "ridgefill_partition": (st, [i64, i64, vp, vp, C.POINTER(i64)]),
        "ridgefill_fill_workspace_bytes": (sz, [C.POINTER(rf_shape), i64, i32]),
        "ridgefill_fill_workspace_bytes_ex": (sz, [C.POINTER(rf_shape), i64, i32, i32]),
        "ridgefill_fill": (st, [C.POINTER(rf_shape), vp, i64, i64, i64, vp, i64,
                                C.POINTER(rf_layer), i32, C.POINTER(rf_paged_kv), vp, sz, vp]),
        "ridgefill_fill_streamed": (st, [C.POINTER(rf_shape), vp, i64, i64, i64, vp, i64,
                                         C.POINTER(rf_layer), i32, C.POINTER(rf_paged_kv), vp,
                                         sz, vp, vp]),
        "ridgefill_fill_noalloc": (st, [C.POINTER(rf_shape), vp, i64, i64, i64, vp, i64,
                                        C.POINTER(rf_layer), i32, C.POINTER(rf_paged_kv), vp, vp]),
        "ridgefill_value_scale_workspace_bytes": (sz, [C.POINTER(rf_shape), i64, i32, i32]),
        "ridgefill_value_scale": (st, [C.POINTER(rf_shape), vp, i64, C.POINTER(vp), i64,
                                       C.POINTER(rf_layer), i32, vp, vp, sz, vp]),
        "ridgefill_quantize_map": (st, [vp, i64, i64, vp, vp, vp]),
        "ridgefill_fold_bytes": (sz, [C.POINTER(rf_shape)]),
        "ridgefill_fold_workspace_bytes": (sz, [C.POINTER(rf_shape)]),
        "ridgefill_fold_workspace_bytes_ex": (sz, [C.POINTER(rf_shape), i32]),
        "ridgefill_fold_workspace_bytes_maps": (sz, [C.POINTER(rf_shape), i32, C.c_uint32]),
        "ridgefill_fold_maps": (st, [C.POINTER(rf_shape), C.POINTER(rf_layer), i32,
                                     C.POINTER(vp), vp, sz, vp]),
        "ridgefill_select_workspace_bytes": (sz, [i64]),
        "ridgefill_select_rows": (st, [vp, i64, i64, vp, vp, vp, sz, vp]),
        "ridgefill_calib_state_bytes": (sz, [i32, i32]),
        "ridgefill_calib_reset": (st, [vp, sz, i32, i32, vp]),
        "ridgefill_calibrate": (st, [vp, sz, i32, i32, vp, C.POINTER(vp), i64, vp]),
        "ridgefill_solve_workspace_bytes": (sz, [i32, i32]),
        "ridgefill_solve": (st, [vp, sz, i32, i32, C.c_double, vp, vp, vp, vp, sz, vp]),
        "ridgefill_calib_state_bytes_ex": (sz, [i32, i32, i32]),
        "ridgefill_calib_reset_ex": (st, [vp, sz, i32, i32, i32, vp]),
        "ridgefill_calibrate_ex": (st, [vp, sz, i32, i32, i32, vp, C.POINTER(vp), i64, vp]),
        "ridgefill_solve_workspace_bytes_ex": (sz, [i32, i32, i32]),
        "ridgefill_solve_ex": (st, [vp, sz, i32, i32, i32, C.c_double, vp, vp, vp, vp, sz, vp]),
        "ridgefill_read_status": (st, [vp, vp]),
        "ridgefill_solve_info": (st, [vp, C.POINTER(C.c_double), C.POINTER(i32), vp]),
        "ridgefill_profile_enable": (st, [i32]),
        "ridgefill_profile_read": (st, [i32, C.POINTER(i64), C.POINTER(C.c_double)]),
        "ridgefill_profile_reset": (st, []),
        "ridgefill_status_string": (C.c_char_p, [st]),
        "ridgefill_last_error": (C.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != RF_OK:
        msg = lib().ridgefill_last_error().decode() or lib().ridgefill_status_string(status).decode()
        raise RidgeFillError(status, msg)


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_shape(d: int, n_kv_heads: int, head_dim: int, rms_eps: float = 1e-5,
               rope_theta: float = 500000.0, d_in: int = 0) -> rf_shape:
    return rf_shape(d, n_kv_heads, head_dim, rms_eps, rope_theta, d_in, 0)


# ------------------------------------------------------------------------------ partition

def ridgefill_partition(N: int, T: int, exact_mask: np.ndarray | None) -> np.ndarray:
    """Host row partition; returns the filled rows (int32, ascending)."""
    P = max(int(N) - int(T), 0)
    out = np.zeros(max(P, 1), dtype=np.int32)
    n = C.c_int64(0)
    m = None
    if exact_mask is not None:
        exact_mask = np.ascontiguousarray(exact_mask, dtype=np.uint8)
        if exact_mask.size < P:
            raise ValueError("exact_mask shorter than the prefix")
        m = exact_mask.ctypes.data
    _check(lib().ridgefill_partition(int(N), int(T), m, out.ctypes.data, C.byref(n)))
    return out[: n.value].copy()


# ------------------------------------------------------------------------------ int8 maps

def ridgefill_quantize_map(A, A_q, A_scale, stream=None) -> None:
    """fp32 [rows][cols] map -> int8 codes A_q (same shape) and fp32 row scales A_scale."""
    _check(lib().ridgefill_quantize_map(_ptr(A), int(A.shape[0]), int(A.shape[1]), _ptr(A_q),
                                        _ptr(A_scale), _stream(stream)))


# ------------------------------------------------------------------------------ selection

def ridgefill_select_workspace_bytes(P: int) -> int:
    return int(lib().ridgefill_select_workspace_bytes(int(P)))


def ridgefill_select_rows(scores, k: int, filled_idx, ws, exact_mask=None, stream=None) -> None:
    """Top-k rows by score (ties to the lower index) -> exact_mask (optional, uint8 [P])
    and the remaining rows in ascending order -> filled_idx (int32 [P - k])."""
    _check(lib().ridgefill_select_rows(_ptr(scores), int(scores.numel()), int(k), _ptr(exact_mask),
                                       _ptr(filled_idx), _ptr(ws), _nbytes(ws), _stream(stream)))


# ------------------------------------------------------------------------------ fill

def ridgefill_fill_workspace_bytes(shape: rf_shape, n_filled: int, n_layers: int,
                                   map_flags: int = 0) -> int:
    return int(lib().ridgefill_fill_workspace_bytes_ex(C.byref(shape), int(n_filled),
                                                       int(n_layers), int(map_flags)))


def _layers(layers: list[dict]):
    """rf_layer array from dicts of torch tensors: A (bf16 [d][d_in]) or A_q (int8) with
    A_scale (fp32 [d]); b (fp32 [d]); norm_w (bf16 [d]); W_K, W_V (bf16 [kv][d]); k_pages,
    v_pages (bf16 [num_pages][page_size][n_kv][hd]); optional k_norm_w (bf16 [hd]) and
    v_scale (fp32 [n_kv]); or, for a folded layer, folded (uint8 device buffer made by
    ridgefill_fold_maps) with the pages and the optional parts."""
    arr = (rf_layer * max(len(layers), 1))()
    for i, l in enumerate(layers):
        g = l.get
        arr[i] = rf_layer(_ptr(g("A")), _ptr(g("b")), _ptr(g("norm_w")), _ptr(g("W_K")),
                          _ptr(g("W_V")), _ptr(g("k_pages")), _ptr(g("v_pages")),
                          _ptr(g("k_norm_w")), _ptr(g("v_scale")), _ptr(g("A_q")),
                          _ptr(g("A_scale")), _ptr(g("folded")))
    return arr


def ridgefill_fold_bytes(shape: rf_shape) -> int:
    """Bytes of one layer's folded buffer (0: the shape cannot be folded)."""
    return int(lib().ridgefill_fold_bytes(C.byref(shape)))


def ridgefill_fold_workspace_bytes(shape: rf_shape) -> int:
    return int(lib().ridgefill_fold_workspace_bytes(C.byref(shape)))


def ridgefill_fold_workspace_bytes_ex(shape: rf_shape, layers_at_once: int) -> int:
    """Fold workspace for layers_at_once layers folded side by side."""
    return int(lib().ridgefill_fold_workspace_bytes_ex(C.byref(shape), layers_at_once))


def ridgefill_fold_workspace_bytes_maps(shape: rf_shape, layers_at_once: int, map_flags: int) -> int:
    """Fold workspace for layers_at_once layers side by side, for bf16 maps (map_flags 0)
    or int8 maps (RF_MAPS_INT8)."""
    return int(lib().ridgefill_fold_workspace_bytes_maps(C.byref(shape), layers_at_once, map_flags))


def ridgefill_fold_maps(shape: rf_shape, layers: list[dict], folded: list, ws, stream=None) -> None:
    """Folded buffers (uint8 device tensors, one per layer) from the layers' plain fields."""
    arr = _layers(layers)
    ptrs = (C.c_void_p * max(len(folded), 1))(*[_ptr(f) for f in folded])
    _check(lib().ridgefill_fold_maps(C.byref(shape), arr, len(layers), ptrs, _ptr(ws),
                                     _nbytes(ws), _stream(stream)))


def ridgefill_fill(shape: rf_shape, x_S, N: int, T: int, filled_idx, n_filled: int,
                   layers: list[dict], block_table, page_size: int, num_pages: int,
                   ws, x_stride: int | None = None, stream=None, copy_stream=None) -> None:
    """The fill; with copy_stream given, the streamed variant (maps in host tensors)."""
    arr = _layers(layers)
    kv = rf_paged_kv(_ptr(block_table), int(block_table.numel()), int(page_size), int(num_pages))
    stride = int(x_stride if x_stride is not None else x_S.stride(0))
    args = (C.byref(shape), _ptr(x_S), int(N), int(T), stride, _ptr(filled_idx), int(n_filled),
            arr, len(layers), C.byref(kv), _ptr(ws), int(ws.numel() * ws.element_size()),
            _stream(stream))
    if copy_stream is None:
        _check(lib().ridgefill_fill(*args))
    else:
        _check(lib().ridgefill_fill_streamed(*args, _stream(copy_stream)))


def ridgefill_fill_noalloc(shape: rf_shape, x_S, N: int, T: int, filled_idx, n_filled: int,
                           layers: list[dict], block_table, page_size: int, num_pages: int,
                           status, x_stride: int | None = None, stream=None) -> None:
    """The fill with the library's fixed device scratch as its workspace (no allocation);
    the device status goes to `status` (a device int32/uint32 tensor of >= 1 element)."""
    arr = _layers(layers)
    kv = rf_paged_kv(_ptr(block_table), int(block_table.numel()), int(page_size), int(num_pages))
    stride = int(x_stride if x_stride is not None else x_S.stride(0))
    _check(lib().ridgefill_fill_noalloc(C.byref(shape), _ptr(x_S), int(N), int(T), stride,
                                        _ptr(filled_idx), int(n_filled), arr, len(layers),
                                        C.byref(kv), _ptr(status), _stream(stream)))


RIDGEFILL_NOALLOC_SCRATCH_BYTES = 64 << 20


def ridgefill_value_scale_workspace_bytes(shape: rf_shape, c: int, n_layers: int,
                                          map_flags: int = 0) -> int:
    return int(lib().ridgefill_value_scale_workspace_bytes(C.byref(shape), int(c), int(n_layers),
                                                           int(map_flags)))


def ridgefill_value_scale(shape: rf_shape, x_S_tail, x_l_tail: list, layers: list[dict], out,
                          ws, x_stride: int | None = None, stream=None) -> None:
    """Value-rescale factors of every layer into out (fp32 [n_layers][n_kv])."""
    arr = _layers(layers)
    ptrs = (C.c_void_p * max(len(x_l_tail), 1))(*[_ptr(t) for t in x_l_tail])
    stride = int(x_stride if x_stride is not None else x_S_tail.stride(0))
    _check(lib().ridgefill_value_scale(C.byref(shape), _ptr(x_S_tail), stride, ptrs,
                                       int(x_S_tail.shape[0]), arr, len(layers), _ptr(out),
                                       _ptr(ws), int(ws.numel() * ws.element_size()),
                                       _stream(stream)))


# ------------------------------------------------------------------------------ calibration

def ridgefill_calib_state_bytes(d: int, n_layers: int, d_out: int | None = None) -> int:
    """State size for x_S of width d (= d_in) and layer inputs of width d_out (default d)."""
    return int(lib().ridgefill_calib_state_bytes_ex(int(d), int(d_out or d), int(n_layers)))


def _nbytes(t) -> int:
    return int(t.numel() * t.element_size())


def ridgefill_calib_reset(state, d: int, n_layers: int, stream=None,
                          d_out: int | None = None) -> None:
    _check(lib().ridgefill_calib_reset_ex(_ptr(state), _nbytes(state), int(d), int(d_out or d),
                                          int(n_layers), _stream(stream)))


def ridgefill_calibrate(state, d: int, n_layers: int, x_S, x_l: list, n_rows: int | None = None,
                        stream=None, d_out: int | None = None) -> None:
    ptrs = (C.c_void_p * max(len(x_l), 1))(*[_ptr(t) for t in x_l])
    n = int(n_rows if n_rows is not None else x_S.shape[0])
    _check(lib().ridgefill_calibrate_ex(_ptr(state), _nbytes(state), int(d), int(d_out or d),
                                        int(n_layers), _ptr(x_S), ptrs, n, _stream(stream)))


def ridgefill_solve_workspace_bytes(d: int, n_layers: int, d_out: int | None = None) -> int:
    return int(lib().ridgefill_solve_workspace_bytes_ex(int(d), int(d_out or d), int(n_layers)))


def ridgefill_solve(state, d: int, n_layers: int, lam: float, A_out, b_out, A_bf16_out, ws,
                    stream=None, d_out: int | None = None) -> None:
    """A_out fp32 [n_layers][d_out][d], b_out [n_layers][d_out] (d_out defaults to d)."""
    _check(lib().ridgefill_solve_ex(_ptr(state), _nbytes(state), int(d), int(d_out or d),
                                    int(n_layers), float(lam), _ptr(A_out), _ptr(b_out),
                                    _ptr(A_bf16_out), _ptr(ws), _nbytes(ws), _stream(stream)))


def ridgefill_read_status(ws, stream=None) -> int:
    """Device status of the last fill/solve/selection on this workspace (waits for the
    stream): RF_OK, RF_E_ROWS, RF_E_NOT_SPD, RF_E_INVALID (a NaN selection score) or
    RF_E_WORKSPACE (a solve on a calibration state that does not match its sizes)."""
    if ws is None:
        raise ValueError("ws is None")
    s = lib().ridgefill_read_status(_ptr(ws), _stream(stream))
    if s not in (RF_OK, RF_E_ROWS, RF_E_NOT_SPD, RF_E_INVALID, RF_E_WORKSPACE):
        _check(s)
    return int(s)


def ridgefill_solve_info(ws, stream=None) -> tuple[float, int]:
    """(kappa_F, parts) of the last solve on this workspace (waits for the stream)."""
    kap = C.c_double(0.0)
    parts = C.c_int32(0)
    _check(lib().ridgefill_solve_info(_ptr(ws), C.byref(kap), C.byref(parts), _stream(stream)))
    return float(kap.value), int(parts.value)


RF_KERNEL_FILL_MAP, RF_KERNEL_FILL_KV, RF_KERNEL_CALIB_MOMENTS, RF_KERNEL_CALIB_SUMS, \
    RF_KERNEL_SOLVE_MAP, RF_KERNEL_FILL_NORM = range(6)


def ridgefill_profile_enable(enable: bool) -> None:
    _check(lib().ridgefill_profile_enable(1 if enable else 0))


def ridgefill_profile_read(kernel: int) -> tuple[int, float]:
    """(launches, summed milliseconds) of one kernel since the last reset."""
    n = C.c_int64(0)
    ms = C.c_double(0.0)
    _check(lib().ridgefill_profile_read(int(kernel), C.byref(n), C.byref(ms)))
    return int(n.value), float(ms.value)


def ridgefill_profile_reset() -> None:
    _check(lib().ridgefill_profile_reset())


def ridgefill_status_string(s: int) -> str:
    return lib().ridgefill_status_string(int(s)).decode()
