"""CPU checks of the C-ABI library: it loads, exports every symbol the header declares,
and its host-only paths (partition, size queries, argument checks) behave.  No call here
reaches the GPU."""

import ctypes as C
import itertools
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from ridge_map_kv_amd import binding as B
from ridge_map_kv_amd import configs, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ridgefill.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ridgefill_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ridgefill_\w+)", out))
    assert set(declared_symbols()) <= exported


def test_partition_bit_exact_vs_oracle_brute_force():
    N, T = 14, 4
    P = N - T
    for k in range(0, 4):
        for E in itertools.combinations(range(P), k):
            mask = np.zeros(P, np.uint8)
            mask[list(E)] = 1
            got = B.ridgefill_partition(N, T, mask)
            want, _, _ = oracle.partition(N, T, E)
            assert np.array_equal(got, want.astype(np.int32))


@pytest.mark.parametrize("name", list(configs.FILL_CONFIGS))
def test_partition_workloads(name):
    cfg = configs.FILL_CONFIGS[name]
    got = B.ridgefill_partition(cfg.N, cfg.T, synth.exact_mask(cfg))
    want, _, _ = oracle.partition(cfg.N, cfg.T, synth.exact_rows(cfg))
    assert got.dtype == np.int32 and np.array_equal(got, want)
    assert got.size == cfg.n_filled


def test_partition_no_mask_and_errors():
    assert np.array_equal(B.ridgefill_partition(10, 3, None), np.arange(7, dtype=np.int32))
    assert B.ridgefill_partition(5, 5, None).size == 0
    with pytest.raises(B.RidgeFillError) as e:
        B.ridgefill_partition(3, 4, None)
    assert e.value.status == B.RF_E_SHAPE


def test_size_queries():
    s = B.make_shape(4096, 8, 128)
    one = B.ridgefill_fill_workspace_bytes(s, 25805, 1)
    twenty = B.ridgefill_fill_workspace_bytes(s, 25805, 20)
    per = twenty - one
    assert one > 0 and per > 0 and per % 19 == 0          # one staging slab per layer
    assert per // 19 >= 25856 * 4096 * 2                    # at least the bf16 staging rows
    assert B.ridgefill_fill_workspace_bytes(s, 25805, 64) == one + 31 * (per // 19)
    assert B.ridgefill_fill_workspace_bytes(B.make_shape(100, 8, 128), 10, 1) == 0
    st = B.ridgefill_calib_state_bytes(4096, 20)
    assert st >= 4 * 4096 * 4096 * 21
    assert B.ridgefill_calib_state_bytes(100, 1) == 0
    assert B.ridgefill_solve_workspace_bytes(4096, 20) > 0


def test_fill_rejects_bad_shapes_before_any_launch():
    L = B.lib()
    kv = B.rf_paged_kv(None, 0, 0, 0)
    for bad in (B.make_shape(300, 8, 128), B.make_shape(4096, 8, 96), B.make_shape(4096, 1, 64),
                B.make_shape(4096, 8, 128, rms_eps=-1.0), B.make_shape(4096, 8, 128, rope_theta=0.5)):
        st = L.ridgefill_fill(C.byref(bad), None, 10, 2, 4096, None, 5, None, 1, C.byref(kv),
                              None, 0, None)
        assert st in (B.RF_E_SHAPE, B.RF_E_INVALID)
        assert L.ridgefill_last_error()
    good = B.make_shape(4096, 8, 128)
    st = L.ridgefill_fill(C.byref(good), None, 10, 2, 4096, None, 9, None, 1, C.byref(kv),
                          None, 0, None)
    assert st == B.RF_E_SHAPE                     # 9 filled rows > 8 prefix rows
    st = L.ridgefill_fill(C.byref(good), None, 10, 2, 4096, None, 5, None, 1, C.byref(kv),
                          None, 0, None)
    assert st == B.RF_E_INVALID                   # null pointers


def test_calib_and_solve_reject_bad_arguments():
    L = B.lib()
    assert L.ridgefill_calib_reset(None, 0, 4096, 20, None) == B.RF_E_INVALID
    assert L.ridgefill_calibrate(None, 0, 4096, 20, None, None, 10, None) == B.RF_E_INVALID
    assert L.ridgefill_solve(None, 0, 4096, 20, 0.1, None, None, None, None, 0, None) == B.RF_E_INVALID


def test_status_strings():
    for s in range(8):
        assert B.ridgefill_status_string(s)


def test_fold_size_queries_and_errors():
    L = B.lib()
    s = B.make_shape(4096, 8, 128)
    fb = B.ridgefill_fold_bytes(s)
    # P [2 kv][d_in] and R [d_in][d_in] in bf16, c, r and kappa in fp32
    assert fb >= (2 * 1024 * 4096 + 4096 * 4096) * 2 + (2 * 1024 + 4096 + 1) * 4
    assert fb % 256 == 0
    w1 = B.ridgefill_fold_workspace_bytes(s)
    assert w1 >= 4096 * 4096 * 8
    # layers folded side by side: one fp64 A^T A block per layer, the rest shared
    assert B.ridgefill_fold_workspace_bytes_ex(s, 1) == w1
    w4 = B.ridgefill_fold_workspace_bytes_ex(s, 4)
    assert (w4 - w1) % 3 == 0 and (w4 - w1) // 3 >= 4096 * 4096 * 8
    assert B.ridgefill_fold_workspace_bytes_ex(s, 0) == 0
    # int8 maps: a second operand slot per layer; unknown map flags give 0
    assert B.ridgefill_fold_workspace_bytes_maps(s, 1, 0) == w1
    assert B.ridgefill_fold_workspace_bytes_maps(s, 4, 0) == w4
    assert B.ridgefill_fold_workspace_bytes_maps(s, 1, B.RF_MAPS_INT8) > w1
    assert B.ridgefill_fold_workspace_bytes_maps(s, 1, B.RF_MAPS_FOLDED) == 0
    # no predicted-input buffer: a folded fill's per-layer workspace is small
    f1 = B.ridgefill_fill_workspace_bytes(s, 25805, 1, B.RF_MAPS_FOLDED)
    f20 = B.ridgefill_fill_workspace_bytes(s, 25805, 20, B.RF_MAPS_FOLDED)
    assert 0 < (f20 - f1) // 19 < 25856 * 4096 // 8
    # wide maps (d_in > d) and ragged d_in cannot be folded
    wide = B.make_shape(4096, 8, 128, d_in=8192)
    assert B.ridgefill_fold_bytes(wide) == 0 and B.ridgefill_fold_workspace_bytes(wide) == 0
    assert B.ridgefill_fill_workspace_bytes(wide, 100, 1, B.RF_MAPS_FOLDED) == 0
    assert B.ridgefill_fold_bytes(B.make_shape(4096, 8, 128, d_in=4032)) == 0
    assert B.ridgefill_fill_workspace_bytes(s, 100, 1, B.RF_MAPS_FOLDED | B.RF_MAPS_INT8) == 0
    # folded layers streamed from host memory: two landing slots of one folded buffer per layer
    fs1 = B.ridgefill_fill_workspace_bytes(s, 100, 1, B.RF_MAPS_FOLDED | B.RF_MAPS_STREAMED)
    assert fs1 >= B.ridgefill_fill_workspace_bytes(s, 100, 1, B.RF_MAPS_FOLDED) + 2 * fb
    arr = (B.rf_layer * 1)()
    assert L.ridgefill_fold_maps(C.byref(wide), arr, 1, None, None, 0, None) == B.RF_E_SHAPE
    assert L.ridgefill_fold_maps(C.byref(s), arr, 1, None, None, 0, None) == B.RF_E_INVALID
    assert L.ridgefill_fold_maps(C.byref(s), arr, 0, None, None, 0, None) == B.RF_E_INVALID
    assert L.ridgefill_last_error()
