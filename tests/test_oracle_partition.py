"""Pins of the oracle's row partition and layer ranges against what the page fixes:
the worked example's counts, the map counts of the two deployments, the compute-bound
figures of the second deployment, brute force over every exact-row choice on the
small workload, and the workloads' closed-form filled counts."""

import itertools
import json
import os

import numpy as np
import pytest

import oracle
from ridge_map_kv_amd import configs, synth


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_worked_example_counts(golden_dir):
    g = _load(golden_dir, "worked_example.json")
    p = g["printed"]
    filled, exact, tail = oracle.partition(p["N"], p["T"], g["reading"]["exact_rows"])
    assert len(filled) + len(exact) == p["prefix_rows"]
    assert len(tail) == p["tail_rows"]
    assert oracle.upper_layers(p["S"], p["layers"]) == p["upper_layers"]
    assert [l for l in range(p["layers"]) if l < p["S"]] == p["lower_layers"]
    assert filled.tolist() == g["reading"]["filled_rows"]
    assert tail.tolist() == g["reading"]["tail_rows"]


def test_map_counts_and_sizes(golden_dir):
    g = _load(golden_dir, "map_sizes.json")
    for c in g["cases"]:
        n = c["n_maps"]
        if "S" in c:
            assert len(oracle.upper_layers(c["S"], c["L"])) == n
        nbytes = n * c["d_in"] * c["d_out"] * c["bytes_per_value"]
        unit = {"MiB": 2 ** 20, "GiB": 2 ** 30}[c["unit"]]
        val = nbytes / unit
        if c["bytes_per_value"] == 2:
            assert val == c["printed"]
        else:
            assert abs(val - c["printed"]) / c["printed"] < 0.05


def test_compute_bound_printed(golden_dir):
    g = _load(golden_dir, "compute_bound.json")
    for c in g["cases"]:
        r = oracle.prefill_compute_fraction(g["S"], g["L"], c["N"], g["T"])
        assert round(1.0 / r, 2) == c["bound_printed"], c


def test_brute_force_tiny_all_exact_choices():
    cfg = configs.TINY
    P = cfg.prefix
    for k in range(0, P + 1):
        for E in itertools.combinations(range(P), k):
            filled, exact, tail = oracle.partition(cfg.N, cfg.T, E)
            brute = [t for t in range(cfg.N) if t < P and t not in E]
            assert filled.tolist() == brute
            assert exact.tolist() == list(E)
            assert tail.tolist() == list(range(P, cfg.N))


@pytest.mark.parametrize("name,expected", [("tiny", 7), ("llama3.1-8b", 25805),
                                           ("qwen3-8b", 12288), ("27b-long", 58368)])
def test_filled_counts_closed_form(name, expected):
    cfg = configs.FILL_CONFIGS[name]
    E = synth.exact_rows(cfg)
    filled, exact, tail = oracle.partition(cfg.N, cfg.T, E)
    assert len(filled) == expected == cfg.n_filled
    assert len(tail) == cfg.T
    assert np.all(np.diff(filled) > 0)
    assert len(np.intersect1d(filled, exact)) == 0


def test_blocks_mask_structure():
    cfg = configs.QWEN27B
    E = synth.exact_rows(cfg)
    assert E.size == cfg.exact_count
    runs = np.split(E, np.flatnonzero(np.diff(E) != 1) + 1)
    long_runs = [r for r in runs if len(r) >= 16]
    assert sum(len(r) for r in long_runs) >= cfg.exact_count // 2 - 80


@pytest.mark.parametrize("bad", [[9], [-1], [3, 3]])
def test_partition_rejects(bad):
    with pytest.raises(ValueError):
        oracle.partition(12, 3, bad)


def test_partition_rejects_tail_longer_than_prompt():
    with pytest.raises(ValueError):
        oracle.partition(3, 4, [])


def test_no_prefix():
    filled, exact, tail = oracle.partition(5, 5, [])
    assert filled.size == 0 and exact.size == 0 and tail.tolist() == [0, 1, 2, 3, 4]
