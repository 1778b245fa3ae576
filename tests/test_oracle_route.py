"""Pins for oracle.route and oracle.bf16_round against library routines,
invariants and the hand-worked example."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import zipf_routing, uniform_distinct_routing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _check_against_library(idx, E):
    r = oracle.route(idx, E)
    flat = np.asarray(idx).reshape(-1)
    M = flat.size
    # library routines: stable argsort, bincount, cumsum
    s_ref = np.argsort(flat, kind="stable")
    np.testing.assert_array_equal(r["sorted_scattered_idxs"], s_ref)
    np.testing.assert_array_equal(r["sorted_expert_idxs"], flat[s_ref])
    cnt = np.bincount(flat, minlength=E)
    np.testing.assert_array_equal(r["counts"], cnt)
    np.testing.assert_array_equal(r["offsets"], np.concatenate([[0], np.cumsum(cnt)]))
    # invariants
    s = r["sorted_scattered_idxs"]
    assert sorted(s.tolist()) == list(range(M))
    assert np.all(np.diff(r["sorted_expert_idxs"]) >= 0)
    for e in range(E):
        seg = s[r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(flat[seg] == e)
    assert r["offsets"][E] == M


@pytest.mark.parametrize("T,E,k,seed", [(1, 1, 1, 0), (7, 3, 2, 1), (64, 8, 2, 2),
                                        (100, 16, 4, 3), (33, 5, 5, 4)])
def test_route_random(T, E, k, seed):
    idx = uniform_distinct_routing(T, E, k, (900, seed))
    _check_against_library(idx, E)


def test_route_skewed_with_empty_experts():
    idx, _ = zipf_routing(2048, 64, 8, 1.1, 8, (901, 0))
    r = oracle.route(idx, 64)
    assert (r["counts"] == 0).sum() >= 8
    _check_against_library(idx, 64)


def test_route_all_on_one_expert_and_repeats():
    # non-distinct choices are legal for the routing arrays
    idx = np.full((9, 3), 2, dtype=np.int32)
    _check_against_library(idx, 4)
    idx = np.array([[3, 3], [0, 3], [3, 0]], dtype=np.int32)
    _check_against_library(idx, 4)


def test_route_empty():
    r = oracle.route(np.zeros((0, 2), dtype=np.int32), 4)
    assert r["offsets"].tolist() == [0, 0, 0, 0, 0]
    assert r["sorted_scattered_idxs"].size == 0


def test_route_golden():
    g = json.load(open(os.path.join(GOLDEN, "pl_tiny.json")))
    r = oracle.route(np.array(g["expert_idxs"]), g["E"])
    for key in ("counts", "offsets", "sorted_scattered_idxs", "sorted_expert_idxs"):
        assert r[key].tolist() == g["route"][key], key


def test_bf16_round_matches_torch_on_fp32_values():
    rng = np.random.default_rng(5)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        # exact ties: bf16 value + half an ulp (bit 15 set, lower bits clear),
        # normal numbers only (the oracle does not model bf16 subnormals)
        ((np.arange(0x3000, 0x3000 + 4000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0], dtype=np.float32),
    ])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_round_idempotent_and_bounded():
    rng = np.random.default_rng(6)
    x = rng.standard_normal(10000) * 10.0
    r = oracle.bf16_round(x)
    np.testing.assert_array_equal(oracle.bf16_round(r), r)
    assert np.all(np.abs(r - x) <= np.abs(x) * 2.0 ** -8 + 1e-300)
