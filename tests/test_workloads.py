"""The seeded generators: reproducible, and the routing structure the
workloads state (distinct pairs; Zipf skew with empty and hot experts)."""
import numpy as np

from workloads import (bf16_bits, bf16_bits_to_f32, make_mlp, make_pl,
                       uniform_distinct_routing, zipf_routing)


def test_seeds_reproduce():
    a = make_mlp(32, 16, 24, 4, 2, "swiglu", "bf16", 77, w_std=0.02)
    b = make_mlp(32, 16, 24, 4, 2, "swiglu", "bf16", 77, w_std=0.02)
    for n in a.tensors:
        np.testing.assert_array_equal(a.tensors[n], b.tensors[n])
    c = make_mlp(32, 16, 24, 4, 2, "swiglu", "bf16", 78, w_std=0.02)
    assert not np.array_equal(a.tensors["x"], c.tensors["x"])


def test_uniform_pairs_are_distinct():
    idx = uniform_distinct_routing(8192, 16, 2, (2, 4))
    assert np.all(idx[:, 0] != idx[:, 1])
    cnt = np.bincount(idx.reshape(-1), minlength=16)
    assert cnt.min() > 0.8 * cnt.mean()


def test_zipf_skew_has_empty_and_hot_experts():
    T = 16384
    idx, gates = zipf_routing(T, 64, 8, 1.1, 8, (4, 4))
    cnt = np.bincount(idx.reshape(-1), minlength=64)
    assert (cnt == 0).sum() >= 1
    assert cnt.max() > 0.10 * T                     # one expert serves > 10% of tokens
    assert np.all(np.sort(idx, axis=1)[:, 1:] != np.sort(idx, axis=1)[:, :-1])
    np.testing.assert_allclose(gates.sum(1), 1.0, rtol=1e-6)


def test_bf16_bits_roundtrip():
    v = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    b = bf16_bits(v)
    np.testing.assert_array_equal(bf16_bits(bf16_bits_to_f32(b)), b)
    assert np.abs(bf16_bits_to_f32(b) - v).max() <= np.abs(v).max() * 2 ** -8


def test_pl_workload_shapes():
    w = make_pl(64, 32, 16, 4, 2, "bf16", 79)
    assert w.tensors["x"].shape == (64, 32)
    assert w.tensors["x_grouped"].shape == (128, 32)
    assert w.tensors["w"].shape == (4, 32, 16)
    assert w.tensors["dy"].shape == (128, 16)
