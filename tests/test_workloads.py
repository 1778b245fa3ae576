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


def test_tile_covering_samples():
    """The full-size parity samples: every block of rows of every expert's
    grouped segment holds a sampled token's row, and every column block a
    sampled column."""
    import oracle
    from tests.gpu_util import cols_covering, tokens_covering_tiles
    rng = np.random.default_rng(3)
    T, k, E = 3000, 2, 7
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    r = oracle.route(idx, E)
    toks = tokens_covering_tiles(r["sorted_scattered_idxs"], r["offsets"], k, 128, 5, 1)
    chosen = np.zeros(T, dtype=bool)
    chosen[toks] = True
    rows_hit = chosen[r["sorted_scattered_idxs"] // k]
    for e in range(E):
        lo, hi = r["offsets"][e], r["offsets"][e + 1]
        for b in range(lo, hi, 128):
            assert rows_hit[b:min(b + 128, hi)].any(), (e, b)
        assert rows_hit[lo] and rows_hit[hi - 1]
    c = cols_covering(1000, 256, 2)
    assert c[0] == 0 and c[-1] == 999
    for b in range(0, 1000, 256):
        assert ((c >= b) & (c < b + 256)).any()


def test_bf16_half_ulp_bounds_rounding():
    """The metric used for the named exceptions to the plain bound removes
    exactly the largest rounding error, half an ulp at each magnitude
    (checked against the oracle's bf16 rounding), and nothing more."""
    import oracle
    from tests.gpu_util import bf16_half_ulp, rel_err_beyond_bf16_rounding
    v = np.random.default_rng(5).standard_normal(20000) * np.exp(np.random.default_rng(6).uniform(-8, 8, 20000))
    r = oracle.bf16_round(v)
    assert np.all(np.abs(r - v) <= bf16_half_ulp(v) * (1 + 1e-12))
    # at 10 RMS a bf16 value can be off by more than 2e-2 RMS ...
    x = np.concatenate([np.ones(999) * 0.1, [10.03]])
    assert np.abs(oracle.bf16_round(x) - x).max() / np.sqrt(np.mean(x ** 2)) > 2e-2
    # ... which this metric does not count, while any further error counts
    assert rel_err_beyond_bf16_rounding(oracle.bf16_round(x), x) == 0.0
    y = oracle.bf16_round(x).copy()
    y[0] += 0.05
    assert rel_err_beyond_bf16_rounding(y, x) > 0.0
