"""Pins for oracle.mlp_fwd / mlp_bwd / mlp_dw_cols: brute-force dense
one-hot evaluation, torch fp64 autograd, central finite differences and the
stated invariants (E=1,k=1 dense; token permutation; identical experts; k = E
with uniform gates as one wide dense MLP)."""
import numpy as np
import pytest
import torch

import oracle
from tests.dense_ref import dense_mlp, t64
from workloads import topk_softmax_routing, uniform_distinct_routing


def _case(act, T=16, d=6, f=10, E=4, k=2, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((E, d, f)) / np.sqrt(d)
    w2 = rng.standard_normal((E, f, d)) / np.sqrt(f)
    w3 = rng.standard_normal((E, d, f)) / np.sqrt(d) if act == "swiglu" else None
    idx, gates = topk_softmax_routing(rng.standard_normal((T, E)), k)
    dout = rng.standard_normal((T, d))
    return x, w1, w2, w3, idx, gates.astype(np.float64), dout


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_forward_vs_dense(act):
    x, w1, w2, w3, idx, gates, _ = _case(act, seed=1)
    out = oracle.mlp_fwd(x, w1, w2, idx, gates, act, w3=w3)
    ref = dense_mlp(t64(x), t64(w1), t64(w2), idx, t64(gates),
                    act, t64(w3) if w3 is not None else None).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_backward_vs_autograd(act):
    x, w1, w2, w3, idx, gates, dout = _case(act, seed=2)
    g = oracle.mlp_bwd(x, w1, w2, idx, gates, act, dout, w3=w3)
    xt, w1t, w2t, gt = (t64(a).requires_grad_() for a in (x, w1, w2, gates))
    w3t = t64(w3).requires_grad_() if w3 is not None else None
    out = dense_mlp(xt, w1t, w2t, idx, gt, act, w3t)
    (out * t64(dout)).sum().backward()
    tol = dict(rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(g["dx"], xt.grad.numpy(), **tol)
    np.testing.assert_allclose(g["dw1"], w1t.grad.numpy(), **tol)
    np.testing.assert_allclose(g["dw2"], w2t.grad.numpy(), **tol)
    np.testing.assert_allclose(g["dgates"], gt.grad.numpy(), **tol)
    if act == "swiglu":
        np.testing.assert_allclose(g["dw3"], w3t.grad.numpy(), **tol)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_backward_finite_differences(act):
    x, w1, w2, w3, idx, gates, dout = _case(act, T=6, d=4, f=5, E=3, k=2, seed=3)
    g = oracle.mlp_bwd(x, w1, w2, idx, gates, act, dout, w3=w3)

    def L(x=x, w1=w1, w2=w2, w3=w3, gates=gates):
        return float((oracle.mlp_fwd(x, w1, w2, idx, gates, act, w3=w3) * dout).sum())

    h = 1e-6
    rng = np.random.default_rng(30)
    named = [("dx", "x", x), ("dw1", "w1", w1), ("dw2", "w2", w2), ("dgates", "gates", gates)]
    if act == "swiglu":
        named.append(("dw3", "w3", w3))
    for gname, aname, arr in named:
        for _ in range(8):
            i = tuple(rng.integers(0, n) for n in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[i] += h
            am[i] -= h
            fd = (L(**{aname: ap}) - L(**{aname: am})) / (2 * h)
            assert abs(fd - g[gname][i]) < 1e-6 * max(1.0, abs(fd)), (gname, i, fd, g[gname][i])


def test_e1_k1_is_dense_mlp():
    x, w1, w2, _, _, _, dout = _case("gelu", E=1, k=1, seed=4)
    idx = np.zeros((x.shape[0], 1), dtype=np.int32)
    gates = np.ones((x.shape[0], 1))
    out = oracle.mlp_fwd(x, w1, w2, idx, gates, "gelu")
    ref = oracle.gelu(x @ w1[0]) @ w2[0]
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_token_permutation_commutes(act):
    x, w1, w2, w3, idx, gates, dout = _case(act, seed=5)
    perm = np.random.default_rng(5).permutation(x.shape[0])
    out = oracle.mlp_fwd(x, w1, w2, idx, gates, act, w3=w3)
    out_p = oracle.mlp_fwd(x[perm], w1, w2, idx[perm], gates[perm], act, w3=w3)
    np.testing.assert_allclose(out_p, out[perm], rtol=1e-12, atol=1e-12)
    g = oracle.mlp_bwd(x, w1, w2, idx, gates, act, dout, w3=w3)
    gp = oracle.mlp_bwd(x[perm], w1, w2, idx[perm], gates[perm], act, dout[perm], w3=w3)
    np.testing.assert_allclose(gp["dx"], g["dx"][perm], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(gp["dgates"], g["dgates"][perm], rtol=1e-11, atol=1e-11)
    for n in ("dw1", "dw2") + (("dw3",) if act == "swiglu" else ()):
        np.testing.assert_allclose(gp[n], g[n], rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_identical_experts_reproduce_single_expert(act):
    x, w1, w2, w3, idx, gates, _ = _case(act, seed=6)
    E = w1.shape[0]
    w1s, w2s = np.repeat(w1[:1], E, 0), np.repeat(w2[:1], E, 0)
    w3s = np.repeat(w3[:1], E, 0) if w3 is not None else None
    gates = gates / gates.sum(1, keepdims=True)                     # sum to 1 in fp64
    out = oracle.mlp_fwd(x, w1s, w2s, idx, gates, act, w3=w3s)
    one = oracle.mlp_fwd(x, w1[:1], w2[:1], np.zeros((x.shape[0], 1), np.int32),
                         np.ones((x.shape[0], 1)), act, w3=w3[:1] if w3 is not None else None)
    np.testing.assert_allclose(out, one, rtol=1e-12, atol=1e-12)


def test_k_equals_e_uniform_gates_is_mean_of_experts():
    x, w1, w2, _, _, _, _ = _case("gelu", E=3, k=3, seed=7)
    T = x.shape[0]
    idx = np.tile(np.array([2, 0, 1], dtype=np.int32), (T, 1))
    gates = np.full((T, 3), 1.0 / 3.0)
    out = oracle.mlp_fwd(x, w1, w2, idx, gates, "gelu")
    ref = sum(oracle.gelu(x @ w1[e]) @ w2[e] for e in range(3)) / 3.0
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("storage", ["f64", "bf16"])
def test_dw_cols_matches_full_backward(act, storage):
    x, w1, w2, w3, idx, gates, dout = _case(act, seed=8)
    g = oracle.mlp_bwd(x, w1, w2, idx, gates, act, dout, w3=w3, storage=storage)
    cols = np.array([0, 3, 9])
    c = oracle.mlp_dw_cols(x, w1, w2, idx, gates, act, dout, cols, w3=w3, storage=storage)
    np.testing.assert_allclose(c["dw1"], g["dw1"][:, :, cols], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(c["dw2"], g["dw2"][:, cols, :], rtol=1e-11, atol=1e-11)
    if act == "swiglu":
        np.testing.assert_allclose(c["dw3"], g["dw3"][:, :, cols], rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_bf16_storage_rounds_at_the_stated_points(act):
    """With bf16 storage the oracle equals the dense evaluation that rounds
    h (h1,h3), a, dh (dh1,dh3) and g*a; and stays within bf16 error of
    the unrounded result."""
    x, w1, w2, w3, idx, gates, dout = _case(act, seed=9)
    T, k = idx.shape
    rd = oracle.bf16_round
    out = oracle.mlp_fwd(x, w1, w2, idx, gates, act, w3=w3, storage="bf16")
    out64 = oracle.mlp_fwd(x, w1, w2, idx, gates, act, w3=w3, storage="f64")
    assert not np.array_equal(out, out64)
    rel = np.abs(out - out64).max() / np.sqrt((out64 ** 2).mean())
    assert rel < 0.05
    # dense evaluation with roundings at the same points
    ref = np.zeros_like(out)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            h = rd(x[t] @ w1[e])
            if act == "gelu":
                a = rd(oracle.gelu(h))
            else:
                a = rd(oracle.silu(h) * rd(x[t] @ w3[e]))
            ref[t] += gates[t, j] * (a @ w2[e])
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_all_experts_with_uniform_gates_is_one_wide_dense_mlp(act):
    """k = E with every gate 1/E: the layer averages all experts, which is
    one dense MLP whose hidden units are all experts' units side by side
    (W1 columns concatenated, W2 rows stacked and scaled by 1/E), evaluated
    here with torch's own GELU / SiLU in fp64.  Each token lists the experts
    in its own shuffled order, which must not matter."""
    rng = np.random.default_rng(61)
    T, d, f, E = 7, 6, 5, 4
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((E, d, f)) * 0.5
    w3 = rng.standard_normal((E, d, f)) * 0.5 if act == "swiglu" else None
    w2 = rng.standard_normal((E, f, d)) * 0.5
    idx = np.stack([rng.permutation(E) for _ in range(T)]).astype(np.int32)
    gates = np.full((T, E), 1.0 / E)
    out = oracle.mlp_fwd(x, w1, w2, idx, gates, act, w3=w3)
    W1 = torch.tensor(np.concatenate(list(w1), axis=1))        # [d, E*f]
    W2 = torch.tensor(np.concatenate(list(w2), axis=0)) / E    # [E*f, d]
    h = torch.tensor(x) @ W1
    if act == "gelu":
        a = torch.nn.functional.gelu(h)
    else:
        a = torch.nn.functional.silu(h) * (torch.tensor(x) @ torch.tensor(np.concatenate(list(w3), axis=1)))
    want = (a @ W2).numpy()
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)
