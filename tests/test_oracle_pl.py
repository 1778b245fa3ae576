"""Pins for oracle.parallel_linear_fwd / _bwd: hand-worked example,
brute-force dense one-hot evaluation, torch fp64 autograd, finite
differences and the stated invariants."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests.dense_ref import dense_all_experts, gate_mask, stable_grouping, t64
from workloads import uniform_distinct_routing, topk_softmax_routing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _case(T=24, E=5, k=2, d_in=7, d_out=6, seed=0):
    rng = np.random.default_rng(seed)
    x_s = rng.standard_normal((T, d_in))
    x_m = rng.standard_normal((T * k, d_in))
    w = rng.standard_normal((E, d_in, d_out))
    idx = uniform_distinct_routing(T, E, k, (910, seed))
    return x_s, x_m, w, idx


def test_golden_tiny():
    g = json.load(open(os.path.join(GOLDEN, "pl_tiny.json")))
    x, w, idx, gates = (np.array(g[n], dtype=np.float64) for n in ("x", "w", "expert_idxs", "gates"))
    idx = idx.astype(np.int32)
    ys = oracle.parallel_linear_fwd(x, w, idx, False, False)
    np.testing.assert_array_equal(ys, g["y_scattered"]["value"])
    yg = oracle.parallel_linear_fwd(x, w, idx, False, True)
    np.testing.assert_array_equal(yg, g["y_grouped"]["value"])
    yc = oracle.parallel_linear_fwd(x, w, idx, False, False, gates=gates)
    np.testing.assert_array_equal(yc, g["combined"]["value"])
    b = g["backward_combined"]
    dx, dw, dg = oracle.parallel_linear_bwd(x, w, idx, False, False, np.array(b["dy"], float), gates=gates)
    np.testing.assert_array_equal(dx, b["dx"])
    np.testing.assert_array_equal(dw, b["dw"])
    np.testing.assert_array_equal(dg, b["dgates"])


# a grouped input always has T*k rows, so x_rows = "T" pairs only with a
# scattered input
@pytest.mark.parametrize("xg,yg,x_rows", [(False, False, "T"), (False, True, "T"), (False, False, "M"),
                                          (False, True, "M"), (True, False, "M"), (True, True, "M")])
def test_forward_vs_dense_one_hot(xg, yg, x_rows):
    x_s, x_m, w, idx = _case(seed=1)
    T, k = idx.shape
    x = x_s if x_rows == "T" else x_m
    y = oracle.parallel_linear_fwd(x, w, idx, xg, yg)
    s, r_of = stable_grouping(idx)
    # dense: evaluate every expert on every input row, then select
    Yall = dense_all_experts(t64(x), t64(w)).numpy()      # [rows, E, d_out]
    flat = idx.reshape(-1)
    ref = np.empty((T * k, w.shape[2]))
    for p in range(T * k):
        in_row = r_of[p] if xg else (p // k if x_rows == "T" else p)
        ref[r_of[p] if yg else p] = Yall[in_row, flat[p]]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_cross_variant_consistency():
    x_s, _, w, idx = _case(seed=2)
    ys = oracle.parallel_linear_fwd(x_s, w, idx, False, False)
    yg = oracle.parallel_linear_fwd(x_s, w, idx, False, True)
    s, _ = stable_grouping(idx)
    np.testing.assert_array_equal(yg, ys[s])
    # grouped input holding the gathered rows gives the same products
    xg_rows = x_s[s // idx.shape[1]]
    np.testing.assert_allclose(oracle.parallel_linear_fwd(xg_rows, w, idx, True, True), yg, rtol=1e-13, atol=1e-13)


def test_e1_k1_is_dense_linear():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, 9))
    w = rng.standard_normal((1, 9, 4))
    idx = np.zeros((20, 1), dtype=np.int32)
    for xg in (False, True):
        for yg in (False, True):
            y = oracle.parallel_linear_fwd(x, w, idx, xg, yg)
            np.testing.assert_allclose(y, x @ w[0], rtol=1e-13, atol=1e-13)
    yc = oracle.parallel_linear_fwd(x, w, idx, False, False, gates=np.ones((20, 1)))
    np.testing.assert_allclose(yc, x @ w[0], rtol=1e-13, atol=1e-13)


def test_linearity():
    x_s, _, w, idx = _case(seed=4)
    rng = np.random.default_rng(4)
    x2 = rng.standard_normal(x_s.shape)
    w2 = rng.standard_normal(w.shape)
    f = lambda x, w: oracle.parallel_linear_fwd(x, w, idx, False, False)
    np.testing.assert_allclose(f(2 * x_s - x2, w), 2 * f(x_s, w) - f(x2, w), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(f(x_s, w + 3 * w2), f(x_s, w) + 3 * f(x_s, w2), rtol=1e-11, atol=1e-11)


def _torch_pl(x, w, idx, xg, yg, gates, x_rows):
    """Dense one-hot ParallelLinear in torch (every expert on every row)."""
    T, k = idx.shape
    s, r_of = stable_grouping(idx)
    flat = torch.as_tensor(idx.reshape(-1), dtype=torch.long)
    Yall = torch.einsum("ti,eio->teo", x, w)
    p = np.arange(T * k)
    in_rows = torch.as_tensor(r_of if xg else (p // k if x_rows == "T" else p))
    ysel = Yall[in_rows, flat]                      # [M, d_out], row p
    if gates is None:
        return ysel[torch.as_tensor(s)] if yg else ysel
    m = ysel.reshape(T, k, -1)
    return (gates[:, :, None] * m).sum(1)


@pytest.mark.parametrize("xg,yg,x_rows,use_gates", [
    (False, False, "T", False), (False, True, "T", False), (True, False, "M", False),
    (True, True, "M", False), (False, False, "M", False),
    (False, False, "T", True), (True, False, "M", True)])
def test_backward_vs_autograd(xg, yg, x_rows, use_gates):
    x_s, x_m, w, idx = _case(seed=5)
    T, k = idx.shape
    x = x_s if x_rows == "T" else x_m
    gates = None
    if use_gates:
        _, gates = topk_softmax_routing(np.random.default_rng(5).standard_normal((T, w.shape[0])), k)
        # use the same expert choices as the case but these gate values
    rng = np.random.default_rng(50)
    dy = rng.standard_normal((T if use_gates else T * k, w.shape[2]))
    dx, dw, dg = oracle.parallel_linear_bwd(x, w, idx, xg, yg, dy, gates=gates)
    xt = t64(x).requires_grad_()
    wt = t64(w).requires_grad_()
    gt = t64(gates).requires_grad_() if use_gates else None
    y = _torch_pl(xt, wt, idx, xg, yg, gt, x_rows)
    (y * t64(dy)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-11, atol=1e-11)
    if use_gates:
        np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-11, atol=1e-11)


def test_backward_finite_differences():
    x_s, _, w, idx = _case(T=10, E=3, k=2, d_in=5, d_out=4, seed=6)
    T, k = idx.shape
    _, gates = topk_softmax_routing(np.random.default_rng(6).standard_normal((T, 3)), k)
    gates = gates.astype(np.float64)
    dy = np.random.default_rng(60).standard_normal((T, 4))
    dx, dw, dg = oracle.parallel_linear_bwd(x_s, w, idx, False, False, dy, gates=gates)
    L = lambda x, w, g: float((oracle.parallel_linear_fwd(x, w, idx, False, False, gates=g) * dy).sum())
    h = 1e-6
    rng = np.random.default_rng(61)
    for _ in range(12):
        i = tuple(rng.integers(0, n) for n in x_s.shape)
        xp, xm = x_s.copy(), x_s.copy(); xp[i] += h; xm[i] -= h
        assert abs((L(xp, w, gates) - L(xm, w, gates)) / (2 * h) - dx[i]) < 1e-6
        i = tuple(rng.integers(0, n) for n in w.shape)
        wp, wm = w.copy(), w.copy(); wp[i] += h; wm[i] -= h
        assert abs((L(x_s, wp, gates) - L(x_s, wm, gates)) / (2 * h) - dw[i]) < 1e-6
        i = tuple(rng.integers(0, n) for n in gates.shape)
        gp, gm = gates.copy(), gates.copy(); gp[i] += h; gm[i] -= h
        assert abs((L(x_s, w, gp) - L(x_s, w, gm)) / (2 * h) - dg[i]) < 1e-6


def test_zero_token_expert_gets_zero_dw():
    x_s, _, w, idx = _case(T=12, E=6, k=2, seed=7)
    idx = np.where(idx == 5, 4, idx)
    idx[:, 1] = np.where(idx[:, 0] == idx[:, 1], (idx[:, 0] + 1) % 5, idx[:, 1])
    dy = np.random.default_rng(70).standard_normal((24, w.shape[2]))
    _, dw, _ = oracle.parallel_linear_bwd(x_s, w, idx, False, False, dy)
    assert np.all(dw[5] == 0.0)
    assert np.any(dw[4] != 0.0)


def test_bf16_storage_only_touches_gated_weight_gradient():
    x_s, _, w, idx = _case(T=8, E=3, k=2, seed=8)
    T, k = idx.shape
    _, gates = topk_softmax_routing(np.random.default_rng(8).standard_normal((T, 3)), k)
    dy = np.random.default_rng(80).standard_normal((T, w.shape[2]))
    a = oracle.parallel_linear_bwd(x_s, w, idx, False, False, dy, gates=gates, storage="f64")
    b = oracle.parallel_linear_bwd(x_s, w, idx, False, False, dy, gates=gates, storage="bf16")
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[2], b[2])
    assert not np.array_equal(a[1], b[1])
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=2.0 ** -7 * np.abs(a[1]).max() * 4)


@pytest.mark.parametrize("xg,yg,use_gates", [(False, True, False), (True, False, True), (False, False, True)])
def test_backward_token_and_column_restriction(xg, yg, use_gates):
    """The restricted backward (sampled tokens, a column slice of dW) is the
    full backward's rows and columns exactly."""
    x_s, x_g, w, idx = _case(T=11, E=4, k=2, d_in=6, d_out=7, seed=9)
    T, k = idx.shape
    x = x_g if xg else x_s
    gates = None
    if use_gates:
        _, gates = topk_softmax_routing(np.random.default_rng(90).standard_normal((T, 4)), k)
        gates = gates.astype(np.float64)
    dy = np.random.default_rng(91).standard_normal((T if use_gates else T * k, 7))
    dx, dw, dg = oracle.parallel_linear_bwd(x, w, idx, xg, yg, dy, gates=gates, storage="bf16")
    toks = [0, 4, 10]
    cols = [0, 3, 6]
    rdx, rdw, rdg = oracle.parallel_linear_bwd(x, w, idx, xg, yg, dy, gates=gates, storage="bf16",
                                               tokens=toks, dw_cols=cols)
    np.testing.assert_array_equal(rdw, dw[:, :, cols])
    rinv = oracle.grouped_position(oracle.route(idx, 4)["sorted_scattered_idxs"])
    rows = [rinv[t * k + j] for t in toks for j in range(k)] if xg else toks
    np.testing.assert_allclose(rdx[rows], dx[rows], rtol=1e-13, atol=1e-13)
    others = np.setdiff1d(np.arange(x.shape[0]), rows)
    assert np.all(np.isnan(rdx[others]))
    if use_gates:
        np.testing.assert_allclose(rdg[toks], dg[toks], rtol=1e-13, atol=1e-13)
