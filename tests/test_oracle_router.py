"""Pins for oracle.router_fwd / router_bwd: numpy's stable argsort and
scipy's softmax (library routines), the tie rule on duplicated gate columns,
k = E (a softmax over all experts), torch fp64 autograd of the softmax over
the chosen logits, central finite differences, and k = 1 (no gradient)."""
import numpy as np
import torch
from scipy.special import softmax

import oracle


def _case(T=12, d=7, E=6, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, d)), rng.standard_normal((d, E)) / np.sqrt(d)


def test_forward_is_sorted_topk_and_softmax():
    x, g = _case(seed=1)
    k = 3
    r = oracle.router_fwd(x, g, k)
    logits = x @ g
    np.testing.assert_allclose(r["logits"], logits, rtol=1e-13, atol=1e-13)
    want = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(r["expert_idxs"], want)
    chosen = np.take_along_axis(logits, want, axis=1)
    np.testing.assert_allclose(r["gates"], softmax(chosen, axis=1), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r["gates"].sum(axis=1), 1.0, rtol=1e-13)


def test_ties_go_to_the_lower_expert():
    x, g = _case(T=5, d=4, E=5, seed=2)
    g[:, 3] = g[:, 1]            # experts 1 and 3 always tie
    g[:, 1] += 5.0               # and beat everything else for positive x sums
    g[:, 3] = g[:, 1]
    x = np.abs(x) + 0.1
    r = oracle.router_fwd(x, g, 2)
    np.testing.assert_array_equal(r["expert_idxs"], np.tile([1, 3], (5, 1)))
    np.testing.assert_allclose(r["gates"], 0.5, rtol=1e-14)


def test_k_equal_to_E_is_a_full_softmax():
    x, g = _case(seed=3)
    E = g.shape[1]
    r = oracle.router_fwd(x, g, E)
    full = softmax(x @ g, axis=1)
    np.testing.assert_allclose(np.take_along_axis(full, r["expert_idxs"], axis=1), r["gates"], rtol=1e-13)


def _loss_torch(x, g, idx, dgates):
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    gt = torch.tensor(g, dtype=torch.float64, requires_grad=True)
    chosen = torch.gather(xt @ gt, 1, torch.tensor(idx, dtype=torch.int64))
    loss = (torch.softmax(chosen, dim=1) * torch.tensor(dgates)).sum()
    loss.backward()
    return xt.grad.numpy(), gt.grad.numpy()


def test_backward_matches_autograd_and_invariants():
    x, g = _case(T=10, d=5, E=7, seed=4)
    k = 3
    f = oracle.router_fwd(x, g, k)
    dgates = np.random.default_rng(5).standard_normal((10, k))
    b = oracle.router_bwd(x, g, f["expert_idxs"], f["gates"], dgates)
    dx, dg = _loss_torch(x, g, f["expert_idxs"], dgates)
    np.testing.assert_allclose(b["dx"], dx, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(b["dG"], dg, rtol=1e-12, atol=1e-13)
    # softmax gradients sum to zero over a token's choices; other logits get none
    np.testing.assert_allclose(b["dlogits"].sum(axis=1), 0.0, atol=1e-14)
    mask = np.zeros_like(b["dlogits"], dtype=bool)
    np.put_along_axis(mask, f["expert_idxs"], True, axis=1)
    assert np.all(b["dlogits"][~mask] == 0.0)


def test_backward_finite_differences():
    x, g = _case(T=6, d=4, E=5, seed=6)
    k = 2
    dgates = np.random.default_rng(7).standard_normal((6, k))

    def loss(xx, gg):
        r = oracle.router_fwd(xx, gg, k)
        return float((r["gates"] * dgates).sum())

    f = oracle.router_fwd(x, g, k)
    b = oracle.router_bwd(x, g, f["expert_idxs"], f["gates"], dgates)
    h = 1e-6
    for (i, j) in [(0, 0), (1, 3), (3, 2), (2, 4)]:
        gp, gm = g.copy(), g.copy()
        gp[i, j] += h
        gm[i, j] -= h
        assert abs((loss(x, gp) - loss(x, gm)) / (2 * h) - b["dG"][i, j]) < 1e-7
    for (i, j) in [(0, 1), (5, 3), (2, 0)]:
        xp, xm = x.copy(), x.copy()
        xp[i, j] += h
        xm[i, j] -= h
        assert abs((loss(xp, g) - loss(xm, g)) / (2 * h) - b["dx"][i, j]) < 1e-7


def test_k1_has_no_gradient():
    x, g = _case(seed=8)
    f = oracle.router_fwd(x, g, 1)
    np.testing.assert_array_equal(f["gates"], 1.0)
    b = oracle.router_bwd(x, g, f["expert_idxs"], f["gates"], np.ones((x.shape[0], 1)))
    assert np.all(b["dG"] == 0.0) and np.all(b["dx"] == 0.0)
