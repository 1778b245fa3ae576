"""Pins for the oracle's bf16 storage model in the BACKWARD passes.

In bf16 runs the method stores, and feeds to bf16 contractions, the
pre-activations h (h1, h3), the activation a, the pre-activation gradients
dh (dh1, dh3), and the gate-scaled operand of a gated weight gradient (g*a
for the MLP's second matrix, g*u for a gated ParallelLinear); everything else
stays exact.  The reference here is written from that statement alone, in a
different form from the oracle's per-token loops: every expert is evaluated
on every token with torch fp64 tensor products, a gate mask (zero for experts
a token did not choose) selects, derivatives of the activations come from
torch's autograd of its own SiLU / GELU, and the rounding to bf16 is torch's
conversion made exact by an intermediate round-to-odd step (Boldo and
Melquiond, "Emulation of FMA and correctly rounded sums: proved algorithms
using rounding to odd", IEEE Trans. Computers 2008: rounding to odd at 24
bits, then to nearest even at 8, equals rounding straight to 8 bits).
"""
import numpy as np
import pytest
import torch

import oracle
from tests.dense_ref import gate_mask, stable_grouping
from workloads import topk_softmax_routing


def bf16_exact(v: torch.Tensor) -> torch.Tensor:
    """fp64 -> nearest bf16 (ties to even), returned as fp64, without the
    double rounding of a plain fp64 -> fp32 -> bf16 conversion."""
    v = v.to(torch.float64)
    f = v.to(torch.float32)
    back = f.to(torch.float64)
    inexact = back != v
    even = (f.view(torch.int32) & 1) == 0
    toward = torch.where(v > back, torch.full_like(f, float("inf")), torch.full_like(f, float("-inf")))
    f = torch.where(inexact & even, torch.nextafter(f, toward), f)
    return f.to(torch.bfloat16).to(torch.float64)


def test_bf16_exact_rounding():
    """The test's own rounding: agrees with torch's fp32 -> bf16 where no
    double rounding can occur, and resolves values just off a bf16 midpoint
    that a plain fp64 -> fp32 -> bf16 conversion gets wrong."""
    rng = np.random.default_rng(7)
    x32 = torch.tensor(rng.standard_normal(20000).astype(np.float32) * 10.0)
    np.testing.assert_array_equal(bf16_exact(x32.to(torch.float64)).numpy(),
                                  x32.to(torch.bfloat16).to(torch.float64).numpy())
    # 1 + 2^-8 is the midpoint between bf16 1 and 1 + 2^-7: ties go to even (1);
    # a hair above it must round up, a hair below down, although the fp32
    # rounding of either lands on the midpoint itself
    mid = 1.0 + 2.0 ** -8
    v = torch.tensor([mid, mid + 2.0 ** -40, mid - 2.0 ** -40, -(mid + 2.0 ** -40)], dtype=torch.float64)
    np.testing.assert_array_equal(bf16_exact(v).numpy(), [1.0, 1.0 + 2.0 ** -7, 1.0, -(1.0 + 2.0 ** -7)])
    assert float(v[1].to(torch.float32).to(torch.bfloat16)) == 1.0   # the double rounding it avoids


def _act_and_grad(name, h):
    """torch's activation of h and its derivative (autograd), elementwise."""
    hh = h.detach().clone().requires_grad_()
    f = torch.nn.functional.silu if name == "silu" else torch.nn.functional.gelu
    y = f(hh)
    (g,) = torch.autograd.grad(y.sum(), hh)
    return y.detach(), g


def _mlp_case(act, T=20, d=6, f=9, E=5, k=2, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((E, d, f)) / np.sqrt(d)
    w3 = rng.standard_normal((E, d, f)) / np.sqrt(d) if act == "swiglu" else None
    w2 = rng.standard_normal((E, f, d)) / np.sqrt(f)
    idx, gates = topk_softmax_routing(rng.standard_normal((T, E)), k)
    dout = rng.standard_normal((T, d))
    return x, w1, w2, w3, idx, gates.astype(np.float64), dout


def dense_mlp_bwd_bf16(x, w1, w2, w3, idx, gates, dout, act):
    """Backward of the SMoE-MLP with bf16 storage at the stated points, every
    expert evaluated on every token and masked by the gates."""
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64))
    x, w1, w2, dout = t(x), t(w1), t(w2), t(dout)
    E = w1.shape[0]
    m = gate_mask(idx, t(gates), E)                           # [T, E]: g or 0
    H1 = bf16_exact(torch.einsum("td,edf->tef", x, w1))       # [T, E, f]
    if act == "swiglu":
        w3 = t(w3)
        H3 = bf16_exact(torch.einsum("td,edf->tef", x, w3))
        s, s_grad = _act_and_grad("silu", H1)
        A = bf16_exact(s * H3)
    else:
        gl, gl_grad = _act_and_grad("gelu", H1)
        A = bf16_exact(gl)
    V = torch.einsum("td,efd->tef", dout, w2)                 # dout W2[e]^T for every expert
    dA = m[:, :, None] * V
    if act == "swiglu":
        dH1 = bf16_exact(dA * H3 * s_grad)
        dH3 = bf16_exact(dA * s)
        dx = torch.einsum("tef,edf->td", dH1, w1) + torch.einsum("tef,edf->td", dH3, w3)
        dw3 = torch.einsum("td,tef->edf", x, dH3)
    else:
        dH1 = bf16_exact(dA * gl_grad)
        dx = torch.einsum("tef,edf->td", dH1, w1)
        dw3 = None
    dw1 = torch.einsum("td,tef->edf", x, dH1)
    gA = bf16_exact(m[:, :, None] * A)                        # the stored g*a (0 where unchosen)
    dw2 = torch.einsum("tef,td->efd", gA, dout)
    Y = torch.einsum("tef,efd->ted", A, w2)                   # every expert's output
    ii = torch.as_tensor(np.asarray(idx), dtype=torch.long)
    dg = torch.einsum("tjd,td->tj", Y[torch.arange(Y.shape[0])[:, None], ii], dout)
    out = {"dx": dx, "dw1": dw1, "dw2": dw2, "dgates": dg}
    if dw3 is not None:
        out["dw3"] = dw3
    return {n: v.numpy() for n, v in out.items()}


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_mlp_bwd_bf16_storage_model(act):
    x, w1, w2, w3, idx, gates, dout = _mlp_case(act, seed=11)
    got = oracle.mlp_bwd(x, w1, w2, idx, gates, act, dout, w3=w3, storage="bf16")
    ref = dense_mlp_bwd_bf16(x, w1, w2, w3, idx, gates, dout, act)
    for name, want in ref.items():
        np.testing.assert_allclose(got[name], want, rtol=1e-12, atol=1e-12, err_msg=name)
    # the roundings are there: the exact backward differs
    exact = oracle.mlp_bwd(x, w1, w2, idx, gates, act, dout, w3=w3, storage="f64")
    for name in ("dx", "dw1", "dw2"):
        assert np.abs(exact[name] - got[name]).max() > 1e-6, name


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_mlp_dw_cols_bf16_storage_model(act):
    """The column-slice form the full-size GPU tests rely on, against the
    same dense reference."""
    x, w1, w2, w3, idx, gates, dout = _mlp_case(act, seed=12)
    cols = np.array([0, 4, 8])
    got = oracle.mlp_dw_cols(x, w1, w2, idx, gates, act, dout, cols, w3=w3, storage="bf16")
    ref = dense_mlp_bwd_bf16(x, w1, w2, w3, idx, gates, dout, act)
    np.testing.assert_allclose(got["dw1"], ref["dw1"][:, :, cols], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["dw2"], ref["dw2"][:, cols, :], rtol=1e-12, atol=1e-12)
    if act == "swiglu":
        np.testing.assert_allclose(got["dw3"], ref["dw3"][:, :, cols], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("x_grouped", [False, True])
def test_gated_parallel_linear_bwd_bf16_storage_model(x_grouped):
    """Gated ParallelLinear (the Mixture-of-Attention O projection's form
    when x is grouped): dw[e] = sum over e's assignments of the stored
    g*u times dy[t]; dx and dgates stay exact."""
    rng = np.random.default_rng(13)
    T, E, k, d_in, d_out = 18, 5, 3, 7, 6
    idx, gates = topk_softmax_routing(rng.standard_normal((T, E)), k)
    gates = gates.astype(np.float64)
    x = rng.standard_normal((T * k if x_grouped else T, d_in))
    w = rng.standard_normal((E, d_in, d_out))
    dy = rng.standard_normal((T, d_out))
    dx, dw, dg = oracle.parallel_linear_bwd(x, w, idx, x_grouped, False, dy, gates=gates, storage="bf16")

    s, r_of = stable_grouping(idx)
    p = np.arange(T * k)
    u = torch.tensor(x[r_of[p]] if x_grouped else x[p // k])            # input row of each assignment
    onehot = torch.zeros(T * k, E, dtype=torch.float64)
    onehot[torch.arange(T * k), torch.as_tensor(idx.reshape(-1), dtype=torch.long)] = 1.0
    gp = torch.tensor(gates.reshape(-1))
    dy_p = torch.tensor(dy[p // k])
    gu = bf16_exact(gp[:, None] * u)                                     # stored g*u
    ref_dw = torch.einsum("pe,pi,po->eio", onehot, gu, dy_p).numpy()
    np.testing.assert_allclose(dw, ref_dw, rtol=1e-12, atol=1e-12)
    # dx: (g dy[t]) W[e]^T back to the input row, exact; k-summed per token
    # when a T-row input was read k times
    W = torch.tensor(w)
    contrib = torch.einsum("pe,po,eio->pi", onehot, gp[:, None] * dy_p, W).numpy()
    ref_dx = np.zeros_like(x)
    np.add.at(ref_dx, r_of[p] if x_grouped else p // k, contrib)
    np.testing.assert_allclose(dx, ref_dx, rtol=1e-12, atol=1e-12)
    y_p = torch.einsum("pe,pi,eio->po", onehot, u, W)
    ref_dg = (y_p * dy_p).sum(1).reshape(T, k).numpy()
    np.testing.assert_allclose(dg, ref_dg, rtol=1e-12, atol=1e-12)
    # the rounding is there
    _, dw64, _ = oracle.parallel_linear_bwd(x, w, idx, x_grouped, False, dy, gates=gates, storage="f64")
    assert np.abs(dw64 - dw).max() > 1e-6
