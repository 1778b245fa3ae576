"""Brute-force dense one-hot evaluation of the SMoE layer, used to pin the
oracle.  Every expert is applied to every token; a one-hot gate mask then
keeps the chosen ones.  Written with torch fp64 tensor ops so that torch's
autograd supplies the reference gradients.  Independent of ``oracle/``.
"""
import math

import numpy as np
import torch


def t64(a):
    return torch.tensor(np.asarray(a, dtype=np.float64), dtype=torch.float64)


def gate_mask(idx, gates, E):
    """m[t, e] = sum_j gates[t, j] * [idx[t, j] == e] (differentiable in gates)."""
    idx = torch.as_tensor(np.asarray(idx), dtype=torch.long)
    T, k = idx.shape
    m = torch.zeros(T, E, dtype=gates.dtype)
    return m.scatter_add(1, idx, gates)


def act_fn(name):
    if name == "gelu":
        return lambda z: z * 0.5 * (1.0 + torch.erf(z / math.sqrt(2.0)))
    if name == "silu":
        return lambda z: z * torch.sigmoid(z)
    raise ValueError(name)


def dense_mlp(x, w1, w2, idx, gates, act, w3=None):
    """out[t] = sum_e m[t,e] * MLP_e(x[t]), every expert evaluated."""
    E = w1.shape[0]
    H = torch.einsum("td,edf->tef", x, w1)
    if act == "gelu":
        A = act_fn("gelu")(H)
    else:
        A = act_fn("silu")(H) * torch.einsum("td,edf->tef", x, w3)
    Y = torch.einsum("tef,efd->ted", A, w2)
    m = gate_mask(idx, gates, E)
    return torch.einsum("te,ted->td", m, Y)


def dense_all_experts(x, w):
    """Y_all[t, e] = x[t] @ W[e] for every token and expert."""
    return torch.einsum("ti,eio->teo", x, w)


def stable_grouping(idx):
    """Grouped order by a library sort: sorted_scattered = stable argsort of
    the flattened choices; r_of_p its inverse permutation."""
    flat = np.asarray(idx).reshape(-1)
    s = np.argsort(flat, kind="stable")
    r = np.empty_like(s)
    r[s] = np.arange(s.size)
    return s, r
