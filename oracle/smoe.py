"""Plain fp64 CPU oracle: routing indices, ParallelLinear (four layouts),
top-k combine, SMoE-MLP (GELU / SwiGLU), the top-k softmax router, the
Mixture-of-Attention core over grouped queries, and their backward passes.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and obvious on
purpose: loops over tokens t and their k choices j, one vector-matrix product
per assignment, fp64 throughout.

Notation.  T tokens, k choices, E experts, M = T*k assignments.  Assignment
p = t*k + j is token t's j-th choice (expert e_p, gate g[t,j]).  "Grouped"
order lists the assignments sorted by expert, ties kept in ascending p; the
grouped position of p is r(p), and s_r is the assignment at grouped row r.

Layouts ([RV1]; [RV2]): the input and the output of ParallelLinear are each
either *grouped* (M rows in grouped order) or *scattered* (token order).  A
scattered input with T rows is read k times (row p // k); one with M rows is
read once (row p).  A scattered output has M rows, row p; with gates it is
combined into T rows.

Precision model for bf16 runs (``storage="bf16"``): every tensor that the
method forms from fp32 values and then feeds to a bf16 contraction is stored
in bf16 (round to nearest even): the pre-activations h (h1, h3), the
activation a, the pre-activation gradients dh (dh1, dh3), and, in the
weight gradient of a gated product, the gate-scaled input row g*u (g*a for
the second MLP matrix): dW[e] = sum (g*u)^T dy, the same exact sum as
u^T (g*dy) with the gate applied to the operand that is stored.
Everything else (scattered expert outputs, k-sums, final results) is kept
exact here.  ``storage="f64"`` rounds nowhere.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np
from scipy.special import erf, expit

__all__ = [
    "bf16_round", "route", "grouped_position", "parallel_linear_fwd",
    "parallel_linear_bwd", "mlp_fwd", "mlp_bwd", "mlp_dw_cols",
    "gelu", "gelu_grad", "silu", "silu_grad", "router_fwd", "router_bwd",
    "moa_attention_fwd", "moa_attention_bwd",
]


# --------------------------------------------------------------------------
# Storage rounding
# --------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round to the nearest bf16 value (8 significant bits), ties to even,
    returned as float64.  frexp gives x = m * 2^e with 0.5 <= |m| < 1, so
    m * 256 carries exactly the 8 bits bf16 keeps; rint rounds half to even.
    Subnormal bf16 (|x| < 2^-126) and overflow are not modelled; no value
    of these workloads comes near either.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def _store(v, storage: str):
    if storage == "bf16":
        return bf16_round(v)
    if storage == "f64":
        return np.asarray(v, dtype=np.float64)
    raise ValueError(storage)


# --------------------------------------------------------------------------
# Activations (exact erf GELU; SiLU for the SwiGLU gate)
# --------------------------------------------------------------------------
def gelu(z):
    z = np.asarray(z, dtype=np.float64)
    return z * 0.5 * (1.0 + erf(z / math.sqrt(2.0)))


def gelu_grad(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * (1.0 + erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z * expit(z)


def silu_grad(z):
    z = np.asarray(z, dtype=np.float64)
    s = expit(z)
    return s * (1.0 + z * (1.0 - s))


# --------------------------------------------------------------------------
# Routing indices  ([PP] "How It Works": the reordering that ParallelLinear
# fuses with the expert transforms; [ART] para. 3)
# --------------------------------------------------------------------------
def route(expert_idxs, E: int) -> Dict[str, np.ndarray]:
    """Counting sort of the assignments by expert.

    counts[e]   = number of assignments p with e_p = e
    offsets     = exclusive prefix sum of counts, E+1 entries, offsets[E] = M
    sorted_scattered_idxs[r] = the assignment p at grouped row r, grouped rows
                  sorted by (e_p, p) ascending
    sorted_expert_idxs[r]    = e of that assignment
    """
    e_of = np.asarray(expert_idxs).reshape(-1)
    M = e_of.shape[0]
    counts = np.zeros(E, dtype=np.int64)
    for p in range(M):
        counts[e_of[p]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    nxt = offsets[:E].copy()
    s_idx = np.empty(M, dtype=np.int64)
    e_idx = np.empty(M, dtype=np.int64)
    for p in range(M):
        e = e_of[p]
        r = nxt[e]
        s_idx[r] = p
        e_idx[r] = e
        nxt[e] += 1
    return {"sorted_expert_idxs": e_idx, "sorted_scattered_idxs": s_idx,
            "counts": counts, "offsets": offsets}


def grouped_position(sorted_scattered_idxs) -> np.ndarray:
    """r(p): inverse of the grouped order."""
    s = np.asarray(sorted_scattered_idxs)
    rinv = np.empty_like(s)
    for r in range(s.shape[0]):
        rinv[s[r]] = r
    return rinv


def _fan(x_rows: int, T: int, k: int, x_grouped: bool) -> int:
    M = T * k
    if x_grouped:
        if x_rows != M:
            raise ValueError("grouped input must have T*k rows")
        return 1
    if x_rows == T:
        return k
    if x_rows == M:
        return 1
    raise ValueError("scattered input must have T or T*k rows")


def _as64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# ParallelLinear forward ([RV1]; [RV2]: the four grouped/scattered
# combinations of one grouped product; [ABS]; [ART] para. 3-4)
# --------------------------------------------------------------------------
def parallel_linear_fwd(x, w, expert_idxs, x_grouped: bool, y_grouped: bool,
                        gates=None, tokens: Optional[Sequence[int]] = None):
    """Y = per-assignment x_row(p) @ W[e_p], placed grouped or scattered.

    Without gates: returns [M, d_out]; row r(p) if y_grouped else row p.
    With gates (scattered output only): returns [T, d_out] with
    Y[t] = sum_j g[t,j] * (x_row(t*k+j) @ W[e]).
    ``tokens`` restricts the work to those tokens (other rows are NaN).
    """
    idx = np.asarray(expert_idxs)
    T, k = idx.shape
    M = T * k
    E = w.shape[0]
    x = _as64(x)
    w = _as64(w)
    fan = _fan(x.shape[0], T, k, x_grouped)
    rinv = grouped_position(route(idx, E)["sorted_scattered_idxs"])
    d_out = w.shape[2]
    todo = range(T) if tokens is None else tokens
    if gates is None:
        Y = np.full((M, d_out), np.nan)
    else:
        if y_grouped:
            raise ValueError("the gate-weighted combine needs scattered output")
        Y = np.full((T, d_out), np.nan)
        g = _as64(gates)
    for t in todo:
        if gates is not None:
            Y[t] = 0.0
        for j in range(k):
            p = t * k + j
            e = idx[t, j]
            u = x[rinv[p]] if x_grouped else x[p // fan]
            v = u @ w[e]
            if gates is None:
                Y[rinv[p] if y_grouped else p] = v
            else:
                Y[t] += g[t, j] * v
    return Y


# --------------------------------------------------------------------------
# ParallelLinear backward ([RV1]: forward and backward both run through the
# same grouped/scattered product; [ART] para. 4: per-expert gradients)
# --------------------------------------------------------------------------
def parallel_linear_bwd(x, w, expert_idxs, x_grouped: bool, y_grouped: bool,
                        dy, gates=None, storage: str = "f64",
                        tokens: Optional[Sequence[int]] = None, dw_cols=None):
    """Gradients of parallel_linear_fwd.

    dy has the forward output's shape.  Per assignment p with input row u:
      dy_p = g[t,j] * dy[t]   (with gates)   or   dy[row of p]   (without)
      dX[input row] += dy_p @ W[e]^T         (k contributions summed when a
                                              T-row input was read k times)
      dW[e]         += u^T (x) dy_p          (with gates: (g*u stored) (x) dy[t])
      dgates[t,j]    = <dy[t], u @ W[e]>     (with gates)
    ``tokens`` restricts dx and dgates to those tokens' assignments (other
    rows NaN); dW still sums over every assignment.  ``dw_cols`` restricts dW
    to those output columns (dW[e][:, c] needs column c of each dy_p alone),
    returned as [E, d_in, len(dw_cols)].
    Returns (dx, dw, dgates or None).
    """
    idx = np.asarray(expert_idxs)
    T, k = idx.shape
    E, d_in, d_out = w.shape
    x = _as64(x)
    w = _as64(w)
    dy = _as64(dy)
    fan = _fan(x.shape[0], T, k, x_grouped)
    rinv = grouped_position(route(idx, E)["sorted_scattered_idxs"])
    cols = np.arange(d_out) if dw_cols is None else np.asarray(dw_cols)
    visit = np.ones(T, dtype=bool)
    if tokens is not None:
        visit[:] = False
        visit[np.asarray(tokens, dtype=np.int64)] = True
    dx = np.zeros_like(x) if tokens is None else np.full(x.shape, np.nan)
    dw = np.zeros((E, d_in, cols.size))
    dg = None
    if gates is not None:
        if y_grouped:
            raise ValueError("the gate-weighted combine needs scattered output")
        g = _as64(gates)
        dg = np.zeros((T, k)) if tokens is None else np.full((T, k), np.nan)
    for t in range(T):
        for j in range(k):
            p = t * k + j
            e = idx[t, j]
            in_row = rinv[p] if x_grouped else p // fan
            u = x[in_row]
            if gates is None:
                dyp = dy[rinv[p] if y_grouped else p]
                dw[e] += np.outer(u, dyp[cols])
            else:
                dyp = g[t, j] * dy[t]
                dw[e] += np.outer(_store(g[t, j] * u, storage), dy[t][cols])
            if visit[t]:
                if gates is not None:
                    dg[t, j] = dy[t] @ (u @ w[e])
                if np.isnan(dx[in_row, 0]):
                    dx[in_row] = 0.0
                dx[in_row] += dyp @ w[e].T
    return dx, dw, dg


# --------------------------------------------------------------------------
# SMoE-MLP ([ART] para. 1 and 5: the SMoE MLP, each token's output is the
# gate-weighted sum of its chosen experts' MLPs; [PP]: the expert linear
# transforms run as ParallelLinear)
# --------------------------------------------------------------------------
def _expert_forward(xt, e, w1, w2, w3, act, storage):
    """One expert MLP on one token row, with the storage roundings."""
    if act == "gelu":
        h = _store(xt @ w1[e], storage)
        h3 = None
        a = _store(gelu(h), storage)
    elif act == "swiglu":
        h = _store(xt @ w1[e], storage)
        h3 = _store(xt @ w3[e], storage)
        a = _store(silu(h) * h3, storage)
    else:
        raise ValueError(act)
    return h, h3, a


def mlp_fwd(x, w1, w2, expert_idxs, gates, act: str, w3=None,
            storage: str = "f64", tokens: Optional[Sequence[int]] = None):
    """out[t] = sum_j g[t,j] * MLP_{e}(x[t]), MLP_e(x) = act(x W1[e]) W2[e]
    (SwiGLU: (silu(x W1[e]) * (x W3[e])) W2[e]).  Rows not in ``tokens`` are
    NaN."""
    idx = np.asarray(expert_idxs)
    T, k = idx.shape
    x, w1, w2 = _as64(x), _as64(w1), _as64(w2)
    w3 = _as64(w3) if w3 is not None else None
    g = _as64(gates)
    out = np.full((T, w2.shape[2]), np.nan)
    for t in (range(T) if tokens is None else tokens):
        acc = np.zeros(w2.shape[2])
        for j in range(k):
            e = idx[t, j]
            _, _, a = _expert_forward(x[t], e, w1, w2, w3, act, storage)
            acc += g[t, j] * (a @ w2[e])
        out[t] = acc
    return out


def mlp_bwd(x, w1, w2, expert_idxs, gates, act: str, dout, w3=None,
            storage: str = "f64", tokens: Optional[Sequence[int]] = None):
    """Backward of mlp_fwd for upstream dout [T, d].

    Per assignment p (token t, choice j, expert e, gate g):
      y_p    = a_p W2[e]
      dg     = <dout[t], y_p>
      dy_p   = g * dout[t]
      dA     = dy_p W2[e]^T
      GELU   : dh  = dA * gelu'(h)
      SwiGLU : dh1 = dA * h3 * silu'(h1);  dh3 = dA * silu(h1)
      dX[t] += dh W1[e]^T (+ dh3 W3[e]^T)
      dW2[e] += (g a_p)^T (x) dout[t];  dW1[e] += x_t^T (x) dh;  dW3[e] += x_t^T (x) dh3
    With ``tokens`` only those tokens are visited: dx and dgates rows are
    exact for them and the returned weight gradients are partial sums.
    Returns dict dx, dw1, dw2, dw3 (None without SwiGLU), dgates.
    """
    idx = np.asarray(expert_idxs)
    T, k = idx.shape
    E = w1.shape[0]
    x, w1, w2, dout = _as64(x), _as64(w1), _as64(w2), _as64(dout)
    w3 = _as64(w3) if w3 is not None else None
    g = _as64(gates)
    dx = np.full(x.shape, np.nan)
    dg = np.full((T, k), np.nan)
    dw1 = np.zeros(w1.shape)
    dw2 = np.zeros(w2.shape)
    dw3 = np.zeros(w1.shape) if act == "swiglu" else None
    for t in (range(T) if tokens is None else tokens):
        dx[t] = 0.0
        for j in range(k):
            e = idx[t, j]
            h, h3, a = _expert_forward(x[t], e, w1, w2, w3, act, storage)
            y = a @ w2[e]
            dg[t, j] = dout[t] @ y
            dyp = g[t, j] * dout[t]
            dA = dyp @ w2[e].T
            if act == "gelu":
                dh = _store(dA * gelu_grad(h), storage)
                dx[t] += dh @ w1[e].T
            else:
                dh = _store(dA * h3 * silu_grad(h), storage)
                dh3 = _store(dA * silu(h), storage)
                dx[t] += dh @ w1[e].T + dh3 @ w3[e].T
                dw3[e] += np.outer(x[t], dh3)
            dw2[e] += np.outer(_store(g[t, j] * a, storage), dout[t])
            dw1[e] += np.outer(x[t], dh)
    return {"dx": dx, "dw1": dw1, "dw2": dw2, "dw3": dw3, "dgates": dg}


def mlp_dw_cols(x, w1, w2, expert_idxs, gates, act: str, dout, cols,
                w3=None, storage: str = "f64"):
    """Weight gradients restricted to hidden columns ``cols`` over ALL tokens.

    Column c of h (and h3, a, dA, dh) depends only on column c of W1 (W3)
    and row c of W2, so the slices dW1[:, :, cols], dW3[:, :, cols] and
    dW2[:, cols, :] follow from the same per-assignment formulas as mlp_bwd
    using those columns alone.  Written per expert as sums over that
    expert's assignments (X_e^T dH_e), which is the definition of dW[e].
    Returns dict dw1, dw2, dw3 slices.
    """
    idx = np.asarray(expert_idxs)
    T, k = idx.shape
    E = w1.shape[0]
    cols = np.asarray(cols)
    x, dout = _as64(x), _as64(dout)
    g = _as64(gates)
    dw1 = np.zeros((E, x.shape[1], cols.size))
    dw2 = np.zeros((E, cols.size, dout.shape[1]))
    dw3 = np.zeros((E, x.shape[1], cols.size)) if act == "swiglu" else None
    for e in range(E):
        tt, jj = np.nonzero(idx == e)
        if tt.size == 0:
            continue
        xe = x[tt]                                   # [n, d]
        ge = g[tt, jj][:, None]                      # [n, 1]
        dye = ge * dout[tt]                          # [n, d]
        w1c = _as64(w1[e][:, cols])
        w2c = _as64(w2[e][cols, :])
        h = _store(xe @ w1c, storage)
        dA = dye @ w2c.T
        if act == "gelu":
            a = _store(gelu(h), storage)
            dh = _store(dA * gelu_grad(h), storage)
        else:
            h3 = _store(xe @ _as64(w3[e][:, cols]), storage)
            a = _store(silu(h) * h3, storage)
            dh = _store(dA * h3 * silu_grad(h), storage)
            dh3 = _store(dA * silu(h), storage)
            dw3[e] = xe.T @ dh3
        dw1[e] = xe.T @ dh
        dw2[e] = _store(ge * a, storage).T @ dout[tt]
    return {"dw1": dw1, "dw2": dw2, "dw3": dw3}


# --------------------------------------------------------------------------
# Router: gate product, top-k and softmax over the chosen logits, backward
# --------------------------------------------------------------------------
def router_fwd(x, g, k: int) -> Dict[str, np.ndarray]:
    """SMoE router ([ART] para. 1: each token goes to k of E experts, its
    output the gate-weighted sum of theirs).  Readings: logits = x G with
    G [d_model, E] (the weight layout of every product here); token t's
    choices are the k largest logits in descending order, ties going to the
    lower expert id (choice j = rank j); the gates are the softmax over the k
    chosen logits (max subtracted).

    x [T, d], g [d, E] -> logits [T, E] (fp64), expert_idxs [T, k] int32,
    gates [T, k] fp64."""
    x = _as64(x)
    g = _as64(g)
    T, E = x.shape[0], g.shape[1]
    logits = np.empty((T, E))
    for t in range(T):
        logits[t] = x[t] @ g
    idx = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        idx[t] = order
        z = logits[t, order]
        w = np.exp(z - z.max())
        gates[t] = w / w.sum()
    return {"logits": logits, "expert_idxs": idx, "gates": gates}


def router_bwd(x, g, expert_idxs, gates, dgates) -> Dict[str, np.ndarray]:
    """Backward of router_fwd for upstream dgates [T, k] (the choice is
    piecewise constant, so only the softmax carries gradient):

      dlogits[t, e_j] = g_j (dg_j - sum_i g_i dg_i),   0 for experts not chosen
      dG = x^T dlogits        [d, E]
      dx = dlogits G^T        [T, d]   (the router's part of the input gradient)
    """
    x = _as64(x)
    g = _as64(g)
    gates = _as64(gates)
    dgates = _as64(dgates)
    idx = np.asarray(expert_idxs)
    T, k = idx.shape
    E = g.shape[1]
    dlogits = np.zeros((T, E))
    for t in range(T):
        s = sum(gates[t, i] * dgates[t, i] for i in range(k))
        for j in range(k):
            dlogits[t, idx[t, j]] = gates[t, j] * (dgates[t, j] - s)
    dg = np.zeros_like(g)
    dx = np.empty_like(x)
    for t in range(T):
        dg += np.outer(x[t], dlogits[t])
        dx[t] = g @ dlogits[t]
    return {"dlogits": dlogits, "dG": dg, "dx": dx}


# --------------------------------------------------------------------------
# Mixture-of-Attention core
# --------------------------------------------------------------------------
def _moa_rows(sorted_scattered_idxs, k: int, seq_len: int, r: int):
    """Grouped query row r belongs to token t = s_r // k (its assignment's
    token); the token is position t % S of sequence t // S; it attends to
    the keys of its own sequence up to and including its own position."""
    t = int(sorted_scattered_idxs[r]) // k
    lo = (t // seq_len) * seq_len
    return t, lo


def moa_attention_fwd(q, kk, v, sorted_scattered_idxs, k: int, seq_len: int) -> Dict[str, np.ndarray]:
    """Attention of grouped expert queries against shared keys and values
    ([ART] para. 4: ScatterMoE runs Mixture-of-Attention, whose experts are
    attention heads, with the same grouped products; the head experts
    share K and V).  Readings: query row r (grouped order, as the Q
    projection's scattered-in / grouped-out product leaves it) is token
    t = s_r // k's query for its expert head; it attends causally within
    its sequence (keys t' with t' // S == t // S and t' <= t); scale
    1/sqrt(hd); the output row stays in grouped order, as the O
    projection's grouped-in input.

    q [M, hd] grouped, kk and v [T, hd] token order (T = B*S) -> o [M, hd],
    lse [M] = log sum_t' exp(score) (the softmax normaliser)."""
    q = _as64(q)
    kk = _as64(kk)
    v = _as64(v)
    M, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    o = np.empty((M, hd))
    lse = np.empty(M)
    for r in range(M):
        t, lo = _moa_rows(sorted_scattered_idxs, k, seq_len, r)
        z = (kk[lo:t + 1] @ q[r]) * scale
        m = z.max()
        w = np.exp(z - m)
        o[r] = (w @ v[lo:t + 1]) / w.sum()
        lse[r] = m + math.log(w.sum())
    return {"o": o, "lse": lse}


def moa_attention_bwd(q, kk, v, sorted_scattered_idxs, k: int, seq_len: int, do,
                      o=None) -> Dict[str, np.ndarray]:
    """Backward of moa_attention_fwd for upstream do [M, hd]: with
    p = softmax(z) over row r's keys, dp_t' = do_r . v_t' and
    D_r = sum p dp (= do_r . o_r),
      dz = p * (dp - D_r),  dq_r = scale * dz @ K,
      dK[t'] += scale * dz_t' q_r,  dV[t'] += p_t' do_r
    (the keys and values gather gradient from every row that reads them).
    With ``o`` (the forward's output as stored, e.g. rounded to bf16), D_r
    is do_r . o_r from it: the one place the backward reads the stored
    output; with the exact o this is the same sum."""
    q = _as64(q)
    kk = _as64(kk)
    v = _as64(v)
    do = _as64(do)
    o = None if o is None else _as64(o)
    M, hd = q.shape
    scale = 1.0 / math.sqrt(hd)
    dq = np.empty_like(q)
    dk = np.zeros_like(kk)
    dv = np.zeros_like(v)
    for r in range(M):
        t, lo = _moa_rows(sorted_scattered_idxs, k, seq_len, r)
        z = (kk[lo:t + 1] @ q[r]) * scale
        w = np.exp(z - z.max())
        p = w / w.sum()
        dp = v[lo:t + 1] @ do[r]
        D = p @ dp if o is None else do[r] @ o[r]
        dz = p * (dp - D)
        dq[r] = scale * (dz @ kk[lo:t + 1])
        dk[lo:t + 1] += scale * np.outer(dz, q[r])
        dv[lo:t + 1] += np.outer(p, do[r])
    return {"dq": dq, "dk": dk, "dv": dv}
