"""Seeded synthetic inputs for the scattered mixture-of-experts hot path.

This module only *draws* inputs.  It holds none of the arithmetic that the
hot path performs (routing-index construction, the grouped products, the
combine, activations or their gradients); both the CPU oracle and the GPU
library receive exactly the arrays produced here.

What the inputs stand for (page "Scattered Mixture-of-Experts Implementation",
abstract; and the article "This Machine Learning Research Presents ScatterMoE",
body): a sparse mixture-of-experts layer in which every token picks k of E
experts and the layer output is the gate-weighted sum of the chosen experts'
outputs.  No page measures on a public dataset; every tensor is synthetic.

Storage convention.  bf16 tensors are returned as ``uint16`` bit patterns
(round-to-nearest-even from a float32 draw); fp32 tensors as ``float32``.
Index tensors are ``int32``; gates are ``float32``.

The router that turns scores into (expert_idxs, gates) lives here because the
hot path starts from the expert choices; the router itself is not part of it.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional

import numpy as np

__all__ = [
    "CONFIGS", "Workload", "bf16_bits", "bf16_bits_to_f32", "make_config", "make_router", "make_moa_attention", "make_moa_layer",
    "make_mlp", "make_pl", "make_moa", "topk_softmax_routing",
    "uniform_distinct_routing", "zipf_routing",
]


# --------------------------------------------------------------------------
# bf16 bit handling (input preparation only)
# --------------------------------------------------------------------------
def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def _normal(shape, std: float, key, dtype: str, per_expert: bool = False):
    """N(0, std^2) draw; bf16 -> uint16 bits, fp32 -> float32.

    With ``per_expert`` the leading axis is drawn slice by slice, each slice
    from its own key (key + (e,)), so big expert weights are drawn in
    parallel threads and any one expert can be re-drawn alone.
    """
    shape = tuple(int(s) for s in shape)

    def one(sub_key, sub_shape):
        x = _rng(*sub_key).standard_normal(sub_shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        return bf16_bits(x) if dtype == "bf16" else x

    if not per_expert:
        return one(key, shape)
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    n = shape[0]

    def fill(e):
        out[e] = one(tuple(key) + (e,), shape[1:])

    if n * int(np.prod(shape[1:])) > (1 << 22):
        with ThreadPoolExecutor(min(8, n)) as ex:
            list(ex.map(fill, range(n)))
    else:
        for e in range(n):
            fill(e)
    return out


# --------------------------------------------------------------------------
# Router choices (input synthesis; the hot path begins after this)
# --------------------------------------------------------------------------
def topk_softmax_routing(scores: np.ndarray, k: int):
    """Pick the k largest scores per row (descending; ties -> lower expert
    id) and weight them by a softmax over the k picked scores.

    Returns (expert_idxs int32 [T,k], gates float32 [T,k]).  Column j of
    expert_idxs is the j-th choice; assignment p = t*k + j.
    """
    s = np.asarray(scores, dtype=np.float64)
    order = np.argsort(-s, axis=1, kind="stable")[:, :k]
    picked = np.take_along_axis(s, order, axis=1)
    z = np.exp(picked - picked.max(axis=1, keepdims=True))
    gates = z / z.sum(axis=1, keepdims=True)
    return order.astype(np.int32), gates.astype(np.float32)


def uniform_distinct_routing(T: int, E: int, k: int, key):
    """k distinct experts per token, uniform over all k-subsets (Gumbel
    top-k over equal scores); no gates."""
    g = _rng(*key).gumbel(size=(T, E))
    idx = np.argsort(-g, axis=1, kind="stable")[:, :k]
    return idx.astype(np.int32)


def zipf_routing(T: int, E: int, k: int, s: float, n_dead: int, key):
    """Zipf(s)-skewed expert popularity with ``n_dead`` experts that nobody
    picks.  Live expert of popularity rank i (1-based) has p ~ i^-s; a seeded
    permutation maps ranks to expert ids (the last n_dead ids of that
    permutation are the dead experts).  k distinct experts per token by
    Gumbel top-k over log p; gates = softmax over the k picked scores.
    """
    rng = _rng(*key)
    perm = rng.permutation(E)
    live = E - n_dead
    logp = np.full(E, -np.inf)
    ranks = np.arange(1, live + 1, dtype=np.float64)
    logp[perm[:live]] = -s * np.log(ranks)
    scores = logp[None, :] + rng.gumbel(size=(T, E))
    idx, gates = topk_softmax_routing(scores, k)
    return idx, gates


# --------------------------------------------------------------------------
# Workload container
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    kind: str            # "mlp" | "pl" | "moa"
    dtype: str           # "f32" | "bf16"
    T: int
    E: int
    k: int
    dims: Dict[str, int]
    act: Optional[str]   # "gelu" | "swiglu" | None
    tensors: Dict[str, np.ndarray]

    @property
    def M(self) -> int:
        return self.T * self.k

    def f32(self, name: str) -> np.ndarray:
        """The named float tensor as float32 values (bf16 bits decoded)."""
        a = self.tensors[name]
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


CONFIGS = {
    # id: (kind, description)
    1: ("mlp", "tiny SMoE-MLP fp32, T=256 d=128 d_ff=256 E=8 k=2, GELU"),
    2: ("pl", "single ParallelLinear bf16, T=8192 2048->2048 E=16 k=2"),
    3: ("mlp", "Mixtral-shaped SMoE-MLP bf16, T=16384 d=4096 d_ff=14336 E=8 k=2, SwiGLU"),
    4: ("mlp", "high-granularity SMoE-MLP bf16, T=16384 d=1024 d_ff=512 E=64 k=8, Zipf(1.1), GELU"),
    5: ("moa", "MoA projections bf16, T=8192 d=2048 E=16 head_dim=128 k=4"),
}


def make_mlp(T, d, f, E, k, act, dtype, cid, routing="softmax", w_std=None,
             x_std=1.0, zipf_s=1.1, n_dead=0, gate_matrix=False) -> Workload:
    """SMoE-MLP workload: x [T,d]; W1 (and W3 for SwiGLU) [E,d,f];
    W2 [E,f,d]; routing (expert_idxs [T,k], gates [T,k]); dout [T,d]."""
    big = E * d * f > (1 << 22)
    t: Dict[str, np.ndarray] = {}
    t["x"] = _normal((T, d), x_std, (cid, 0), dtype)
    std1 = w_std if w_std is not None else d ** -0.5
    std2 = w_std if w_std is not None else f ** -0.5
    t["w1"] = _normal((E, d, f), std1, (cid, 1), dtype, per_expert=big)
    t["w2"] = _normal((E, f, d), std2, (cid, 2), dtype, per_expert=big)
    if act == "swiglu":
        t["w3"] = _normal((E, d, f), std1, (cid, 3), dtype, per_expert=big)
    if routing == "gate":
        # logits from a seeded [d,E] gate matrix applied to the (stored) x
        G = _rng(cid, 4).standard_normal((d, E), dtype=np.float32) * np.float32(d ** -0.5)
        xs = bf16_bits_to_f32(t["x"]) if dtype == "bf16" else t["x"]
        logits = xs.astype(np.float64) @ G.astype(np.float64)
        t["gate_w"] = G
        t["logits"] = logits.astype(np.float32)
        t["expert_idxs"], t["gates"] = topk_softmax_routing(logits, k)
    elif routing == "softmax":
        logits = _rng(cid, 4).standard_normal((T, E), dtype=np.float32)
        t["logits"] = logits
        t["expert_idxs"], t["gates"] = topk_softmax_routing(logits, k)
    elif routing == "zipf":
        t["expert_idxs"], t["gates"] = zipf_routing(T, E, k, zipf_s, n_dead, (cid, 4))
    else:
        raise ValueError(routing)
    t["dout"] = _normal((T, d), 1.0, (cid, 5), dtype)
    return Workload(f"mlp{cid}", "mlp", dtype, T, E, k,
                    {"d_model": d, "d_ff": f}, act, t)


def make_pl(T, d_in, d_out, E, k, dtype, cid, x_std=0.02, w_std=0.02,
            with_gates=False) -> Workload:
    """ParallelLinear workload: scattered x [T,d_in], grouped x [T*k,d_in],
    W [E,d_in,d_out], distinct uniform expert pairs, upstream dy [T*k,d_out]
    (and dy_comb [T,d_out] with gates when ``with_gates``)."""
    big = E * d_in * d_out > (1 << 22)
    t: Dict[str, np.ndarray] = {}
    t["x"] = _normal((T, d_in), x_std, (cid, 0), dtype)
    t["x_grouped"] = _normal((T * k, d_in), x_std, (cid, 6), dtype)
    t["w"] = _normal((E, d_in, d_out), w_std, (cid, 1), dtype, per_expert=big)
    t["expert_idxs"] = uniform_distinct_routing(T, E, k, (cid, 4))
    if with_gates:
        logits = _rng(cid, 7).standard_normal((T, E), dtype=np.float32)
        idx, gates = topk_softmax_routing(logits, k)
        t["expert_idxs"], t["gates"] = idx, gates
        t["dy_comb"] = _normal((T, d_out), 1.0, (cid, 8), dtype)
    t["dy"] = _normal((T * k, d_out), 1.0, (cid, 5), dtype)
    return Workload(f"pl{cid}", "pl", dtype, T, E, k,
                    {"d_in": d_in, "d_out": d_out}, None, t)


def make_moa(T, d, hd, E, k, dtype, cid, w_std=0.02) -> Workload:
    """Mixture-of-Attention projection workload: X [T,d]; Wq [E,d,hd];
    Wo [E,hd,d]; grouped attention output O_in [T*k,hd]; router top-k
    softmax over N(0,1) logits [T,E]; upstream dQ [T*k,hd] (grouped) and
    dOut [T,d]."""
    t: Dict[str, np.ndarray] = {}
    t["x"] = _normal((T, d), 1.0, (cid, 0), dtype)
    t["wq"] = _normal((E, d, hd), w_std, (cid, 1), dtype)
    t["wo"] = _normal((E, hd, d), w_std, (cid, 2), dtype)
    t["o_in"] = _normal((T * k, hd), 1.0, (cid, 3), dtype)
    logits = _rng(cid, 4).standard_normal((T, E), dtype=np.float32)
    t["logits"] = logits
    t["expert_idxs"], t["gates"] = topk_softmax_routing(logits, k)
    t["dq"] = _normal((T * k, hd), 1.0, (cid, 5), dtype)
    t["dout"] = _normal((T, d), 1.0, (cid, 6), dtype)
    return Workload(f"moa{cid}", "moa", dtype, T, E, k,
                    {"d_model": d, "head_dim": hd}, None, t)


def make_router(T, d, E, k, dtype, cid, x_std=1.0) -> Workload:
    """Router workload: x [T,d] ~ N(0, x_std^2); gate matrix G [d,E] ~
    N(0, 1/d) (logits of unit scale); upstream dgates [T,k] ~ N(0,1) fp32
    and an incoming dx [T,d] ~ N(0,1) for the accumulate form."""
    t: Dict[str, np.ndarray] = {}
    t["x"] = _normal((T, d), x_std, (cid, 0), dtype)
    t["gate_w"] = _normal((d, E), d ** -0.5, (cid, 1), dtype)
    t["dgates"] = _normal((T, k), 1.0, (cid, 2), "f32")
    t["dx_in"] = _normal((T, d), 1.0, (cid, 3), dtype)
    return Workload(f"router{cid}", "router", dtype, T, E, k,
                    {"d_model": d}, None, t)


def make_moa_attention(B, S, hd, E, k, dtype, cid) -> Workload:
    """Mixture-of-Attention core workload: B sequences of S tokens; grouped
    queries q [T*k, hd] ~ N(0,1) (the Q projection's grouped output), shared
    keys and values [T, hd] ~ N(0,1) (dense, as the MoA workload gives
    them), top-k softmax routing over N(0,1) logits [T, E], upstream do
    [T*k, hd] ~ N(0,1)."""
    T = B * S
    t: Dict[str, np.ndarray] = {}
    t["q"] = _normal((T * k, hd), 1.0, (cid, 0), dtype)
    t["k"] = _normal((T, hd), 1.0, (cid, 1), dtype)
    t["v"] = _normal((T, hd), 1.0, (cid, 2), dtype)
    logits = _rng(cid, 3).standard_normal((T, E), dtype=np.float32)
    t["expert_idxs"], t["gates"] = topk_softmax_routing(logits, k)
    t["do"] = _normal((T * k, hd), 1.0, (cid, 4), dtype)
    return Workload(f"moa_attn{cid}", "moa_attn", dtype, T, E, k,
                    {"seq_len": S, "head_dim": hd, "batch": B}, None, t)


def make_moa_layer(B, S, d, hd, E, k, dtype, cid, w_std=0.02) -> Workload:
    """A whole Mixture-of-Attention layer: x [T, d] ~ N(0,1); per-head-expert
    Wq [E, d, hd] and Wo [E, hd, d] ~ N(0, w_std^2); shared keys and values
    [T, hd] ~ N(0,1); top-k softmax routing over N(0,1) logits; upstream
    dout [T, d] ~ N(0,1).  T = B * S."""
    T = B * S
    t: Dict[str, np.ndarray] = {}
    t["x"] = _normal((T, d), 1.0, (cid, 0), dtype)
    t["wq"] = _normal((E, d, hd), w_std, (cid, 1), dtype)
    t["wo"] = _normal((E, hd, d), w_std, (cid, 2), dtype)
    t["k"] = _normal((T, hd), 1.0, (cid, 3), dtype)
    t["v"] = _normal((T, hd), 1.0, (cid, 4), dtype)
    logits = _rng(cid, 5).standard_normal((T, E), dtype=np.float32)
    t["expert_idxs"], t["gates"] = topk_softmax_routing(logits, k)
    t["dout"] = _normal((T, d), 1.0, (cid, 6), dtype)
    return Workload(f"moa_layer{cid}", "moa_layer", dtype, T, E, k,
                    {"seq_len": S, "batch": B, "d_model": d, "head_dim": hd}, None, t)


def make_config(cid: int) -> Workload:
    """The five named workloads, shapes and distributions as stated."""
    if cid == 1:
        return make_mlp(256, 128, 256, 8, 2, "gelu", "f32", 1, routing="gate")
    if cid == 2:
        return make_pl(8192, 2048, 2048, 16, 2, "bf16", 2)
    if cid == 3:
        return make_mlp(16384, 4096, 14336, 8, 2, "swiglu", "bf16", 3,
                        routing="softmax", w_std=0.02)
    if cid == 4:
        return make_mlp(16384, 1024, 512, 64, 8, "gelu", "bf16", 4,
                        routing="zipf", w_std=0.02, zipf_s=1.1, n_dead=8)
    if cid == 5:
        return make_moa(8192, 2048, 128, 16, 4, "bf16", 5)
    raise KeyError(cid)
