"""smoe_router_fwd / smoe_router_bwd on the GPU against the oracle.

The oracle reads the gate matrix as G [d, E] (logits = x G); the library
takes it as w = G^T [E, d] and returns dw = dG^T.  The GPU forms the logits
in fp32 from the stored inputs, the oracle in fp64.  Each logit's error is
bounded by (ceil(d/64) + 24) * 2^-24 * sum_i |x_i g_ie|: the products are
exact (bf16 x bf16, or fp32 rounded once), each lane or matrix-core
accumulator adds at most ceil(d/64) partial sums in sequence, a matrix-core
step sums 16 products before adding them, and the final cross-lane or
cross-wave sums add at most 6 more.  A token's choice is unique where the
gaps between its sorted oracle logits, down to the (k+1)-th, exceed twice
that bound: there the expert ids must match exactly; elsewhere the GPU's
choice must be a valid top-k (distinct ids whose oracle logits lie within
the bound of the sorted ones).  The gates are checked against the softmax of
the oracle's logits at the GPU's ids.  The backward takes the oracle's
forward choice as input on both sides; dw is fp32 (tolerance 1e-4 of its
RMS), dx is in the input dtype: fp32 is held to 1e-4 of its RMS; bf16 dx is
a named exception to the plain 2e-2 bound (tokens with large dlogits put
elements far above the RMS, whose own bf16 rounding exceeds 2e-2 RMS): it is
held to 1e-4 RMS beyond its final rounding, and its plain error printed."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import F32_TOL, dev_tensor, host, rel_err, rel_err_beyond_bf16_rounding, say
from workloads import bf16_bits_to_f32, make_config, make_router

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def wt_tensor(g: np.ndarray) -> torch.Tensor:
    """The oracle's G [d, E] as the library's gate weight w = G^T [E, d]."""
    return dev_tensor(np.ascontiguousarray(g.T))


def logit_bound(x, g):
    d = x.shape[1]
    return (-(-d // 64) + 24) * U32 * (np.abs(x) @ np.abs(g))


def check_fwd(smoe, x, g, k, xd, gd):
    T, E = x.shape[0], g.shape[1]
    r = smoe.smoe_router_fwd(xd, gd, k, want_logits=True)
    torch.cuda.synchronize()
    ref = oracle.router_fwd(x, g, k)
    bound = logit_bound(x, g)
    lg = host(r["logits"])
    assert lg.shape == (T, E)
    assert np.all(np.abs(lg - ref["logits"]) <= bound), float(np.max(np.abs(lg - ref["logits"]) - bound))
    idx = r["expert_idxs"].cpu().numpy()
    gates = host(r["gates"])
    if T == 0:
        return r, ref
    # unique choices: every gap down to the (k+1)-th sorted logit is wide
    zs = -np.sort(-ref["logits"], axis=1)
    tb = bound.max(axis=1, keepdims=True)
    nk = min(k + 1, E)
    gaps = zs[:, :nk - 1] - zs[:, 1:nk]
    unique = np.all(gaps > 2 * tb, axis=1) if nk > 1 else np.ones(T, bool)
    say(f"  {unique.sum()}/{T} tokens with a unique choice")
    np.testing.assert_array_equal(idx[unique], ref["expert_idxs"][unique])
    # the rest: a valid top-k within the bound
    assert np.all((idx >= 0) & (idx < E))
    assert np.all(np.sort(idx, axis=1)[:, 1:] != np.sort(idx, axis=1)[:, :-1])
    z_at = np.take_along_axis(ref["logits"], idx.astype(np.int64), axis=1)
    assert np.all(np.abs(z_at - zs[:, :k]) <= 2 * tb)
    # gates: softmax of the oracle logits at the GPU's choice
    w = np.exp(z_at - z_at.max(axis=1, keepdims=True))
    want = w / w.sum(axis=1, keepdims=True)
    gerr = np.abs(gates - want).max()
    say(f"  gates max abs err {gerr:.2e}")
    assert gerr <= 4 * tb.max() + 1e-6
    return r, ref


def check_bwd(smoe, x, g, ref_fwd, dgates, xd, gd, dtype, dx_in=None, dx_in_d=None):
    idx = ref_fwd["expert_idxs"]
    gates32 = ref_fwd["gates"].astype(np.float32)
    dev = xd.device
    dg, dx = smoe.smoe_router_bwd(xd, gd, torch.from_numpy(idx).to(dev), torch.from_numpy(gates32).to(dev),
                                  torch.from_numpy(dgates).to(dev),
                                  dx=dx_in_d, accumulate=dx_in_d is not None)
    torch.cuda.synchronize()
    rb = oracle.router_bwd(x, g, idx, gates32.astype(np.float64), dgates.astype(np.float64))
    e = rel_err(host(dg), rb["dG"].T)
    say(f"  dw err {e:.2e}")
    assert e <= F32_TOL
    want_dx = rb["dx"] + (dx_in if dx_in is not None else 0.0)
    got_dx = host(dx)
    e = rel_err(got_dx, want_dx)
    if dtype == "f32":
        say(f"  dx max err / RMS {e:.2e}")
    else:
        plain, e = e, rel_err_beyond_bf16_rounding(got_dx, want_dx)
        say(f"  dx max err / RMS {plain:.2e} (named exception; beyond its bf16 rounding {e:.2e})")
    assert e <= F32_TOL
    return dg, dx


def run_case(smoe, T, d, E, k, dtype, cid, accumulate=False):
    say(f"router T={T} d={d} E={E} k={k} {dtype} acc={accumulate}")
    w = make_router(T, d, E, k, dtype, cid)
    x = w.f32("x").astype(np.float64)
    g = w.f32("gate_w").astype(np.float64)
    xd, gd = dev_tensor(w.tensors["x"]), wt_tensor(w.tensors["gate_w"])
    _, ref = check_fwd(smoe, x, g, k, xd, gd)
    dx_in = w.f32("dx_in").astype(np.float64) if accumulate else None
    dx_in_d = dev_tensor(w.tensors["dx_in"]) if accumulate else None
    return check_bwd(smoe, x, g, ref, w.tensors["dgates"], xd, gd, dtype, dx_in, dx_in_d)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1000, 200, 6, 3), (517, 72, 64, 8), (300, 136, 13, 1), (64, 64, 8, 8)])
def test_router_ragged(smoe, dtype, shape):
    T, d, E, k = shape
    run_case(smoe, T, d, E, k, dtype, 300 + E)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_router_accumulate(smoe, dtype):
    run_case(smoe, 777, 320, 16, 4, dtype, 320, accumulate=True)


def test_router_tiny_workload_reproduces_its_routing(smoe):
    """The tiny fp32 workload (T=256, d=128, E=8, k=2) draws its routing
    from a gate matrix: the router on that x and G gives the same ids."""
    w = make_config(1)
    x = w.f32("x").astype(np.float64)
    g = w.tensors["gate_w"].astype(np.float64)
    r, ref = check_fwd(smoe, x, g, w.k, dev_tensor(w.tensors["x"]), wt_tensor(w.tensors["gate_w"]))
    np.testing.assert_array_equal(ref["expert_idxs"], w.tensors["expert_idxs"])


def test_router_single_expert(smoe):
    """E = k = 1: every token picks expert 0 with gate 1; no gradient."""
    say("router E=k=1")
    w = make_router(100, 96, 1, 1, "f32", 331)
    xd, gd = dev_tensor(w.tensors["x"]), wt_tensor(w.tensors["gate_w"])
    r = smoe.smoe_router_fwd(xd, gd, 1)
    assert np.all(r["expert_idxs"].cpu().numpy() == 0)
    assert np.all(r["gates"].cpu().numpy() == 1.0)
    dg, dx = smoe.smoe_router_bwd(xd, gd, r["expert_idxs"], r["gates"], dev_tensor(w.tensors["dgates"]))
    assert np.all(dg.cpu().numpy() == 0.0) and np.all(dx.cpu().numpy() == 0.0)


def test_router_no_tokens(smoe):
    say("router T=0")
    x = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    g = torch.randn((8, 64), dtype=torch.float32, device="cuda")
    r = smoe.smoe_router_fwd(x, g, 2, want_logits=True)
    assert r["expert_idxs"].shape == (0, 2) and r["logits"].shape == (0, 8)
    dg, dx = smoe.smoe_router_bwd(x, g, r["expert_idxs"], r["gates"], torch.empty((0, 2), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert dx.shape == (0, 64) and dg.shape == (8, 64) and np.all(dg.cpu().numpy() == 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("E", [8, 40])
def test_router_ties_go_to_lower_expert(smoe, dtype, E):
    """Equal logits (repeated gate columns): the lower id wins, in order."""
    say(f"router ties {dtype} E={E}")
    T, d, k = 200, 64, 4
    w = make_router(T, d, E, k, dtype, 332)
    gm = w.tensors["gate_w"].copy()
    gm[:, 5] = gm[:, 2]
    gm[:, 7] = gm[:, 2]
    gm[:, 6] = gm[:, 1]
    x = w.f32("x").astype(np.float64)
    g = bf16_bits_to_f32(gm) if dtype == "bf16" else gm
    r, ref = check_fwd(smoe, x, g.astype(np.float64), k, dev_tensor(w.tensors["x"]), wt_tensor(gm))
    idx = r["expert_idxs"].cpu().numpy()
    # bitwise-equal columns give bitwise-equal fp32 logits: exact tie order
    for t in range(T):
        pos = {e: j for j, e in enumerate(idx[t])}
        for lo, hi in ((2, 5), (2, 7), (5, 7), (1, 6)):
            if lo in pos and hi in pos:
                assert pos[lo] < pos[hi], (t, idx[t])
            assert not (hi in pos and lo not in pos), (t, idx[t])


def test_router_deterministic(smoe):
    say("router determinism")
    w = make_router(3000, 1024, 16, 2, "bf16", 333)
    xd, gd = dev_tensor(w.tensors["x"]), wt_tensor(w.tensors["gate_w"])
    a = smoe.smoe_router_fwd(xd, gd, 2, want_logits=True)
    b = smoe.smoe_router_fwd(xd, gd, 2, want_logits=True)
    for n in a:
        assert torch.equal(a[n], b[n]), n
    dgs = dev_tensor(w.tensors["dgates"])
    dg1, dx1 = smoe.smoe_router_bwd(xd, gd, a["expert_idxs"], a["gates"], dgs)
    dg2, dx2 = smoe.smoe_router_bwd(xd, gd, a["expert_idxs"], a["gates"], dgs)
    assert torch.equal(dg1, dg2) and torch.equal(dx1, dx2)


@pytest.mark.parametrize("shape", [(16384, 4096, 8, 2), (16384, 1024, 64, 8), (8192, 2048, 16, 4)])
def test_router_full_size(smoe, shape):
    """The routers of the Mixtral-shaped, high-granularity and MoA
    workloads at their full token counts, bf16, in full."""
    T, d, E, k = shape
    run_case(smoe, T, d, E, k, "bf16", 340 + E)


def test_full_chain_tiny_workload(smoe):
    """The tiny fp32 workload end to end on the GPU: router -> SMoE-MLP
    forward -> MLP backward -> router backward, the router's dx added to the
    MLP's; every output against the oracle's same chain."""
    say("full chain, tiny fp32 workload")
    w = make_config(1)
    f = lambda n: w.f32(n).astype(np.float64)
    x, G, w1, w2, dout = f("x"), w.tensors["gate_w"].astype(np.float64), f("w1"), f("w2"), f("dout")
    rf = oracle.router_fwd(x, G, w.k)
    ref_out = oracle.mlp_fwd(x, w1, w2, rf["expert_idxs"], rf["gates"], w.act, storage="f64")
    mb = oracle.mlp_bwd(x, w1, w2, rf["expert_idxs"], rf["gates"], w.act, dout, storage="f64")
    rb = oracle.router_bwd(x, G, rf["expert_idxs"], rf["gates"], mb["dgates"])

    xd, wt = dev_tensor(w.tensors["x"]), wt_tensor(w.tensors["gate_w"])
    w1d, w2d, doutd = dev_tensor(w.tensors["w1"]), dev_tensor(w.tensors["w2"]), dev_tensor(w.tensors["dout"])
    r = smoe.smoe_router_fwd(xd, wt, w.k)
    out, saved = smoe.smoe_mlp_fwd(xd, w1d, w2d, r["expert_idxs"], r["gates"], w.act)
    g = smoe.smoe_mlp_bwd(doutd, xd, w1d, w2d, r["expert_idxs"], r["gates"], w.act, saved)
    dwg, dx = smoe.smoe_router_bwd(xd, wt, r["expert_idxs"], r["gates"], g["dgates"], dx=g["dx"], accumulate=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(r["expert_idxs"].cpu().numpy(), rf["expert_idxs"])
    checks = {"out": (out, ref_out), "gates": (r["gates"], rf["gates"]), "dgates": (g["dgates"], mb["dgates"]),
              "dw1": (g["dw1"], mb["dw1"]), "dw2": (g["dw2"], mb["dw2"]), "dG": (dwg, rb["dG"].T),
              "dx": (dx, mb["dx"] + rb["dx"])}
    for n, (got, want) in checks.items():
        e = rel_err(host(got), want)
        say(f"  {n} err {e:.2e}")
        assert e <= F32_TOL, n


def test_router_bwd_many_tokens(smoe):
    """9 M tokens: more 128-token chunks than the dx grid's y extent, so
    blocks stride over chunks.  dx is per-token, checked against the oracle
    on sampled tokens; dw against the property that each token's dlogits sum
    to zero when its gates do (so every column of dw sums to ~0 over
    experts), relative to the column's size."""
    from workloads import bf16_bits, topk_softmax_routing
    T, d, E, k = 9_000_000, 8, 4, 2
    say(f"router bwd T={T} d={d} E={E} k={k} bf16")
    rng = np.random.default_rng([345, 0])
    xb = bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
    wb = bf16_bits(rng.standard_normal((E, d), dtype=np.float32) * np.float32(d ** -0.5))
    idx, gates = topk_softmax_routing(rng.standard_normal((T, E), dtype=np.float32), k)
    dgates = rng.standard_normal((T, k), dtype=np.float32)
    dev = lambda a: torch.from_numpy(a).cuda()
    xd = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).cuda()
    wd = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).cuda()
    dw, dx = smoe.smoe_router_bwd(xd, wd, dev(idx), dev(gates), dev(dgates))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(7).choice(T, 4000, replace=False))
    rows = np.concatenate([rows, np.arange(T - 300, T)])   # the last chunks too
    x64 = (xb[rows].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g64 = ((wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)).T   # G [d, E]
    rb = oracle.router_bwd(x64, g64, idx[rows], gates[rows].astype(np.float64), dgates[rows].astype(np.float64))
    got_dx = host(dx[torch.from_numpy(rows).cuda()])
    e = rel_err_beyond_bf16_rounding(got_dx, rb["dx"])
    say(f"  dx (sampled) max err / RMS {rel_err(got_dx, rb['dx']):.2e} (named exception; beyond its bf16 rounding "
        f"{e:.2e})")
    assert e <= F32_TOL
    dwh = host(dw)
    scale = np.abs(dwh).sum(axis=0)
    colsum = np.abs(dwh.sum(axis=0))
    say(f"  max |sum_e dw| / sum_e |dw| = {float((colsum / scale).max()):.2e}")
    assert np.all(colsum <= 1e-3 * scale)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_router_large_logits(smoe, dtype):
    """x scaled by 64 (exact in bf16 and fp32): logits of size ~64, so
    exp of an unshifted logit would overflow fp32; the softmax over the
    chosen k must shift by the top one.  Choices, gates, dw and dx against
    the oracle, everything finite."""
    T, d, E, k = 500, 256, 16, 4
    say(f"router large logits T={T} d={d} E={E} k={k} {dtype}")
    w = make_router(T, d, E, k, dtype, 360)
    x = w.f32("x").astype(np.float64) * 64.0
    g = w.f32("gate_w").astype(np.float64)
    xd, gd = dev_tensor(w.tensors["x"]) * 64, wt_tensor(w.tensors["gate_w"])
    assert np.array_equal(host(xd), x)
    assert np.abs(x @ g).max() > 88.0          # exp(88.7) is the fp32 limit
    r, ref = check_fwd(smoe, x, g, k, xd, gd)
    assert torch.isfinite(r["gates"]).all()
    dw, dx = check_bwd(smoe, x, g, ref, w.tensors["dgates"], xd, gd, dtype)
    assert torch.isfinite(dw).all() and torch.isfinite(dx.float()).all()
