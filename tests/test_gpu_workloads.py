"""The three large bf16 workloads on the GPU, at their full sizes and in the
launch configuration the benchmark uses, against the oracle on sampled
outputs:

* Mixtral-shaped SMoE-MLP (T=16384, d_model=4096, d_ff=14336, E=8, k=2,
  SwiGLU): out, dx and dgates rows of sampled tokens; dW1 / dW3 column
  slices and dW2 row slices over every token; routing arrays in full.
* high-granularity SMoE-MLP (T=16384, d_model=1024, d_ff=512, E=64, k=8,
  Zipf routing with empty experts, GELU): the same samples; empty experts
  get exactly zero weight gradients.
* Mixture-of-Attention projections (T=8192, d_model=2048, 16 head experts
  of 128, k=4): Q = scattered-in / grouped-out, O = grouped-in /
  scattered-out with the gate-weighted combine, forward and backward.

Each token's outputs depend only on that token and the weights, and a
column of the hidden layer only on that column of W1 (W3) and row of W2, so
the samples are exact oracle values, not approximations."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import BF16_TOL, host, rel_err, rel_err_stored_bf16, say, upload
from workloads import make_config

pytestmark = pytest.mark.gpu


def _sample(n, count, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, count, replace=False)]))


def _check_mlp_workload(smoe, cid, n_tokens, n_cols, seed):
    w = make_config(cid)
    T, k, E = w.T, w.k, w.E
    d, f, act = w.dims["d_model"], w.dims["d_ff"], w.act
    say(f"workload {cid}: T={T} d={d} d_ff={f} E={E} k={k} {act}")
    dd = upload(w, ["x", "w1", "w2", "w3", "expert_idxs", "gates", "dout"])
    out, saved = smoe.smoe_mlp_fwd(dd["x"], dd["w1"], dd["w2"], dd["expert_idxs"], dd["gates"], act,
                                   w3=dd.get("w3"))
    g = smoe.smoe_mlp_bwd(dd["dout"], dd["x"], dd["w1"], dd["w2"], dd["expert_idxs"], dd["gates"], act, saved,
                          w3=dd.get("w3"))
    torch.cuda.synchronize()
    v = smoe.saved_views(saved, T, k, E, d, f, act, torch.bfloat16)
    idx = w.tensors["expert_idxs"]
    r = oracle.route(idx, E)
    for n in ("sorted_expert_idxs", "sorted_scattered_idxs", "counts", "offsets"):
        np.testing.assert_array_equal(v[n].cpu().numpy(), r[n])
    got = {"out": host(out), "dx": host(g["dx"]), "dgates": host(g["dgates"])}
    dws = {n: host(g[n]) for n in ("dw1", "dw2", "dw3") if g.get(n) is not None}
    del dd, out, saved, g, v
    torch.cuda.empty_cache()

    f64 = lambda n: w.f32(n).astype(np.float64)
    x, w1, w2, dout = f64("x"), f64("w1"), f64("w2"), f64("dout")
    w3 = f64("w3") if act == "swiglu" else None
    gates = w.tensors["gates"].astype(np.float64)
    toks = _sample(T, n_tokens, seed)
    say(f"  oracle on {toks.size} tokens")
    ref_out = oracle.mlp_fwd(x, w1, w2, idx, gates, act, w3=w3, storage="bf16", tokens=toks)
    ref = oracle.mlp_bwd(x, w1, w2, idx, gates, act, dout, w3=w3, storage="bf16", tokens=toks)
    for name, want in (("out", ref_out), ("dx", ref["dx"]), ("dgates", ref["dgates"])):
        # out and dx are stored in bf16, dgates in fp32
        metric = rel_err if name == "dgates" else rel_err_stored_bf16
        e = metric(got[name][toks], want[toks])
        say(f"  {name} err {e:.2e} (plain max err / RMS {rel_err(got[name][toks], want[toks]):.2e})")
        assert e <= BF16_TOL, name
    cols = _sample(f, n_cols, seed + 1)
    say(f"  oracle weight-gradient slices on {cols.size} hidden columns")
    rc = oracle.mlp_dw_cols(x, w1, w2, idx, gates, act, dout, cols, w3=w3, storage="bf16")
    slices = {"dw1": dws["dw1"][:, :, cols], "dw2": dws["dw2"][:, cols, :]}
    if act == "swiglu":
        slices["dw3"] = dws["dw3"][:, :, cols]
    for name, gs in slices.items():
        e = rel_err(gs, rc[name])
        say(f"  {name}[cols] err {e:.2e}")
        assert e <= BF16_TOL, name
    empty = np.nonzero(r["counts"] == 0)[0]
    for name, full in dws.items():
        assert np.all(full[empty] == 0.0), name
        assert np.all(np.isfinite(full)), name
    return r["counts"]


def test_mixtral_shaped_mlp(smoe):
    _check_mlp_workload(smoe, 3, n_tokens=10, n_cols=14, seed=301)


def test_high_granularity_zipf_mlp(smoe):
    counts = _check_mlp_workload(smoe, 4, n_tokens=62, n_cols=30, seed=401)
    assert (counts == 0).sum() >= 1 and counts.max() > 0.10 * 16384


def test_moa_projections(smoe):
    """Q: X [T,2048] scattered (read k times) -> grouped [T*k,128];
    O: grouped [T*k,128] -> scattered, combined with the gates -> [T,2048];
    forward and backward of both."""
    w = make_config(5)
    T, k, E = w.T, w.k, w.E
    say(f"MoA projections T={T} E={E} k={k}")
    dd = upload(w, ["x", "wq", "wo", "o_in", "dq", "dout", "gates", "expert_idxs"])
    rt = smoe.smoe_route(dd["expert_idxs"], E)
    s, off = rt["sorted_scattered_idxs"], rt["offsets"]
    q = smoe.smoe_parallel_linear_fwd(dd["x"], dd["wq"], T, k, s, off, False, True)
    dx, dwq, _ = smoe.smoe_parallel_linear_bwd(dd["x"], dd["wq"], T, k, s, off, False, True, dd["dq"])
    o = smoe.smoe_parallel_linear_fwd(dd["o_in"], dd["wo"], T, k, s, off, True, False, dd["gates"])
    doin, dwo, dg = smoe.smoe_parallel_linear_bwd(dd["o_in"], dd["wo"], T, k, s, off, True, False, dd["dout"],
                                                  dd["gates"], need_dgates=True)
    torch.cuda.synchronize()
    got = {n: host(t) for n, t in (("q", q), ("dx", dx), ("dwq", dwq), ("o", o), ("doin", doin), ("dwo", dwo),
                                  ("dg", dg))}
    idx = w.tensors["expert_idxs"]
    r = oracle.route(idx, E)
    np.testing.assert_array_equal(s.cpu().numpy(), r["sorted_scattered_idxs"])
    np.testing.assert_array_equal(off.cpu().numpy(), r["offsets"])
    f64 = lambda n: w.f32(n).astype(np.float64)
    gates = w.tensors["gates"].astype(np.float64)
    x, wq, wo, o_in = f64("x"), f64("wq"), f64("wo"), f64("o_in")
    toks = _sample(T, 200, 501)
    rinv = oracle.grouped_position(r["sorted_scattered_idxs"])
    grows = np.array([rinv[t * k + j] for t in toks for j in range(k)])
    hcols = _sample(128, 10, 502)
    dcols = _sample(2048, 14, 503)

    ref_q = oracle.parallel_linear_fwd(x, wq, idx, False, True, tokens=toks)
    rdx, rdwq, _ = oracle.parallel_linear_bwd(x, wq, idx, False, True, f64("dq"), storage="bf16", tokens=toks,
                                              dw_cols=hcols)
    ref_o = oracle.parallel_linear_fwd(o_in, wo, idx, True, False, gates=gates, tokens=toks)
    rdoin, rdwo, rdg = oracle.parallel_linear_bwd(o_in, wo, idx, True, False, f64("dout"), gates=gates,
                                                  storage="bf16", tokens=toks, dw_cols=dcols)
    # q, dx, o and doin are stored in bf16; the weight and gate gradients in fp32
    for name, a, b, stored in (("q", got["q"][grows], ref_q[grows], True), ("dx", got["dx"][toks], rdx[toks], True),
                               ("dwq[cols]", got["dwq"][:, :, hcols], rdwq, False),
                               ("o", got["o"][toks], ref_o[toks], True),
                               ("doin", got["doin"][grows], rdoin[grows], True),
                               ("dwo[cols]", got["dwo"][:, :, dcols], rdwo, False),
                               ("dgates", got["dg"][toks], rdg[toks], False)):
        e = rel_err_stored_bf16(a, b) if stored else rel_err(a, b)
        say(f"  {name} err {e:.2e} (plain max err / RMS {rel_err(a, b):.2e})")
        assert e <= BF16_TOL, name
