"""smoe_mlp_fwd / smoe_mlp_bwd on the GPU against the oracle: GELU and
SwiGLU, fp32 and bf16, ragged tiles, empty experts; the tiny fp32 workload
in full; saved routing arrays bit-exact; determinism across runs."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import BF16_TOL, F32_TOL, dev_tensor, host, rel_err, say, upload
from workloads import make_config, make_mlp

pytestmark = pytest.mark.gpu


def run_mlp(smoe, w):
    d = upload(w)
    out, saved = smoe.smoe_mlp_fwd(d["x"], d["w1"], d["w2"], d["expert_idxs"], d["gates"], w.act, w3=d.get("w3"))
    g = smoe.smoe_mlp_bwd(d["dout"], d["x"], d["w1"], d["w2"], d["expert_idxs"], d["gates"], w.act, saved,
                          w3=d.get("w3"))
    torch.cuda.synchronize()
    return out, saved, g


def check_full(smoe, w):
    tol = F32_TOL if w.dtype == "f32" else BF16_TOL
    storage = "f64" if w.dtype == "f32" else "bf16"
    out, saved, g = run_mlp(smoe, w)
    f = lambda n: w.f32(n).astype(np.float64)
    w3 = f("w3") if w.act == "swiglu" else None
    idx, gates = w.tensors["expert_idxs"], w.tensors["gates"].astype(np.float64)
    ref = oracle.mlp_fwd(f("x"), f("w1"), f("w2"), idx, gates, w.act, w3=w3, storage=storage)
    e = rel_err(host(out), ref)
    say(f"  out err {e:.2e}")
    assert e <= tol
    rg = oracle.mlp_bwd(f("x"), f("w1"), f("w2"), idx, gates, w.act, f("dout"), w3=w3, storage=storage)
    names = ["dx", "dw1", "dw2", "dgates"] + (["dw3"] if w.act == "swiglu" else [])
    for n in names:
        e = rel_err(host(g[n]), rg[n])
        say(f"  {n} err {e:.2e}")
        assert e <= tol, n
    # routing arrays saved by the forward are the oracle's, bit for bit
    v = smoe.saved_views(saved, w.T, w.k, w.E, w.dims["d_model"], w.dims["d_ff"], w.act,
                         torch.float32 if w.dtype == "f32" else torch.bfloat16)
    r = oracle.route(idx, w.E)
    for n in ("sorted_expert_idxs", "sorted_scattered_idxs", "counts", "offsets"):
        np.testing.assert_array_equal(v[n].cpu().numpy(), r[n])
    return out, g


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_mlp_small(smoe, dtype, act):
    say(f"mlp small {dtype} {act}")
    w = make_mlp(300, 136, 200, 6, 2, act, dtype, 130, routing="softmax", w_std=0.08)
    check_full(smoe, w)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_mlp_empty_experts_and_skew(smoe, act):
    say(f"mlp zipf empty experts bf16 {act}")
    w = make_mlp(1200, 128, 256, 12, 3, act, "bf16", 131, routing="zipf", w_std=0.05, n_dead=3)
    cnt = np.bincount(w.tensors["expert_idxs"].reshape(-1), minlength=12)
    assert (cnt == 0).sum() == 3
    out, g = check_full(smoe, w)
    dead = np.nonzero(cnt == 0)[0]
    assert np.all(host(g["dw1"])[dead] == 0) and np.all(host(g["dw2"])[dead] == 0)


def test_mlp_tiny_fp32_workload(smoe):
    """T=256, d_model=128, d_ff=256, E=8, k=2, GELU, fp32: everything in full."""
    say("mlp tiny fp32 workload")
    check_full(smoe, make_config(1))


def test_mlp_single_token_and_k1(smoe):
    say("mlp T=1 k=1 and T=3 k=4")
    check_full(smoe, make_mlp(1, 64, 64, 4, 1, "gelu", "bf16", 132, w_std=0.1))
    check_full(smoe, make_mlp(3, 64, 128, 4, 4, "swiglu", "f32", 133, w_std=0.1))


def test_mlp_deterministic(smoe):
    say("mlp determinism bf16")
    w = make_mlp(700, 128, 192, 8, 2, "swiglu", "bf16", 134, w_std=0.05)
    o1, _, g1 = run_mlp(smoe, w)
    o2, _, g2 = run_mlp(smoe, w)
    assert torch.equal(o1, o2)
    for n in ("dx", "dw1", "dw2", "dw3", "dgates"):
        assert torch.equal(g1[n], g2[n]), n


def test_mlp_backward_with_second_stream(smoe):
    """A shape whose dX product has whole rounds of tiles and a partial last
    round (T=4096, d_model=2048, d_ff=512, E=8, k=2, SwiGLU, bf16): dW1 then
    runs on the caller's second stream beside that last round.  Two calls
    in a row give identical results (the fork/join events are reused), and
    dx / dgates of sampled tokens and dW1 / dW3 / dW2 slices over every token
    match the oracle."""
    say("mlp backward with the second stream")
    w = make_mlp(4096, 2048, 512, 8, 2, "swiglu", "bf16", 135, w_std=0.02)
    o1, _, g1 = run_mlp(smoe, w)
    o2, _, g2 = run_mlp(smoe, w)
    assert torch.equal(o1, o2)
    for n in ("dx", "dw1", "dw2", "dw3", "dgates"):
        assert torch.equal(g1[n], g2[n]), n
    f = lambda n: w.f32(n).astype(np.float64)
    x, w1, w2, w3, dout = f("x"), f("w1"), f("w2"), f("w3"), f("dout")
    idx, gates = w.tensors["expert_idxs"], w.tensors["gates"].astype(np.float64)
    rng = np.random.default_rng(1351)
    toks = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, 24, replace=False)]))
    ref = oracle.mlp_bwd(x, w1, w2, idx, gates, "swiglu", dout, w3=w3, storage="bf16", tokens=toks)
    for n in ("dx", "dgates"):
        e = rel_err(host(g1[n])[toks], ref[n][toks])
        say(f"  {n}[tokens] err {e:.2e}")
        assert e <= BF16_TOL, n
    cols = np.unique(np.concatenate([[0, 511], rng.choice(512, 10, replace=False)]))
    rc = oracle.mlp_dw_cols(x, w1, w2, idx, gates, "swiglu", dout, cols, w3=w3, storage="bf16")
    for n, got in (("dw1", host(g1["dw1"])[:, :, cols]), ("dw3", host(g1["dw3"])[:, :, cols]),
                   ("dw2", host(g1["dw2"])[:, cols, :])):
        e = rel_err(got, rc[n])
        say(f"  {n}[cols] err {e:.2e}")
        assert e <= BF16_TOL, n


@pytest.mark.parametrize("dtype,act,T,k,E,routing", [
    ("f32", "gelu", 300, 2, 6, "softmax"),
    ("bf16", "swiglu", 300, 2, 6, "softmax"),
    ("bf16", "gelu", 1200, 3, 12, "zipf"),
    ("bf16", "swiglu", 517, 8, 16, "softmax"),
])
def test_mlp_fused_combine(smoe, dtype, act, T, k, E, routing):
    """smoe_mlp_fwd_fused_combine: out against the oracle to the same bar as
    smoe_mlp_fwd and close to it; the saved buffer is bit-identical, so the
    backward is unchanged; for k = 2 two runs agree bit for bit."""
    say(f"mlp fused combine {dtype} {act} T={T} k={k} E={E} {routing}")
    w = make_mlp(T, 136 if dtype == "f32" else 128, 200 if dtype == "f32" else 256, E, k, act, dtype,
                 140 + k, routing=routing, w_std=0.06)
    d = upload(w)
    args = (d["x"], d["w1"], d["w2"], d["expert_idxs"], d["gates"], act)
    o_ref, s_ref = smoe.smoe_mlp_fwd(*args, w3=d.get("w3"))
    o1, s1 = smoe.smoe_mlp_fwd(*args, w3=d.get("w3"), fused_combine=True)
    o2, _ = smoe.smoe_mlp_fwd(*args, w3=d.get("w3"), fused_combine=True)
    torch.cuda.synchronize()
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    d_model, d_ff = w.dims["d_model"], w.dims["d_ff"]
    v1 = smoe.saved_views(s1, T, k, E, d_model, d_ff, act, dt)
    v_ref = smoe.saved_views(s_ref, T, k, E, d_model, d_ff, act, dt)
    for n in v_ref:
        assert torch.equal(v1[n], v_ref[n]), n
    if k <= 2:
        assert torch.equal(o1, o2)
    tol = F32_TOL if dtype == "f32" else BF16_TOL
    f = lambda n: w.f32(n).astype(np.float64)
    w3 = f("w3") if act == "swiglu" else None
    idx, gates = w.tensors["expert_idxs"], w.tensors["gates"].astype(np.float64)
    ref = oracle.mlp_fwd(f("x"), f("w1"), f("w2"), idx, gates, act, w3=w3,
                         storage="f64" if dtype == "f32" else "bf16")
    e = rel_err(host(o1), ref)
    e_same = rel_err(host(o1), host(o_ref).astype(np.float64))
    say(f"  out err {e:.2e}  vs unfused {e_same:.2e}")
    assert e <= tol
    assert e_same <= tol


def test_mlp_fused_combine_with_second_stream(smoe):
    """A shape whose forward runs its routing-dependent m-tiles on the second
    stream (T=4096, d_model=2048, d_ff=512, E=8, k=2, SwiGLU, bf16): both
    streams' W2 tiles add into the one token buffer; sampled tokens against
    the oracle, all tokens against smoe_mlp_fwd."""
    say("mlp fused combine with the second stream")
    w = make_mlp(4096, 2048, 512, 8, 2, "swiglu", "bf16", 145, w_std=0.02)
    d = upload(w)
    args = (d["x"], d["w1"], d["w2"], d["expert_idxs"], d["gates"], "swiglu")
    o_ref, _ = smoe.smoe_mlp_fwd(*args, w3=d["w3"])
    o1, _ = smoe.smoe_mlp_fwd(*args, w3=d["w3"], fused_combine=True)
    torch.cuda.synchronize()
    e_same = rel_err(host(o1), host(o_ref).astype(np.float64))
    say(f"  vs unfused {e_same:.2e}")
    assert e_same <= BF16_TOL
    f = lambda n: w.f32(n).astype(np.float64)
    idx, gates = w.tensors["expert_idxs"], w.tensors["gates"].astype(np.float64)
    toks = np.unique(np.concatenate([[0, w.T - 1], np.random.default_rng(1451).choice(w.T, 24, replace=False)]))
    ref = oracle.mlp_fwd(f("x"), f("w1"), f("w2"), idx, gates, "swiglu", w3=f("w3"), storage="bf16",
                         tokens=toks)
    e = rel_err(host(o1)[toks], ref[toks])
    say(f"  out[tokens] err {e:.2e}")
    assert e <= BF16_TOL


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_mlp_caller_stream_only_matches_second_stream(smoe, act):
    """The same call with and without the caller's second stream (aux): the
    tiles and their arithmetic are the same, only the streams differ, so
    every output is identical bit for bit (a shape whose forward and dx
    products both split their tiles across the two streams)."""
    say(f"mlp with and without the second stream, {act}")
    w = make_mlp(4096, 2048, 512, 8, 2, act, "bf16", 136, w_std=0.02)
    d = upload(w)
    res = []
    for aux in (True, False):
        out, saved = smoe.smoe_mlp_fwd(d["x"], d["w1"], d["w2"], d["expert_idxs"], d["gates"], act, w3=d.get("w3"),
                                       aux=aux)
        g = smoe.smoe_mlp_bwd(d["dout"], d["x"], d["w1"], d["w2"], d["expert_idxs"], d["gates"], act, saved,
                              w3=d.get("w3"), aux=aux)
        torch.cuda.synchronize()
        res.append((out, g))
    assert torch.equal(res[0][0], res[1][0])
    for n in ("dx", "dw1", "dw2", "dgates") + (("dw3",) if act == "swiglu" else ()):
        assert torch.equal(res[0][1][n], res[1][1][n]), n


def test_mlp_bf16_weight_gradients_are_the_rounded_fp32_ones(smoe):
    """dw_dtype = bf16: every weight gradient is summed in fp32 exactly as
    for an fp32 result and rounded once (nearest even), so it equals the
    fp32 result rounded, bit for bit; experts with no tokens get 0."""
    say("mlp bf16 weight gradients")
    w = make_mlp(1500, 128, 256, 10, 2, "swiglu", "bf16", 137, routing="zipf", w_std=0.05, n_dead=2)
    d = upload(w)
    out, saved = smoe.smoe_mlp_fwd(d["x"], d["w1"], d["w2"], d["expert_idxs"], d["gates"], "swiglu", w3=d["w3"])
    g32 = smoe.smoe_mlp_bwd(d["dout"], d["x"], d["w1"], d["w2"], d["expert_idxs"], d["gates"], "swiglu", saved,
                            w3=d["w3"])
    g16 = smoe.smoe_mlp_bwd(d["dout"], d["x"], d["w1"], d["w2"], d["expert_idxs"], d["gates"], "swiglu", saved,
                            w3=d["w3"], dw_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for n in ("dw1", "dw2", "dw3"):
        assert g16[n].dtype == torch.bfloat16
        assert torch.equal(g16[n], g32[n].to(torch.bfloat16)), n
    assert torch.equal(g16["dx"], g32["dx"]) and torch.equal(g16["dgates"], g32["dgates"])
