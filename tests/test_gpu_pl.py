"""smoe_parallel_linear_fwd / _bwd on the GPU against the oracle: all four
grouped/scattered layouts, both fan-outs of a scattered input, the
gate-weighted combine, fp32 and bf16, ragged tiles and empty experts; the
single-ParallelLinear workload (T=8192, 2048->2048, E=16, k=2) on sampled
rows."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import BF16_TOL, F32_TOL, dev_tensor, host, rel_err, say
from workloads import make_pl

pytestmark = pytest.mark.gpu

VARIANTS = [  # (x_grouped, y_grouped, x rows, gates)
    (False, True, "T", False),   # scatter -> group
    (False, False, "T", False),  # scatter -> scatter
    (True, True, "M", False),    # group -> group
    (True, False, "M", False),   # group -> scatter
    (False, False, "M", False),  # scatter (one row per assignment) -> scatter
    (False, False, "T", True),   # scatter -> scatter, combined with gates
    (True, False, "M", True),    # group -> scatter, combined with gates
]


def _setup(smoe, w, xg, x_rows):
    t = w.tensors
    x_np = t["x_grouped"] if (xg or x_rows == "M") else t["x"]
    idx = torch.from_numpy(t["expert_idxs"]).cuda()
    rt = smoe.smoe_route(idx, w.E)
    return x_np, rt


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("xg,yg,x_rows,use_gates", VARIANTS)
def test_forward_backward_small(smoe, dtype, xg, yg, x_rows, use_gates):
    w = make_pl(1000, 200, 136, 7, 2, dtype, 120, x_std=1.0, w_std=0.1, with_gates=use_gates)
    # leave experts 5 and 6 without rows
    idx = w.tensors["expert_idxs"]
    idx[idx >= 5] = (idx[idx >= 5] * 7) % 5
    idx[:, 1] = np.where(idx[:, 0] == idx[:, 1], (idx[:, 0] + 1) % 5, idx[:, 1])
    say(f"pl small {dtype} xg={xg} yg={yg} x_rows={x_rows} gates={use_gates}")
    x_np, rt = _setup(smoe, w, xg, x_rows)
    T, k = w.T, w.k
    xd = dev_tensor(x_np)
    wd = dev_tensor(w.tensors["w"])
    gd = dev_tensor(w.tensors["gates"]) if use_gates else None
    y = smoe.smoe_parallel_linear_fwd(xd, wd, T, k, rt["sorted_scattered_idxs"], rt["offsets"], xg, yg, gd)
    dy_np = w.tensors["dy_comb"] if use_gates else w.tensors["dy"]
    dx, dw, dg = smoe.smoe_parallel_linear_bwd(xd, wd, T, k, rt["sorted_scattered_idxs"], rt["offsets"], xg, yg,
                                                dev_tensor(dy_np), gd, need_dgates=use_gates)
    torch.cuda.synchronize()
    f = lambda n: w.f32(n).astype(np.float64)
    xs = f("x_grouped") if (xg or x_rows == "M") else f("x")
    gates = w.tensors["gates"].astype(np.float64) if use_gates else None
    ref = oracle.parallel_linear_fwd(xs, f("w"), idx, xg, yg, gates=gates)
    tol = F32_TOL if dtype == "f32" else BF16_TOL
    e = rel_err(host(y), ref)
    say(f"  y err {e:.2e}")
    assert e <= tol
    storage = "bf16" if dtype == "bf16" else "f64"
    rdx, rdw, rdg = oracle.parallel_linear_bwd(xs, f("w"), idx, xg, yg, f("dy_comb") if use_gates else f("dy"),
                                               gates=gates, storage=storage)
    for name, got, want in (("dx", dx, rdx), ("dw", dw, rdw)) + ((("dg", dg, rdg),) if use_gates else ()):
        e = rel_err(host(got), want)
        say(f"  {name} err {e:.2e}")
        assert e <= tol, name
    assert np.all(host(dw)[5:] == 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_experts_split_weight_gradient(smoe, dtype):
    """More than 64 experts (100, five of them empty) with about 490 rows
    each: the grouped products' tile lookup takes its path for more than 64
    experts, and the weight gradient splits every expert into row chunks
    whose partials are summed by the reduction, which counts the chunks
    before an expert 64 experts at a time."""
    w = make_pl(24576, 128, 128, 100, 2, dtype, 121, x_std=1.0, w_std=0.1)
    idx = w.tensors["expert_idxs"]
    idx[idx >= 95] = (idx[idx >= 95] * 13) % 95
    idx[:, 1] = np.where(idx[:, 0] == idx[:, 1], (idx[:, 0] + 1) % 95, idx[:, 1])
    say(f"pl many experts {dtype}: E=100, counts {np.bincount(idx.ravel(), minlength=100)[[0, 63, 64, 99]]}")
    x_np, rt = _setup(smoe, w, False, "T")
    T, k = w.T, w.k
    xd = dev_tensor(x_np)
    wd = dev_tensor(w.tensors["w"])
    y = smoe.smoe_parallel_linear_fwd(xd, wd, T, k, rt["sorted_scattered_idxs"], rt["offsets"], False, True, None)
    dx, dw, _ = smoe.smoe_parallel_linear_bwd(xd, wd, T, k, rt["sorted_scattered_idxs"], rt["offsets"], False, True,
                                              dev_tensor(w.tensors["dy"]), None, need_dgates=False)
    torch.cuda.synchronize()
    f = lambda n: w.f32(n).astype(np.float64)
    ref = oracle.parallel_linear_fwd(f("x"), f("w"), idx, False, True)
    tol = F32_TOL if dtype == "f32" else BF16_TOL
    storage = "bf16" if dtype == "bf16" else "f64"
    rdx, rdw, _ = oracle.parallel_linear_bwd(f("x"), f("w"), idx, False, True, f("dy"), storage=storage)
    for name, got, want in (("y", y, ref), ("dx", dx, rdx), ("dw", dw, rdw)):
        e = rel_err(host(got), want)
        say(f"  {name} err {e:.2e}")
        assert e <= tol, name
    assert np.all(host(dw)[95:] == 0.0)


def _sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, n, replace=False)]))


@pytest.mark.parametrize("xg,yg", [(False, True), (False, False), (True, True), (True, False)])
def test_single_parallel_linear_workload(smoe, xg, yg):
    """T=8192, d_in=d_out=2048, E=16, k=2, bf16; rows of 48 sampled tokens."""
    w = make_pl(8192, 2048, 2048, 16, 2, "bf16", 2)
    say(f"pl C2 xg={xg} yg={yg}")
    x_np, rt = _setup(smoe, w, xg, "M" if xg else "T")
    xd, wd = dev_tensor(x_np), dev_tensor(w.tensors["w"])
    y = smoe.smoe_parallel_linear_fwd(xd, wd, w.T, w.k, rt["sorted_scattered_idxs"], rt["offsets"], xg, yg)
    torch.cuda.synchronize()
    y = host(y)
    toks = _sample_tokens(w.T, 46, 7)
    idx = w.tensors["expert_idxs"]
    ref = oracle.parallel_linear_fwd(w.f32("x_grouped" if xg else "x"), w.f32("w"), idx, xg, yg, tokens=toks)
    s = rt["sorted_scattered_idxs"].cpu().numpy()
    rinv = np.empty_like(s)
    rinv[s] = np.arange(s.size)
    rows = [(rinv[p] if yg else p) for t in toks for p in range(t * w.k, (t + 1) * w.k)]
    e = rel_err(y[rows], ref[rows])
    say(f"  y err {e:.2e}")
    assert e <= BF16_TOL
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("xg,x_rows,use_gates", [(False, "T", False), (True, "M", True), (False, "T", True)])
def test_backward_output_types_and_accumulation(smoe, xg, x_rows, use_gates):
    """dx_dtype = fp32 keeps the exact sum unrounded (the bf16 dx is exactly
    its rounding); dw_dtype = bf16 is the fp32 dw rounded once; with
    accumulate_dw the gradient is added to the given dw (fp32 and bf16)."""
    w = make_pl(900, 136, 200, 6, 3, "bf16", 121, x_std=1.0, w_std=0.1, with_gates=use_gates)
    say(f"pl backward output types xg={xg} x_rows={x_rows} gates={use_gates}")
    x_np, rt = _setup(smoe, w, xg, x_rows)
    T, k = w.T, w.k
    xd, wd = dev_tensor(x_np), dev_tensor(w.tensors["w"])
    gd = dev_tensor(w.tensors["gates"]) if use_gates else None
    dyd = dev_tensor(w.tensors["dy_comb"] if use_gates else w.tensors["dy"])
    s, off = rt["sorted_scattered_idxs"], rt["offsets"]
    dx16, dw32, _ = smoe.smoe_parallel_linear_bwd(xd, wd, T, k, s, off, xg, False, dyd, gd)
    dx32, dw16, _ = smoe.smoe_parallel_linear_bwd(xd, wd, T, k, s, off, xg, False, dyd, gd,
                                                  dx_dtype=torch.float32, dw_dtype=torch.bfloat16)
    init32 = torch.randn(dw32.shape, device="cuda", dtype=torch.float32)
    init16 = init32.to(torch.bfloat16)
    acc32, acc16 = init32.clone(), init16.clone()
    smoe.smoe_parallel_linear_bwd(xd, wd, T, k, s, off, xg, False, dyd, gd, need_dx=False, dw=acc32,
                                  accumulate_dw=True)
    smoe.smoe_parallel_linear_bwd(xd, wd, T, k, s, off, xg, False, dyd, gd, need_dx=False, dw=acc16,
                                  accumulate_dw=True)
    torch.cuda.synchronize()
    assert dx32.dtype == torch.float32 and dw16.dtype == torch.bfloat16
    assert torch.equal(dx16, dx32.to(torch.bfloat16))
    assert torch.equal(dw16, dw32.to(torch.bfloat16))
    assert torch.equal(acc32, dw32 + init32)
    assert torch.equal(acc16, (dw32 + init16.float()).to(torch.bfloat16))
    # and the fp32 dx against the oracle
    f = lambda n: w.f32(n).astype(np.float64)
    xs = f("x_grouped") if (xg or x_rows == "M") else f("x")
    gates = w.tensors["gates"].astype(np.float64) if use_gates else None
    rdx, _, _ = oracle.parallel_linear_bwd(xs, f("w"), w.tensors["expert_idxs"], xg, False,
                                           f("dy_comb") if use_gates else f("dy"), gates=gates, storage="bf16")
    e = rel_err(host(dx32), rdx)
    say(f"  dx (fp32) max err / RMS {e:.2e}")
    assert e <= BF16_TOL
