#!/usr/bin/env python3
"""SMoE-MLP training-step benchmark on one MI355X.

One step = smoe_mlp_fwd + smoe_mlp_bwd (routing, the fused W1/W3 product
with SwiGLU, the W2 product with scattered output, the gate-weighted
combine, and the whole backward: dA with the activation backward and gate
gradient, dW2, dX with its k-sum, dW1, dW3) on the Mixtral-shaped
workload: T=16384 tokens (4 x 4096), d_model=4096, d_ff=14336, E=8, k=2,
bf16, softmax-top-2 routing over N(0,1) logits, weights N(0, 0.02^2),
synthetic seeded inputs resident in HBM before timing starts.

Prints one JSON line: tokens/s (whole job), ms/step, TFLOP/s and MFMA
utilisation over the expert products, the roofline of the dominant kernel
(HIP events on the library's stream), and the CPU oracle timed on a
bounded token sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--cpu-tokens 24]

HBM traffic of the dominant kernel comes from two rocprofv3 counter runs
(FETCH_SIZE, then WRITE_SIZE) of this script with --copy-mib, which also
times a plain elementwise copy of known size whose counter readings give the
KiB -> byte scale:

    rocprofv3 --pmc FETCH_SIZE -d DIR_F -o run --output-format csv -- \
        python3 bench.py --steps 1 --warmup 1 --cpu-tokens 0 --copy-mib 1024
    (the same with WRITE_SIZE into DIR_W)
    python bench.py --pmc-summary DIR_F DIR_W > profiles/gemm_traffic_mixtral.txt

The summary records a hash of the GEMM kernel sources; the traffic figure is
reported only while the sources still hash to it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

GEMM_ROLES = ["up", "down", "dA", "dW2", "dX", "dW1", "dW3"]

ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["gemm.hip", "gemm_kernel.h", "gemm_store_k.hip", "gemm_store_mn.hip", "gemm_act_fwd.hip",
                  "gemm_act_bwd.hip", "gemm_dw.hip", "common.h", "kernels.h"]
# one step launches the grouped-product kernel once per role, in this order
# (route, then up, down, combine, dA, dgates, dW2, dX, k-sum, dW1, dW3)
# grouped-product launches of one step in enqueue order: the forward
# enqueues both layers' routing-dependent m-tiles on the second stream first,
# then the rest of each layer; the dX product is two launches (its whole
# rounds of tiles, then the rest, with dW1 enqueued on the second stream in
# between).  A role's bytes are summed over its launches.
GEMM_ORDER = ["up", "down", "up", "down", "dA", "dX", "dW1", "dX", "dW2", "dW3"]
GEMM_KERNEL_HINT = "smoe::gemm_bf16_kernel<"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic_mixtral.txt")
COPY_KERNEL_HINT = "neg"


def kernel_sources_hash():
    h = hashlib.sha256()
    for n in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "sparse_mixture_experts_top_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _read_dispatches(d):
    """[(dispatch id, kernel name, counter value)] in dispatch order from a
    rocprofv3 csv directory (values of one dispatch summed over instances)."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    assert files, f"no counter_collection.csv under {d}"
    out = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                key = int(r["Dispatch_Id"])
                name, v = out.get(key, (r["Kernel_Name"], 0.0))
                out[key] = (name, v + float(r["Counter_Value"]))
    return [(k, n, v) for k, (n, v) in sorted(out.items())]


def pmc_summary(dir_fetch, dir_write, copy_bytes):
    """Text summary: per-launch HBM bytes of each grouped-product role, from
    the two counter runs, scaled by the counters' reading for the copy
    kernel of known size.  Roles are assigned by launch order within a step."""
    lines = []
    res = {}
    for ctr, d in (("FETCH_SIZE", dir_fetch), ("WRITE_SIZE", dir_write)):
        disp = _read_dispatches(d)
        copy = [v for _, n, v in disp if COPY_KERNEL_HINT in n and "smoe" not in n]
        gemm = [v for _, n, v in disp if GEMM_KERNEL_HINT in n]
        assert copy and gemm and len(gemm) % len(GEMM_ORDER) == 0, (ctr, len(copy), len(gemm))
        copy_kib = float(np.median(copy))
        scale = copy_bytes / (copy_kib * 1024.0)
        lines.append(f"{ctr}: copy kernel {copy_kib:.0f} KiB/dispatch for {copy_bytes} bytes -> "
                     f"scale {scale:.4f}; {len(gemm) // len(GEMM_ORDER)} steps")
        per_role = {}
        for i, role in enumerate(GEMM_ORDER):
            per_role[role] = per_role.get(role, 0.0) + float(np.mean(gemm[i::len(GEMM_ORDER)]))
        for role, kib in per_role.items():
            res.setdefault(role, {})[ctr] = kib * 1024.0 * scale
            lines.append(f"  {role}: {kib:.0f} KiB per launch of the product")
    for role in dict.fromkeys(GEMM_ORDER):
        lines.append(f"{role}_fetch_bytes_per_launch: {res[role]['FETCH_SIZE']:.6e}")
        lines.append(f"{role}_write_bytes_per_launch: {res[role]['WRITE_SIZE']:.6e}")
    lines.append(f"kernel_sources_sha256_16: {kernel_sources_hash()}")
    return "\n".join(lines)


def _read_durations(d):
    """{dispatch id: duration ns} from the kernel trace of a rocprofv3 run."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    assert files, f"no kernel_trace.csv under {d}"
    out = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                out[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return out


def _short_kernel(name):
    """Kernel name without its argument list (template arguments kept)."""
    n = name.split("(")[0].replace("void ", "").replace("smoe::", "")
    return n if len(n) < 140 else n[:137] + "..."


def kernel_traffic_summary(dir_fetch, dir_write, copy_bytes):
    """Text summary of two rocprofv3 runs of one command (--kernel-trace
    --pmc FETCH_SIZE, then WRITE_SIZE) with --copy-mib: per kernel, its
    launches, mean duration and mean HBM bytes fetched and written per
    launch, each counter scaled by its reading for the copy kernel of known
    size in the same run."""
    per = {}
    scales = {}
    for ctr, d in (("FETCH_SIZE", dir_fetch), ("WRITE_SIZE", dir_write)):
        disp = _read_dispatches(d)
        copy = [v for _, n, v in disp if COPY_KERNEL_HINT in n and "smoe" not in n]
        assert copy, ctr
        scales[ctr] = copy_bytes / (float(np.median(copy)) * 1024.0)
        for _, n, v in disp:
            if "smoe" not in n:
                continue
            per.setdefault(_short_kernel(n), {}).setdefault(ctr, []).append(v * 1024.0 * scales[ctr])
    dur = _read_durations(dir_fetch)
    names = {}
    for k, n, _ in _read_dispatches(dir_fetch):
        if "smoe" in n:
            names.setdefault(_short_kernel(n), []).append(dur[k])
    lines = [f"counter scale: FETCH_SIZE {scales['FETCH_SIZE']:.4f}, WRITE_SIZE {scales['WRITE_SIZE']:.4f} "
             f"bytes per counted byte (copy kernel of {copy_bytes} bytes)",
             "kernel | launches | mean ms (under the profiler) | MB fetched | MB written | GB/s"]
    for n, ds in sorted(names.items(), key=lambda kv: -sum(kv[1])):
        f = float(np.mean(per[n]["FETCH_SIZE"])) if "FETCH_SIZE" in per[n] else 0.0
        w = float(np.mean(per[n].get("WRITE_SIZE", [0.0])))
        ms = float(np.mean(ds)) / 1e6
        lines.append(f"{n} | {len(ds)} | {ms:.4f} | {f / 1e6:.1f} | {w / 1e6:.1f} | {(f + w) / (ms * 1e-3) / 1e9:.0f}")
    lines.append(f"kernel_sources_sha256_16: {kernel_sources_hash()}")
    return "\n".join(lines)


def mfma_busy_summary(d):
    """Text summary of one rocprofv3 run with --kernel-trace and
    --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES: per
    grouped-product role, the clock (GRBM_GUI_ACTIVE is summed over the 8
    XCDs: cycles per XCD / duration) and the matrix cores' busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES counts busy cycles summed over the 1024 SIMDs,
    32 per 32x32x16 multiply: busy / (1024 x cycles per XCD)); the
    register-only MFMA loop of the same run is the reference."""
    rows = {}
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    assert files, f"no counter_collection.csv under {d}"
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                key = int(r["Dispatch_Id"])
                e = rows.setdefault(key, {"name": r["Kernel_Name"]})
                e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    dur = _read_durations(d)
    disp = [(k, rows[k]) for k in sorted(rows)]
    gemm = [(k, e) for k, e in disp if GEMM_KERNEL_HINT in e["name"]]
    loop = [(k, e) for k, e in disp if "mfma_loop_kernel" in e["name"]]
    assert gemm and len(gemm) % len(GEMM_ORDER) == 0, len(gemm)

    def stats(items):
        cyc = np.mean([e["GRBM_GUI_ACTIVE"] / 8.0 for _, e in items])
        busy = np.mean([e["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024.0 * e["GRBM_GUI_ACTIVE"] / 8.0) for _, e in items])
        ns = np.mean([dur[k] for k, _ in items])
        return ns / 1e6, cyc / ns, busy

    lines = [f"{len(gemm) // len(GEMM_ORDER)} steps; per launch: ms (under the profiler), clock GHz, "
             f"matrix cores busy (fraction of cycles), busy x clock / 2.4 GHz (fraction of the bf16 peak rate)"]
    for i, role in enumerate(GEMM_ORDER):
        items = gemm[i::len(GEMM_ORDER)]
        ms, ghz, busy = stats(items)
        lines.append(f"  launch {i} {role:>4}: {ms:8.3f} ms  {ghz:5.2f} GHz  busy {busy:5.3f}  "
                     f"rate {busy * ghz / 2.4:5.3f}")
    if loop:
        ms, ghz, busy = stats(loop)
        lines.append(f"  mfma loop probe: {ms:8.3f} ms  {ghz:5.2f} GHz  busy {busy:5.3f}  rate {busy * ghz / 2.4:5.3f}")
    lines.append(f"kernel_sources_sha256_16: {kernel_sources_hash()}")
    return "\n".join(lines)


def read_traffic(role):
    """HBM bytes per launch of a role's kernel from the committed counter
    summary, or None if absent or taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        m = re.match(r"^(\w+):\s*(\S+)\s*$", line.strip())
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("kernel_sources_sha256_16") != kernel_sources_hash():
        return None
    if f"{role}_fetch_bytes_per_launch" not in kv:
        return None
    return float(kv[f"{role}_fetch_bytes_per_launch"]) + float(kv[f"{role}_write_bytes_per_launch"])


def copy_calibration(mib):
    """A plain elementwise copy (y = -x, fp32) of known size, three times:
    each launch reads and writes mib MiB."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    del x, y
    log(f"copy calibration: 3 launches of {mib} MiB read + {mib} MiB written")


def gemm_flops(T, k, d, f, act):
    """Algorithmic FLOPs of each expert product of one fwd+bwd step."""
    M = T * k
    one = 2.0 * M * d * f
    up = 2 * one if act == "swiglu" else one
    fl = {"up": up, "down": one, "dA": one, "dW2": one,
          "dX": up, "dW1": one}
    if act == "swiglu":
        fl["dW3"] = one
    return fl


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-tokens", type=int, default=24,
                    help="tokens of the oracle's CPU-baseline sample (0 skips it)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain copy of this many MiB (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the traffic summary of two rocprofv3 --pmc runs and exit")
    ap.add_argument("--kernel-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print the per-kernel traffic summary of two rocprofv3 --kernel-trace --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) of any workload run with --copy-mib, and exit")
    ap.add_argument("--busy-summary", metavar="DIR",
                    help="print the clock / matrix-core busy summary of one rocprofv3 run with "
                         "--kernel-trace --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES and exit")
    ap.add_argument("--workload", default="mixtral", choices=["mixtral", "granular", "moa", "pl", "router", "attention", "sparsity",
                                                            "combine"],
                    help="mixtral (the measured line); the others print supplementary lines: "
                         "granular = high-granularity Zipf SMoE-MLP, moa = Mixture-of-Attention "
                         "projections, pl = single ParallelLinear in its four layouts, router = the "
                         "top-k softmax router forward and backward at the three workloads' shapes, "
                         "attention = the Mixture-of-Attention core at the MoA workload's shape, "
                         "sparsity = SMoE-MLP at fixed E with k swept, each beside a dense MLP of the same "
                         "active FLOPs, and the memory footprint of the Mixtral-shaped step; combine = "
                         "the SMoE-MLP forward with the separate combine and with the combine fused into "
                         "the W2 product, at the Mixtral and high-granularity shapes")
    return ap.parse_args()


def cpu_baseline(w, n_tokens):
    """Time the fp64 CPU oracle (fwd + bwd) on a seeded sample of tokens."""
    import oracle
    from threadpoolctl import threadpool_info
    rng = np.random.default_rng(12345)
    toks = np.sort(rng.choice(w.T, n_tokens, replace=False))
    f = lambda n: w.f32(n).astype(np.float64)
    x, w1, w2, w3, dout = f("x"), f("w1"), f("w2"), f("w3") if w.act == "swiglu" else None, f("dout")
    idx, gates = w.tensors["expert_idxs"], w.tensors["gates"].astype(np.float64)
    t0 = time.perf_counter()
    oracle.mlp_fwd(x, w1, w2, idx, gates, w.act, w3=w3, storage="bf16", tokens=toks)
    oracle.mlp_bwd(x, w1, w2, idx, gates, w.act, dout, w3=w3, storage="bf16", tokens=toks)
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    affinity = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": int(min(threads, affinity)), "kind": "oracle",
            "cpu_model": model, "affinity_cores": affinity, "blas_threads": int(threads),
            "sample": f"{n_tokens} seeded tokens of the same workload, fwd+bwd per token and "
                      f"choice in fp64 ({dt:.1f} s); per-token cost is constant so tokens/s "
                      f"extrapolates to the full batch"}


def main():
    args = parse()
    if args.pmc_summary:
        print(pmc_summary(*args.pmc_summary, copy_bytes=(args.copy_mib or 1024) << 20))
        return
    if args.kernel_traffic:
        print(kernel_traffic_summary(*args.kernel_traffic, copy_bytes=(args.copy_mib or 1024) << 20))
        return
    if args.busy_summary:
        print(mfma_busy_summary(args.busy_summary))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build runs the hot path "
              "on a single MI355X and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_mixture_experts_top_amd as smoe
    from workloads import make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_mib:
        copy_calibration(args.copy_mib)
    if args.workload != "mixtral":
        print(json.dumps(supplementary(args)), flush=True)
        return
    log("generating the Mixtral-shaped workload")
    w = make_config(3)
    T, k, E = w.T, w.k, w.E
    d, f, act = w.dims["d_model"], w.dims["d_ff"], w.act

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    t = {n: dev(w.tensors[n]) for n in ("x", "w1", "w2", "w3", "expert_idxs", "gates", "dout")}
    ws_f = torch.empty(smoe.lib.smoe_mlp_fwd_workspace_bytes(T, k, E, d, f, smoe.ACT_SWIGLU, smoe.BF16),
                       dtype=torch.uint8, device="cuda")
    ws_b = torch.empty(smoe.lib.smoe_mlp_bwd_workspace_bytes(T, k, E, d, f, smoe.ACT_SWIGLU, smoe.BF16),
                       dtype=torch.uint8, device="cuda")

    def step():
        out, saved = smoe.smoe_mlp_fwd(t["x"], t["w1"], t["w2"], t["expert_idxs"], t["gates"], act,
                                       w3=t["w3"], ws=ws_f)
        g = smoe.smoe_mlp_bwd(t["dout"], t["x"], t["w1"], t["w2"], t["expert_idxs"], t["gates"], act, saved,
                              w3=t["w3"], ws=ws_b)
        return out, g

    log(f"inputs resident; {args.warmup} warmup steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")

    # per-kernel events for every step of the timed region
    roles = GEMM_ROLES + ["route", "combine", "ksum", "dg_reduce", "dw_reduce"]
    evs = [{r: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for r in roles}
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for r in roles:
            smoe.smoe_set_role_events(r, *evs[i][r])
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for r in roles:
        smoe.smoe_set_role_events(r, None, None)

    ms = (t1 - t0) * 1e3 / args.steps
    kern_ms = {r: float(np.mean([evs[i][r][0].elapsed_time(evs[i][r][1]) for i in range(args.steps)]))
               for r in roles}
    fl = gemm_flops(T, k, d, f, act)
    total_flops = sum(fl.values())
    tflops = total_flops / (ms * 1e-3) / 1e12
    dom = max(fl, key=lambda r: kern_ms[r])
    achieved = fl[dom] / (kern_ms[dom] * 1e-3) / 1e12

    res = {
        "metric": "SMoE-MLP tokens/s fwd+bwd bf16 and MFMA util % of peak, 1 MI355X",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Mixtral-shaped SMoE-MLP fwd+bwd: T=16384 (4x4096), d_model=4096, "
                               "d_ff=14336, E=8, k=2, SwiGLU, bf16",
                   "T": T, "d_model": d, "d_ff": f, "E": E, "k": k, "act": act},
        "tflops": tflops,
        "mfma_util_pct": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "expert_gemm_tflop_per_step": total_flops / 1e12,
        "kernels_ms": kern_ms,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": read_traffic(dom),
                     "flop_per_launch": fl[dom], "avg_launch_ms": kern_ms[dom]},
    }
    # the matrix cores' reachable rate on this device (register-only MFMA
    # loop, outside the timed region), the second reference for utilisation
    loop = mfma_loop_peak()
    res["mfma_loop_peak"] = {"tflops": loop, "util_pct_of_loop": 100.0 * tflops / loop,
                             "probe": "bf16 32x32x16 MFMA loop on registers: 2048 workgroups x 4 waves x "
                                      f"{MFMA_LOOP_ITERS} rounds of 16 multiplies, best of 3"}
    del t, ws_f, ws_b
    torch.cuda.empty_cache()
    if args.cpu_tokens > 0:
        log(f"CPU oracle on {args.cpu_tokens} tokens")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_tokens)
    print(json.dumps(res), flush=True)


MFMA_LOOP_ITERS = 4000


def mfma_loop_peak():
    """TFLOP/s of smoe_probe_mfma_loop (best of three launches)."""
    import torch
    import sparse_mixture_experts_top_amd as smoe
    blocks = 2048
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    smoe.smoe_probe_mfma_loop(out, blocks, 100)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        smoe.smoe_probe_mfma_loop(out, blocks, MFMA_LOOP_ITERS)
        b.record()
        torch.cuda.synchronize()
        fl = blocks * 4.0 * MFMA_LOOP_ITERS * 16 * 32768
        best = max(best, fl / (a.elapsed_time(b) * 1e-3) / 1e12)
    return best


def _dev(a):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _time_steps(step, steps, warmup):
    """Mean wall time per step (ms) between device synchronisations."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def supplementary(args):
    """One JSON line for a workload other than the measured Mixtral-shaped
    one: step time, tokens/s, expert-product TFLOP/s and per-launch times."""
    import torch
    import sparse_mixture_experts_top_amd as smoe
    from workloads import make_config
    steps, warmup = args.steps, args.warmup
    if args.workload == "router":
        return router_lines(args)
    if args.workload == "attention":
        return attention_line(args)
    if args.workload == "sparsity":
        return sparsity_line(args)
    if args.workload == "combine":
        return combine_line(args)
    if args.workload == "granular":
        w = make_config(4)
        T, k, E = w.T, w.k, w.E
        d, f, act = w.dims["d_model"], w.dims["d_ff"], w.act
        t = {n: _dev(w.tensors[n]) for n in ("x", "w1", "w2", "expert_idxs", "gates", "dout")}

        def step():
            out, saved = smoe.smoe_mlp_fwd(t["x"], t["w1"], t["w2"], t["expert_idxs"], t["gates"], act)
            smoe.smoe_mlp_bwd(t["dout"], t["x"], t["w1"], t["w2"], t["expert_idxs"], t["gates"], act, saved)

        roles = [r for r in GEMM_ROLES if r != "dW3"]
        fl = sum(gemm_flops(T, k, d, f, act).values())
        name = ("high-granularity SMoE-MLP fwd+bwd: T=16384, d_model=1024, d_ff=512, E=64, k=8, "
                "Zipf(1.1) routing with 8 empty experts, GELU, bf16")
    elif args.workload == "moa":
        w = make_config(5)
        T, k, E = w.T, w.k, w.E
        d, hd = w.dims["d_model"], w.dims["head_dim"]
        t = {n: _dev(w.tensors[n]) for n in ("x", "wq", "wo", "o_in", "dq", "dout", "gates", "expert_idxs")}

        def step():
            rt = smoe.smoe_route(t["expert_idxs"], E)
            s, off = rt["sorted_scattered_idxs"], rt["offsets"]
            smoe.smoe_parallel_linear_fwd(t["x"], t["wq"], T, k, s, off, False, True)
            smoe.smoe_parallel_linear_fwd(t["o_in"], t["wo"], T, k, s, off, True, False, t["gates"])
            smoe.smoe_parallel_linear_bwd(t["x"], t["wq"], T, k, s, off, False, True, t["dq"])
            smoe.smoe_parallel_linear_bwd(t["o_in"], t["wo"], T, k, s, off, True, False, t["dout"], t["gates"],
                                          need_dgates=True)

        roles = ["pl_fwd", "pl_dx", "pl_dw"]
        fl = 6 * 2.0 * T * k * d * hd
        name = ("Mixture-of-Attention projections fwd+bwd: T=8192, d_model=2048, E=16 heads of 128, k=4, "
                "Q scattered->grouped, O grouped->scattered with the combine, bf16")
    else:
        w = make_config(2)
        T, k, E = w.T, w.k, w.E
        d_in, d_out = w.dims["d_in"], w.dims["d_out"]
        x, xg, wt = _dev(w.tensors["x"]), _dev(w.tensors["x_grouped"]), _dev(w.tensors["w"])
        rt = smoe.smoe_route(_dev(w.tensors["expert_idxs"]), E)
        s, off = rt["sorted_scattered_idxs"], rt["offsets"]
        fl = 2.0 * T * k * d_in * d_out
        variants = {}
        for xgrp, ygrp, label in ((False, True, "scatter->group"), (False, False, "scatter->scatter"),
                                  (True, True, "group->group"), (True, False, "group->scatter")):
            step = lambda: smoe.smoe_parallel_linear_fwd(xg if xgrp else x, wt, T, k, s, off, xgrp, ygrp)
            ms = _time_steps(step, steps, warmup)
            variants[label] = {"ms": ms, "tflops": fl / (ms * 1e-3) / 1e12}
        best = min(v["ms"] for v in variants.values())
        return {"metric": "ParallelLinear forward TFLOP/s per layout (supplementary), 1 MI355X",
                "value": fl / (best * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
                "warmup": warmup, "dtype": "bf16", "data": "synthetic",
                "config": {"workload": "single ParallelLinear forward: T=8192, 2048->2048, E=16, k=2, "
                                       "distinct uniform expert pairs, bf16"},
                "variants": variants, "mfma_util_pct_best": 100.0 * fl / (best * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    ms = _time_steps(step, steps, warmup)
    evs = {r: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for r in roles}
    for r in roles:
        smoe.smoe_set_role_events(r, *evs[r])
    step()
    torch.cuda.synchronize()
    for r in roles:
        smoe.smoe_set_role_events(r, None, None)
    tflops = fl / (ms * 1e-3) / 1e12
    return {"metric": "tokens/s fwd+bwd (supplementary), 1 MI355X", "value": T / (ms * 1e-3),
            "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": ms,
            "dtype": "bf16", "data": "synthetic", "config": {"workload": name},
            "tflops": tflops, "mfma_util_pct": 100.0 * tflops / PEAK_BF16_TFLOPS,
            "expert_gemm_tflop_per_step": fl / 1e12,
            "kernels_ms_last_launch": {r: evs[r][0].elapsed_time(evs[r][1]) for r in roles}}


def _event_ms(fn, steps, warmup):
    """Mean device time per call (ms), events on the stream the calls use."""
    import torch
    for _ in range(warmup):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def router_lines(args):
    """Router forward (logits, top-k, softmax) and backward (dx written, dG)
    at the token counts and widths of the three bf16 workloads: time per
    call and GB/s of algorithmic bytes (x, G, routing arrays and outputs;
    the backward's per-chunk partials are scratch and not counted)."""
    import sparse_mixture_experts_top_amd as smoe
    from workloads import make_router
    steps, warmup = max(args.steps, 20), max(args.warmup, 3)
    shapes = {"mixtral": (16384, 4096, 8, 2), "granular": (16384, 1024, 64, 8), "moa": (8192, 2048, 16, 4)}
    out = {}
    for name, (T, d, E, k) in shapes.items():
        w = make_router(T, d, E, k, "bf16", 900 + E)
        x, dgs = _dev(w.tensors["x"]), _dev(w.tensors["dgates"])
        g = _dev(np.ascontiguousarray(w.tensors["gate_w"].T))   # gate weight [E, d]
        r = smoe.smoe_router_fwd(x, g, k)
        fwd_ms = _event_ms(lambda: smoe.smoe_router_fwd(x, g, k), steps, warmup)
        bwd_ms = _event_ms(lambda: smoe.smoe_router_bwd(x, g, r["expert_idxs"], r["gates"], dgs), steps, warmup)
        fwd_b = 2 * T * d + 2 * d * E + 8 * T * k
        bwd_b = 4 * T * d + 2 * d * E + 12 * T * k + 4 * d * E
        out[name] = {"T": T, "d_model": d, "E": E, "k": k, "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
                     "bytes": fwd_b + bwd_b,
                     "fwd_GBps": fwd_b / (fwd_ms * 1e-3) / 1e9, "bwd_GBps": bwd_b / (bwd_ms * 1e-3) / 1e9}
    m = out["mixtral"]
    return {"metric": "router fwd+bwd GB/s (supplementary), 1 MI355X",
            "value": m["bytes"] / ((m["fwd_ms"] + m["bwd_ms"]) * 1e-3) / 1e9, "unit": "GB/s",
            "n_gpus": 1, "steps": steps, "warmup": warmup, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "top-k softmax router, bf16: logits x w^T, top-k, softmax; backward dx, dw; "
                                   "value at T=16384, d_model=4096, E=8, k=2"},
            "peak_GBps": 8000.0, "shapes": out}


def sparsity_line(args):
    """SMoE-MLP fwd+bwd at fixed E = 16 (T=16384, d_model=1024, d_ff=1024 per
    expert, GELU, bf16) with k = 1, 2, 4, 8, 16, each timed beside a dense
    MLP of the same active FLOPs (this library's own path with E = 1, k = 1
    and d_ff * k hidden units).  Also the memory footprint of the
    Mixtral-shaped step from the library's size functions, beside the
    grouped input copy a copy-based design would add."""
    import sparse_mixture_experts_top_amd as smoe
    from workloads import make_mlp
    steps, warmup = args.steps, args.warmup
    T, d, f, E = 16384, 1024, 1024, 16
    pts = []
    for k in (1, 2, 4, 8, 16):
        row = {"k": k}
        for kind, (EE, kk, ff) in (("smoe", (E, k, f)), ("dense", (1, 1, f * k))):
            w = make_mlp(T, d, ff, EE, kk, "gelu", "bf16", 960 + 2 * k + (kind == "dense"), routing="softmax",
                         w_std=0.02)
            t = {n: _dev(w.tensors[n]) for n in ("x", "w1", "w2", "expert_idxs", "gates", "dout")}

            def step():
                out, saved = smoe.smoe_mlp_fwd(t["x"], t["w1"], t["w2"], t["expert_idxs"], t["gates"], "gelu")
                smoe.smoe_mlp_bwd(t["dout"], t["x"], t["w1"], t["w2"], t["expert_idxs"], t["gates"], "gelu", saved)

            ms = _event_ms(step, steps, warmup)
            fl = sum(gemm_flops(T, kk, d, ff, "gelu").values())
            row[kind] = {"ms": ms, "tokens_per_s": T / (ms * 1e-3), "tflops": fl / (ms * 1e-3) / 1e12}
            del t, w
        row["smoe_over_dense"] = row["dense"]["ms"] / row["smoe"]["ms"]
        pts.append(row)
    # memory footprint of the Mixtral-shaped step (bytes)
    Tm, km, Em, dm, fm = 16384, 2, 8, 4096, 14336
    a, bf = smoe.ACT_SWIGLU, smoe.BF16
    mem = {"saved": smoe.lib.smoe_mlp_saved_bytes(Tm, km, Em, dm, fm, a, bf),
           "fwd_workspace": smoe.lib.smoe_mlp_fwd_workspace_bytes(Tm, km, Em, dm, fm, a, bf),
           "fwd_workspace_fused_combine": smoe.lib.smoe_mlp_fwd_fused_combine_workspace_bytes(Tm, km, Em, dm, fm,
                                                                                              a, bf),
           "bwd_workspace": smoe.lib.smoe_mlp_bwd_workspace_bytes(Tm, km, Em, dm, fm, a, bf),
           "grouped_input_copy_avoided": Tm * km * dm * 2,
           "what": "Mixtral-shaped step; saved holds the routing arrays and h1, h3 (a is recomputed); the "
                   "scattered-in products read x in place, so no grouped copy of x (T*k*d_model*2 bytes) exists"}
    best = max(p["smoe_over_dense"] for p in pts)
    return {"metric": "SMoE-MLP over dense MLP of equal active FLOPs, time ratio (supplementary), 1 MI355X",
            "value": pts[1]["smoe_over_dense"], "unit": "x (dense ms / SMoE ms at k=2)", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "SMoE-MLP fwd+bwd, T=16384, d_model=1024, d_ff=1024 per expert, E=16, GELU, "
                                   "k swept 1..16; dense twin E=1, k=1, d_ff=1024*k"},
            "points": pts, "best_ratio": best, "memory_bytes": mem}


def combine_line(args):
    """SMoE-MLP forward (bf16) with the separate combine (smoe_mlp_fwd) and
    with the combine fused into the W2 product (smoe_mlp_fwd_fused_combine),
    at the Mixtral shape (k = 2) and the high-granularity shape (k = 8):
    device time per forward, and the W2 and combine launches of one call."""
    import torch
    import sparse_mixture_experts_top_amd as smoe
    from workloads import make_config
    steps, warmup = args.steps, args.warmup
    res = {}
    for cfg, label in ((3, "mixtral"), (4, "granular")):
        w = make_config(cfg)
        t = {n: _dev(w.tensors[n]) for n in ("x", "w1", "w2", "w3", "expert_idxs", "gates") if n in w.tensors}
        ws = None
        row = {"T": w.T, "k": w.k, "E": w.E}
        for fused in (False, True):
            def fwd():
                smoe.smoe_mlp_fwd(t["x"], t["w1"], t["w2"], t["expert_idxs"], t["gates"], w.act, w3=t.get("w3"),
                                  ws=ws, fused_combine=fused)
            ms = _event_ms(fwd, steps, warmup)
            evs = {r: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for r in ("down", "combine")}
            for r in evs:
                smoe.smoe_set_role_events(r, *evs[r])
            fwd()
            torch.cuda.synchronize()
            for r in evs:
                smoe.smoe_set_role_events(r, None, None)
            row["fused" if fused else "separate"] = {
                "fwd_ms": ms, "down_ms_last": evs["down"][0].elapsed_time(evs["down"][1]),
                "combine_ms_last": evs["combine"][0].elapsed_time(evs["combine"][1])}
        row["fused_over_separate"] = row["fused"]["fwd_ms"] / row["separate"]["fwd_ms"]
        dims = (w.T, w.k, w.E, w.dims["d_model"], w.dims["d_ff"], smoe.ACT_SWIGLU if w.act == "swiglu"
                else smoe.ACT_GELU, smoe.BF16)
        row["separate"]["ws_bytes"] = smoe.lib.smoe_mlp_fwd_workspace_bytes(*dims)
        row["fused"]["ws_bytes"] = smoe.lib.smoe_mlp_fwd_fused_combine_workspace_bytes(*dims)
        res[label] = row
        del t, w
        torch.cuda.empty_cache()
    return {"metric": "SMoE-MLP forward ms, separate vs fused combine (supplementary), 1 MI355X",
            "value": res["mixtral"]["fused"]["fwd_ms"], "unit": "ms (fused, Mixtral shape)", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "SMoE-MLP forward: Mixtral shape (T=16384, d_model=4096, d_ff=14336, E=8, "
                                   "k=2, SwiGLU) and high-granularity shape (T=16384, d_model=1024, d_ff=512, "
                                   "E=64, k=8, Zipf, GELU)"},
            "shapes": res}


def attention_line(args):
    """Mixture-of-Attention core, forward and backward, at the MoA workload's
    shape (2 sequences of 4096 tokens, 16 head experts of 128, k = 4, bf16).
    Algorithmic FLOP over the causal pairs (row r, key t'), n pairs in all:
    forward 4 * hd * n (q k^T and p v), backward 10 * hd * n (scores again,
    dp, dq, dk, dv)."""
    import torch
    import sparse_mixture_experts_top_amd as smoe
    from workloads import make_moa_attention
    steps, warmup = args.steps, args.warmup
    B, S, hd, E, k = 2, 4096, 128, 16, 4
    w = make_moa_attention(B, S, hd, E, k, "bf16", 950)
    t = {n: _dev(w.tensors[n]) for n in ("q", "k", "v", "do")}
    rt = smoe.smoe_route(_dev(w.tensors["expert_idxs"]), E)
    sidx = rt["sorted_scattered_idxs"]
    pairs = k * B * S * (S + 1) // 2
    fl_f, fl_b = 4.0 * hd * pairs, 10.0 * hd * pairs
    o, lse = smoe.smoe_moa_attention_fwd(t["q"], t["k"], t["v"], sidx, k, S)
    fwd_ms = _event_ms(lambda: smoe.smoe_moa_attention_fwd(t["q"], t["k"], t["v"], sidx, k, S), steps, warmup)
    bwd_ms = _event_ms(lambda: smoe.smoe_moa_attention_bwd(t["q"], t["k"], t["v"], sidx, k, S, o, lse, t["do"]),
                       steps, warmup)
    roles = ["attn_fwd", "attn_dq", "attn_dkv"]
    evs = {r: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for r in roles}
    for r in roles:
        smoe.smoe_set_role_events(r, *evs[r])
    smoe.smoe_moa_attention_fwd(t["q"], t["k"], t["v"], sidx, k, S)
    smoe.smoe_moa_attention_bwd(t["q"], t["k"], t["v"], sidx, k, S, o, lse, t["do"])
    torch.cuda.synchronize()
    for r in roles:
        smoe.smoe_set_role_events(r, None, None)
    kms = {r: evs[r][0].elapsed_time(evs[r][1]) for r in roles}
    tf = (fl_f + fl_b) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12
    fwd_tf = fl_f / (kms["attn_fwd"] * 1e-3) / 1e12
    # the whole layer: Q projection -> attention -> O projection with the
    # combine, forward and backward (2048-wide model, as the MoA workload)
    from workloads import make_moa_layer
    lw = make_moa_layer(B, S, 2048, hd, E, k, "bf16", 951)
    L = {n: _dev(lw.tensors[n]) for n in ("x", "wq", "wo", "k", "v", "dout", "expert_idxs", "gates")}
    T = lw.T

    def layer():
        rt2 = smoe.smoe_route(L["expert_idxs"], E)
        s2, off2 = rt2["sorted_scattered_idxs"], rt2["offsets"]
        qg = smoe.smoe_parallel_linear_fwd(L["x"], L["wq"], T, k, s2, off2, False, True)
        og, lse2 = smoe.smoe_moa_attention_fwd(qg, L["k"], L["v"], s2, k, S)
        smoe.smoe_parallel_linear_fwd(og, L["wo"], T, k, s2, off2, True, False, L["gates"])
        dog, _, _ = smoe.smoe_parallel_linear_bwd(og, L["wo"], T, k, s2, off2, True, False, L["dout"], L["gates"],
                                                  need_dgates=True)
        dqg, _, _ = smoe.smoe_moa_attention_bwd(qg, L["k"], L["v"], s2, k, S, og, lse2, dog)
        smoe.smoe_parallel_linear_bwd(L["x"], L["wq"], T, k, s2, off2, False, True, dqg)

    layer_ms = _event_ms(layer, steps, warmup)
    return {"metric": "MoA attention core fwd+bwd TFLOP/s (supplementary), 1 MI355X", "value": tf,
            "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "Mixture-of-Attention core: 2 sequences x 4096 tokens, 16 head experts of 128, "
                                   "k=4, grouped queries against shared K/V, causal, bf16"},
            "fwd_ms": fwd_ms, "bwd_ms": bwd_ms, "fwd_tflops": fl_f / (fwd_ms * 1e-3) / 1e12,
            "bwd_tflops": fl_b / (bwd_ms * 1e-3) / 1e12, "kernels_ms_last_launch": kms,
            "moa_layer": {"ms_per_step": layer_ms, "tokens_per_s": T / (layer_ms * 1e-3),
                          "what": "route + Q projection + attention core + O projection with the combine, "
                                  "forward and backward, d_model=2048"},
            "roofline": {"bound": "mfma", "kernel": "attn_fwd", "achieved": fwd_tf, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": fwd_tf / PEAK_BF16_TFLOPS, "traffic": None,
                         "flop_per_launch": fl_f, "avg_launch_ms": kms["attn_fwd"]}}


if __name__ == "__main__":
    main()
