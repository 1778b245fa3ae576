"""Python binding of libsmoe.so, the C-ABI scattered mixture-of-experts
library for MI355X (gfx950).

Argument marshalling only: torch supplies device memory (outputs, workspaces)
and the current stream; every step of the computation runs in the library's
HIP kernels.  The function names are the C entry points' names.  Importing
this package fails loudly when the library has not been built.

Layouts follow include/smoe.h: x [rows, d], weights [E, d_in, d_out],
expert choices and gates [T, k], assignment p = t*k + j.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Optional

import torch

__all__ = [
    "LIB_PATH", "SmoeError", "lib", "smoe_route", "smoe_parallel_linear_fwd",
    "smoe_parallel_linear_bwd", "smoe_mlp_fwd", "smoe_mlp_bwd", "saved_views",
    "header_functions", "F32", "BF16", "ACT_GELU", "ACT_SWIGLU", "ROLES", "smoe_set_role_events",
    "smoe_probe_mfma_loop", "smoe_router_fwd", "smoe_router_bwd", "smoe_moa_attention_fwd",
    "smoe_moa_attention_bwd", "SmoeAux", "default_aux",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsmoe.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "smoe.h")

F32, BF16 = 0, 1
ACT_GELU, ACT_SWIGLU = 0, 1
_ACTS = {"gelu": ACT_GELU, "swiglu": ACT_SWIGLU}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python sparse_mixture_experts_top_amd/build.py` (hipcc, gfx950)")
lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


class SmoeAux(ctypes.Structure):
    """struct smoe_aux: the caller's second stream and its fork / join events."""
    _fields_ = [("stream", _vp), ("fork_event", _vp), ("join_event", _vp)]


_AUXP = ctypes.POINTER(SmoeAux)
_SIGS = {
    "smoe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "smoe_last_error": (ctypes.c_char_p, []),
    "smoe_abi_version": (ctypes.c_int, []),
    "smoe_route_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "smoe_route": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "smoe_route_noalloc": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "smoe_parallel_linear_fwd_workspace_bytes": (_sz, [_i64, _i32, _i32, _i64, _i64, _i32, _i32]),
    "smoe_parallel_linear_fwd": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _i32, _i64, _i32, _vp, _vp,
                                                _i32, _i32, _vp, _vp, _i32, _vp, _sz, _vp]),
    "smoe_parallel_linear_bwd_workspace_bytes": (_sz, [_i64, _i32, _i32, _i64, _i64, _i64, _i32, _i32, _i32]),
    "smoe_parallel_linear_bwd": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _i32, _i64, _i32, _vp, _vp,
                                                _i32, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _vp, _i32, _vp,
                                                _sz, _vp]),
    "smoe_mlp_saved_bytes": (_sz, [_i64, _i32, _i32, _i64, _i64, _i32, _i32]),
    "smoe_mlp_saved_offsets": (ctypes.c_int, [_i64, _i32, _i32, _i64, _i64, _i32, _i32, ctypes.POINTER(_sz)]),
    "smoe_mlp_fwd_workspace_bytes": (_sz, [_i64, _i32, _i32, _i64, _i64, _i32, _i32]),
    "smoe_mlp_fwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _i32, _i32,
                                    _vp, _vp, _sz, _vp, _sz, _AUXP, _vp]),
    "smoe_mlp_fwd_fused_combine_workspace_bytes": (_sz, [_i64, _i32, _i32, _i64, _i64, _i32, _i32]),
    "smoe_mlp_fwd_fused_combine": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp,
                                                  _i32, _i32, _vp, _vp, _sz, _vp, _sz, _AUXP, _vp]),
    "smoe_mlp_bwd_workspace_bytes": (_sz, [_i64, _i32, _i32, _i64, _i64, _i32, _i32]),
    "smoe_set_role_events": (ctypes.c_int, [_i32, _vp, _vp]),
    "smoe_probe_mfma_loop": (ctypes.c_int, [_vp, _i32, _i32, _vp]),
    "smoe_router_fwd": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "smoe_router_bwd_workspace_bytes": (_sz, [_i64, _i64, _i32]),
    "smoe_router_bwd": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32,
                                       _vp, _sz, _vp]),
    "smoe_moa_attention_fwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i64, _i64, _i32, _vp, _vp, _vp]),
    "smoe_moa_attention_bwd_workspace_bytes": (_sz, [_i64, _i32, _i64, _i64]),
    "smoe_moa_attention_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i32, _i64, _i64, _i32, _vp, _vp, _vp,
                                              _vp, _vp, _vp, _vp, _sz, _vp]),
    "smoe_mlp_bwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _i32,
                                    _i32, _vp, _sz, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _sz, _AUXP, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def header_functions():
    """Names of the functions declared in include/smoe.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(smoe_\w+)\s*\(", text, re.M)))


class SmoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib.smoe_last_error().decode() or lib.smoe_status_string(status).decode()
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


def _check(status: int, where: str):
    if status != 0:
        raise SmoeError(status, where)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_AUX = {}


def default_aux(device) -> SmoeAux:
    """A second stream (default priority) and two events for `device`,
    created through torch once and kept for the process."""
    dev = torch.device(device)
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    if key not in _AUX:
        with torch.cuda.device(key):
            side = torch.cuda.Stream(device=key)
            evs = [torch.cuda.Event(enable_timing=False), torch.cuda.Event(enable_timing=False)]
            for ev in evs:        # torch creates the HIP event on first record
                ev.record()
            torch.cuda.current_stream(key).synchronize()
        _AUX[key] = (side, evs, SmoeAux(side.cuda_stream, evs[0].cuda_event, evs[1].cuda_event))
    return _AUX[key][2]


def _aux_arg(aux, device):
    """aux=True: the device's default second stream; False/None: none;
    an SmoeAux: as given."""
    if aux is True:
        return ctypes.pointer(default_aux(device))
    if isinstance(aux, SmoeAux):
        return ctypes.pointer(aux)
    return None


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


# --------------------------------------------------------------------------
def smoe_route(expert_idxs: torch.Tensor, E: int) -> Dict[str, torch.Tensor]:
    """Routing indices of expert_idxs [T, k] (int32, on the GPU)."""
    _contig(expert_idxs)
    T, k = expert_idxs.shape
    dev = expert_idxs.device
    M = T * k
    out = {
        "sorted_expert_idxs": torch.empty(M, dtype=torch.int32, device=dev),
        "sorted_scattered_idxs": torch.empty(M, dtype=torch.int32, device=dev),
        "counts": torch.empty(E, dtype=torch.int32, device=dev),
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
    }
    ws = _ws(lib.smoe_route_workspace_bytes(T, k, E), dev)
    _check(lib.smoe_route(_p(expert_idxs), T, k, E, _p(out["sorted_expert_idxs"]),
                          _p(out["sorted_scattered_idxs"]), _p(out["counts"]), _p(out["offsets"]),
                          _p(ws), ws.numel(), _stream(dev)), "smoe_route")
    return out


def smoe_router_fwd(x: torch.Tensor, w: torch.Tensor, k: int, want_logits: bool = False) -> Dict[str, torch.Tensor]:
    """Top-k softmax router: x [T, d], gate weight w [E, d] (logits = x w^T)
    -> expert_idxs [T, k] int32, gates [T, k] fp32 (and logits [T, E] fp32)."""
    _contig(x, w)
    T, d = x.shape
    E = w.shape[0]
    dev = x.device
    out = {"expert_idxs": torch.empty((T, k), dtype=torch.int32, device=dev),
           "gates": torch.empty((T, k), dtype=torch.float32, device=dev)}
    if want_logits:
        out["logits"] = torch.empty((T, E), dtype=torch.float32, device=dev)
    _check(lib.smoe_router_fwd(_p(x), _p(w), T, d, E, k, _dtype_code(x), _p(out["expert_idxs"]), _p(out["gates"]),
                               _p(out.get("logits")), _stream(dev)), "smoe_router_fwd")
    return out


def smoe_router_bwd(x, w, expert_idxs, gates, dgates, dx=None, accumulate: bool = False):
    """Backward of smoe_router_fwd: returns (dw [E, d] fp32, dx [T, d]); with
    accumulate the router's dx is added to the given dx."""
    _contig(x, w, expert_idxs, gates, dgates, dx)
    T, d = x.shape
    E = w.shape[0]
    k = expert_idxs.shape[1]
    dev = x.device
    dw = torch.empty((E, d), dtype=torch.float32, device=dev)
    if dx is None:
        dx = torch.empty_like(x)
        accumulate = False
    ws = _ws(lib.smoe_router_bwd_workspace_bytes(T, d, E), dev)
    _check(lib.smoe_router_bwd(_p(x), _p(w), T, d, E, k, _dtype_code(x), _p(expert_idxs), _p(gates), _p(dgates),
                               _p(dw), _p(dx), int(accumulate), _p(ws), ws.numel(), _stream(dev)), "smoe_router_bwd")
    return dw, dx


def smoe_moa_attention_fwd(q, k_, v, sorted_scattered_idxs, k: int, seq_len: int):
    """Mixture-of-Attention core: grouped queries q [T*k, hd] against shared
    k_, v [T, hd] (causal within sequences of seq_len tokens) -> (o [T*k, hd]
    grouped, lse [T*k] fp32)."""
    _contig(q, k_, v, sorted_scattered_idxs)
    T, hd = k_.shape
    dev = q.device
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[0],), dtype=torch.float32, device=dev)
    _check(lib.smoe_moa_attention_fwd(_p(q), _p(k_), _p(v), _p(sorted_scattered_idxs), T, k, seq_len, hd,
                                      _dtype_code(q), _p(o), _p(lse), _stream(dev)), "smoe_moa_attention_fwd")
    return o, lse


def smoe_moa_attention_bwd(q, k_, v, sorted_scattered_idxs, k: int, seq_len: int, o, lse, dout):
    """Backward of smoe_moa_attention_fwd: returns (dq [T*k, hd], dk, dv [T, hd])."""
    _contig(q, k_, v, sorted_scattered_idxs, o, lse, dout)
    T, hd = k_.shape
    dev = q.device
    dq = torch.empty_like(q)
    dk = torch.empty_like(k_)
    dv = torch.empty_like(v)
    ws = _ws(lib.smoe_moa_attention_bwd_workspace_bytes(T, k, seq_len, hd), dev)
    _check(lib.smoe_moa_attention_bwd(_p(q), _p(k_), _p(v), _p(sorted_scattered_idxs), T, k, seq_len, hd,
                                      _dtype_code(q), _p(o), _p(lse), _p(dout), _p(dq), _p(dk), _p(dv), _p(ws),
                                      ws.numel(), _stream(dev)), "smoe_moa_attention_bwd")
    return dq, dk, dv


def smoe_parallel_linear_fwd(x, w, T, k, sorted_scattered_idxs, offsets, x_grouped: bool,
                             y_grouped: bool, gates=None):
    """scatter2scatter forward; returns y ([T*k, d_out], or [T, d_out] with gates)."""
    _contig(x, w, sorted_scattered_idxs, offsets, gates)
    E, d_in, d_out = w.shape
    dev = x.device
    dt = _dtype_code(x)
    y = torch.empty((T if gates is not None else T * k, d_out), dtype=x.dtype, device=dev)
    ws = _ws(lib.smoe_parallel_linear_fwd_workspace_bytes(T, k, E, d_in, d_out, int(gates is not None), dt), dev)
    _check(lib.smoe_parallel_linear_fwd(_p(x), x.shape[0], d_in, _p(w), d_out, E, T, k,
                                        _p(sorted_scattered_idxs), _p(offsets), int(x_grouped),
                                        int(y_grouped), _p(gates), _p(y), dt, _p(ws), ws.numel(),
                                        _stream(dev)), "smoe_parallel_linear_fwd")
    return y


def smoe_parallel_linear_bwd(x, w, T, k, sorted_scattered_idxs, offsets, x_grouped: bool,
                             y_grouped: bool, dy, gates=None, need_dx=True, need_dw=True,
                             need_dgates=False, dx_dtype=None, dw_dtype=torch.float32, dw=None,
                             accumulate_dw=False):
    """Backward of smoe_parallel_linear_fwd; returns (dx, dw, dgates fp32).
    dx_dtype (default: x's dtype) and dw_dtype pick the output types; with
    dw given and accumulate_dw the gradient is added to it."""
    _contig(x, w, dy, sorted_scattered_idxs, offsets, gates, dw)
    E, d_in, d_out = w.shape
    dev = x.device
    dt = _dtype_code(x)
    dx_dt = x.dtype if dx_dtype is None else dx_dtype
    dx = torch.empty(x.shape, dtype=dx_dt, device=dev) if need_dx else None
    if dw is None and need_dw:
        dw = torch.empty((E, d_in, d_out), dtype=dw_dtype, device=dev)
        accumulate_dw = False
    dg = torch.empty((T, k), dtype=torch.float32, device=dev) if need_dgates else None
    ws = _ws(lib.smoe_parallel_linear_bwd_workspace_bytes(T, k, E, x.shape[0], d_in, d_out, int(x_grouped),
                                                          int(gates is not None), dt), dev)
    _check(lib.smoe_parallel_linear_bwd(_p(x), x.shape[0], d_in, _p(w), d_out, E, T, k,
                                        _p(sorted_scattered_idxs), _p(offsets), int(x_grouped),
                                        int(y_grouped), _p(gates), _p(dy), _p(dx),
                                        _dtype_code(dx) if dx is not None else dt, _p(dw),
                                        _dtype_code(dw) if dw is not None else F32, int(accumulate_dw), _p(dg),
                                        dt, _p(ws), ws.numel(), _stream(dev)), "smoe_parallel_linear_bwd")
    return dx, dw, dg


def _mlp_dims(x, w1, w2, expert_idxs):
    T, d_model = x.shape
    E, _, d_ff = w1.shape
    k = expert_idxs.shape[1]
    return T, d_model, d_ff, E, k


def smoe_mlp_fwd(x, w1, w2, expert_idxs, gates, act: str, w3=None, ws=None, fused_combine=False, aux=True):
    """SMoE-MLP forward; returns (out [T, d_model], saved buffer).
    fused_combine=True calls smoe_mlp_fwd_fused_combine (the gated k-sum
    added with fp32 atomics inside the W2 product).  aux: the second stream
    (True: the device's default one; False: run on the current stream only;
    or an SmoeAux)."""
    _contig(x, w1, w2, w3, expert_idxs, gates)
    T, d_model, d_ff, E, k = _mlp_dims(x, w1, w2, expert_idxs)
    dev = x.device
    dt = _dtype_code(x)
    a = _ACTS[act]
    out = torch.empty((T, d_model), dtype=x.dtype, device=dev)
    saved = _ws(lib.smoe_mlp_saved_bytes(T, k, E, d_model, d_ff, a, dt), dev)
    need = (lib.smoe_mlp_fwd_fused_combine_workspace_bytes if fused_combine
            else lib.smoe_mlp_fwd_workspace_bytes)(T, k, E, d_model, d_ff, a, dt)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    fn, name = ((lib.smoe_mlp_fwd_fused_combine, "smoe_mlp_fwd_fused_combine") if fused_combine
                else (lib.smoe_mlp_fwd, "smoe_mlp_fwd"))
    _check(fn(_p(x), _p(w1), _p(w3), _p(w2), T, d_model, d_ff, E, k, _p(expert_idxs),
              _p(gates), a, dt, _p(out), _p(saved), saved.numel(), _p(ws), ws.numel(),
              _aux_arg(aux, dev), _stream(dev)), name)
    return out, saved


def smoe_mlp_bwd(dout, x, w1, w2, expert_idxs, gates, act: str, saved, w3=None, ws=None,
                 need_dgates=True, dw_dtype=torch.float32, aux=True):
    """SMoE-MLP backward; returns dict dx, dw1, dw2, dw3 (dw_dtype), dgates.
    aux as in smoe_mlp_fwd."""
    _contig(dout, x, w1, w2, w3, expert_idxs, gates, saved)
    T, d_model, d_ff, E, k = _mlp_dims(x, w1, w2, expert_idxs)
    dev = x.device
    dt = _dtype_code(x)
    a = _ACTS[act]
    dx = torch.empty_like(x)
    dw1 = torch.empty(w1.shape, dtype=dw_dtype, device=dev)
    dw2 = torch.empty(w2.shape, dtype=dw_dtype, device=dev)
    dw3 = torch.empty(w1.shape, dtype=dw_dtype, device=dev) if w3 is not None else None
    dg = torch.empty((T, k), dtype=torch.float32, device=dev) if need_dgates else None
    need = lib.smoe_mlp_bwd_workspace_bytes(T, k, E, d_model, d_ff, a, dt)
    if ws is None or ws.numel() < need:
        ws = _ws(need, dev)
    _check(lib.smoe_mlp_bwd(_p(dout), _p(x), _p(w1), _p(w3), _p(w2), T, d_model, d_ff, E, k,
                            _p(expert_idxs), _p(gates), a, dt, _p(saved), saved.numel(), _p(dx), _p(dw1),
                            _p(dw3), _p(dw2), _dtype_code(dw1), _p(dg), _p(ws), ws.numel(), _aux_arg(aux, dev),
                            _stream(dev)), "smoe_mlp_bwd")
    return {"dx": dx, "dw1": dw1, "dw2": dw2, "dw3": dw3, "dgates": dg}


ROLES = ["route", "up", "down", "combine", "dA", "dW2", "dX", "ksum", "dW1", "dW3", "dw_reduce",
         "dg_reduce", "pl_fwd", "pl_dx", "pl_dw", "router_fwd", "router_dx", "router_dw", "attn_fwd",
         "attn_dq", "attn_dkv"]


def smoe_set_role_events(role: str, start=None, stop=None):
    """Attach torch.cuda.Event objects (enable_timing=True) to a launch role;
    None detaches.  Events are recorded once first so that they exist."""
    if start is not None:
        for ev in (start, stop):
            if not ev.cuda_event:
                ev.record()
    _check(lib.smoe_set_role_events(ROLES.index(role), ctypes.c_void_p(start.cuda_event) if start else None,
                                    ctypes.c_void_p(stop.cuda_event) if stop else None),
           "smoe_set_role_events")


def smoe_probe_mfma_loop(out: torch.Tensor, blocks: int, iters: int):
    """Enqueue the matrix-core rate probe on the current stream; out is a
    float32 device tensor of blocks*256 elements.  FLOP = blocks * 4 * iters
    * 16 * 32768."""
    assert out.dtype == torch.float32 and out.is_cuda and out.numel() >= blocks * 256
    _check(lib.smoe_probe_mfma_loop(_p(out), blocks, iters, _stream(out.device)), "smoe_probe_mfma_loop")


def workspace_bytes(kind: str, **kw) -> int:
    """Bytes of scratch the named entry point needs (for callers that keep
    one workspace across calls)."""
    f = getattr(lib, f"smoe_{kind}_workspace_bytes")
    return int(f(*kw.values()))


def saved_views(saved: torch.Tensor, T: int, k: int, E: int, d_model: int, d_ff: int, act: str,
                dtype: torch.dtype) -> Dict[str, torch.Tensor]:
    """Views into the `saved` buffer of smoe_mlp_fwd (routing arrays, h)."""
    off = (ctypes.c_size_t * 6)()
    dt = BF16 if dtype == torch.bfloat16 else F32
    _check(lib.smoe_mlp_saved_offsets(T, k, E, d_model, d_ff, _ACTS[act], dt, off), "smoe_mlp_saved_offsets")
    M = T * k
    es = 2 if dt == BF16 else 4

    def view(o, n, tdt, nbytes):
        return saved[o:o + nbytes].view(tdt)[:n]

    v = {
        "sorted_expert_idxs": view(off[0], M, torch.int32, M * 4),
        "sorted_scattered_idxs": view(off[1], M, torch.int32, M * 4),
        "counts": view(off[2], E, torch.int32, E * 4),
        "offsets": view(off[3], E + 1, torch.int32, (E + 1) * 4),
        "h": view(off[4], M * d_ff, dtype, M * d_ff * es).view(M, d_ff),
    }
    if act == "swiglu":
        v["h3"] = view(off[5], M * d_ff, dtype, M * d_ff * es).view(M, d_ff)
    return v
