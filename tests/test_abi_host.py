"""The C-ABI library loads on the CPU, exports every function that
include/smoe.h declares, and rejects bad arguments on the host without
touching a device (no compute calls here)."""
import ctypes

import pytest

smoe = pytest.importorskip("sparse_mixture_experts_top_amd")
lib = smoe.lib

NULL = None


def test_every_declared_symbol_is_exported():
    names = smoe.header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    for n in ("smoe_route", "smoe_parallel_linear_fwd", "smoe_parallel_linear_bwd",
              "smoe_mlp_fwd", "smoe_mlp_bwd"):
        assert n in names


def test_status_strings_and_version():
    assert lib.smoe_abi_version() == 2
    for s in range(7):
        assert lib.smoe_status_string(s)
    assert lib.smoe_status_string(0) == b"ok"


def test_workspace_sizes_are_consistent():
    assert lib.smoe_route_workspace_bytes(16384, 8, 64) >= 4 * 64 * 32
    b_small = lib.smoe_mlp_bwd_workspace_bytes(256, 2, 8, 128, 256, smoe.ACT_GELU, smoe.F32)
    b_big = lib.smoe_mlp_bwd_workspace_bytes(16384, 2, 8, 4096, 14336, smoe.ACT_SWIGLU, smoe.BF16)
    assert 0 < b_small < b_big
    s = lib.smoe_mlp_saved_bytes(16384, 2, 8, 4096, 14336, smoe.ACT_SWIGLU, smoe.BF16)
    assert s >= 2 * 32768 * 14336 * 2
    off = (ctypes.c_size_t * 6)()
    assert lib.smoe_mlp_saved_offsets(100, 2, 4, 64, 96, smoe.ACT_GELU, smoe.F32, off) == 0
    assert off[5] == ctypes.c_size_t(-1).value
    assert all(o % 256 == 0 for i, o in enumerate(off) if i != 5)
    assert lib.smoe_parallel_linear_fwd_workspace_bytes(8, 2, 4, 64, 64, 0, smoe.BF16) <= 256
    assert lib.smoe_parallel_linear_fwd_workspace_bytes(8, 2, 4, 64, 64, 1, smoe.BF16) >= 16 * 64 * 4


def _fake(addr=4096):
    return ctypes.c_void_p(addr)


def test_route_rejects_bad_arguments():
    f = lib.smoe_route
    assert f(_fake(), 4, 2, 0, _fake(), _fake(), _fake(), _fake(), _fake(), 1 << 20, NULL) == 2   # E = 0
    assert f(_fake(), 4, 2, 2000, _fake(), _fake(), _fake(), _fake(), _fake(), 1 << 20, NULL) == 2
    assert f(_fake(), 4, 0, 4, _fake(), _fake(), _fake(), _fake(), _fake(), 1 << 20, NULL) == 2   # k = 0
    assert f(NULL, 4, 2, 4, _fake(), _fake(), _fake(), _fake(), _fake(), 1 << 20, NULL) == 1
    assert f(_fake(), 4, 2, 4, _fake(), _fake(), _fake(), _fake(), _fake(), 0, NULL) == 4         # ws
    assert b"ws_bytes" in lib.smoe_last_error()


def test_parallel_linear_rejects_bad_arguments():
    f = lib.smoe_parallel_linear_fwd
    args = dict(x=_fake(), x_rows=8, d_in=64, w=_fake(), d_out=64, E=4, T=8, k=2, sidx=_fake(),
                off=_fake(), xg=0, yg=0, gates=NULL, y=_fake(), dtype=smoe.BF16, ws=_fake(),
                wsb=1 << 20, st=NULL)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(*a.values())

    assert call(dtype=7) == 3
    assert call(d_in=12) == 2                      # not a multiple of 8
    assert call(x_rows=5) == 2                     # neither T nor T*k
    assert call(xg=1, x_rows=8) == 2               # grouped input needs T*k rows
    assert call(w=NULL) == 1
    assert call(x=_fake(4098)) == 2                # misaligned
    assert call(gates=_fake(), yg=1) == 2          # combine needs scattered output
    assert call(gates=_fake(), wsb=16) == 4


def test_parallel_linear_bwd_rejects_bad_arguments():
    """The backward's output types and accumulation flag are checked on the
    host; fp32 runs take fp32 outputs only."""
    f = lib.smoe_parallel_linear_bwd
    args = dict(x=_fake(), x_rows=8, d_in=64, w=_fake(), d_out=64, E=4, T=8, k=2, sidx=_fake(), off=_fake(),
                xg=0, yg=0, gates=NULL, dy=_fake(), dx=_fake(), dx_dtype=smoe.BF16, dw=_fake(),
                dw_dtype=smoe.F32, acc=0, dg=NULL, dtype=smoe.BF16, ws=_fake(), wsb=1 << 20, st=NULL)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(*a.values())

    assert call(dx_dtype=4) == 3
    assert call(dw_dtype=-1) == 3
    assert call(dtype=smoe.F32, dx_dtype=smoe.BF16, dw_dtype=smoe.F32) == 3
    assert call(dtype=smoe.F32, dx_dtype=smoe.F32, dw_dtype=smoe.BF16) == 3
    assert call(dg=_fake()) == 1                   # dgates needs gates
    assert call(gates=_fake(), yg=1) == 2
    assert call(wsb=0) == 4


def test_gated_parallel_linear_bwd_keeps_no_scaled_copy_of_x():
    """With gates, the workspace grows by the gate-gradient partials and
    one float per assignment (the gates in grouped order, which scale the
    weight-gradient product's rows in registers), never by a [T*k, d_in]
    copy of the gate-scaled input."""
    for T, k, E, d_in, d_out, xg in ((8192, 4, 16, 128, 2048, 1), (8192, 4, 16, 2048, 128, 0),
                                     (16384, 2, 8, 4096, 4096, 0)):
        for dt in (smoe.F32, smoe.BF16):
            x_rows = T * k if xg else T
            plain = lib.smoe_parallel_linear_bwd_workspace_bytes(T, k, E, x_rows, d_in, d_out, xg, 0, dt)
            gated = lib.smoe_parallel_linear_bwd_workspace_bytes(T, k, E, x_rows, d_in, d_out, xg, 1, dt)
            slots = 4 * ((d_in + 255) // 256) if dt == smoe.BF16 else (d_in + 63) // 64
            extra = gated - plain
            assert extra <= slots * T * k * 4 + T * k * 4 + 1024, (T, k, d_in, dt, extra)
            assert extra < T * k * d_in * (2 if dt == smoe.BF16 else 4)


def test_aux_struct_layout():
    """struct smoe_aux is three pointers: stream, fork event, join event."""
    assert ctypes.sizeof(smoe.SmoeAux) == 3 * ctypes.sizeof(ctypes.c_void_p)
    assert [n for n, _ in smoe.SmoeAux._fields_] == ["stream", "fork_event", "join_event"]


@pytest.mark.parametrize("entry", ["smoe_mlp_fwd", "smoe_mlp_fwd_fused_combine"])
def test_mlp_rejects_bad_arguments(entry):
    f = getattr(lib, entry)
    base = [_fake(), _fake(), NULL, _fake(), 16, 64, 128, 4, 2, _fake(), _fake(), smoe.ACT_GELU,
            smoe.BF16, _fake(), _fake(), 1 << 30, _fake(), 1 << 30, NULL, NULL]
    a = list(base); a[11] = 5
    assert f(*a) == 3                              # unknown activation
    a = list(base); a[11] = smoe.ACT_SWIGLU
    assert f(*a) == 1                              # SwiGLU without w3
    a = list(base); a[2] = _fake()
    assert f(*a) == 1                              # w3 given for GELU
    a = list(base); a[15] = 8
    assert f(*a) == 4                              # saved too small
    a = list(base); a[17] = 8
    assert f(*a) == 4                              # workspace too small
    g = lib.smoe_mlp_bwd

    def bwd(dw3=NULL, dtype=smoe.BF16, dw_dtype=smoe.F32):
        return g(_fake(), _fake(), _fake(), NULL, _fake(), 16, 64, 128, 4, 2, _fake(), _fake(),
                 smoe.ACT_GELU, dtype, _fake(), 1 << 30, _fake(), _fake(), dw3, _fake(), dw_dtype, NULL,
                 _fake(), 1 << 30, NULL, NULL)

    assert bwd(dw3=_fake()) == 1                   # dw3 given for GELU
    assert bwd(dw_dtype=5) == 3                    # unknown weight-gradient type
    assert bwd(dtype=smoe.F32, dw_dtype=smoe.BF16) == 3   # fp32 runs give fp32 dw


def test_bf16_operands_beyond_32bit_offsets_are_rejected():
    """bf16 grouped products address operands with 32-bit byte offsets: a
    call whose [T*k, d] rows or one expert's weights reach 4 GiB fails on
    the host with a shape error instead of reading wrapped offsets."""
    f = lib.smoe_parallel_linear_fwd
    T, k = 300000, 2
    # [T*k, 4096] bf16 = 4.9 GB
    assert f(_fake(), T, 4096, _fake(), 64, 4, T, k, _fake(), _fake(), 0, 0, NULL, _fake(), smoe.BF16,
             _fake(), 1 << 30, NULL) == 2
    assert b"4 GiB" in lib.smoe_last_error()
    # one expert's weights [65536, 40000] bf16 = 5.2 GB
    assert f(_fake(), 8, 65536, _fake(), 40000, 4, 8, 2, _fake(), _fake(), 0, 0, NULL, _fake(), smoe.BF16,
             _fake(), 1 << 30, NULL) == 2
    assert b"w[e]" in lib.smoe_last_error()
    g = lib.smoe_mlp_fwd
    # hidden rows [2 * 160000, 14336] bf16 = 9.2 GB
    assert g(_fake(), _fake(), NULL, _fake(), 160000, 64, 14336, 4, 2, _fake(), _fake(), smoe.ACT_GELU,
             smoe.BF16, _fake(), _fake(), 1 << 40, _fake(), 1 << 40, NULL, NULL) == 2
    assert b"hidden rows" in lib.smoe_last_error()


def test_probe_rejects_bad_arguments():
    f = lib.smoe_probe_mfma_loop
    assert f(NULL, 8, 10, NULL) == 1
    assert f(_fake(), 0, 10, NULL) == 2
    assert f(_fake(), 8, 0, NULL) == 2


def test_router_rejects_bad_arguments():
    fwd, bwd = lib.smoe_router_fwd, lib.smoe_router_bwd

    def f(T=64, d=128, E=8, k=2, dtype=smoe.F32, x=_fake(), g=_fake()):
        return fwd(x, g, T, d, E, k, dtype, _fake(), _fake(), NULL, NULL)

    assert f(E=65) == 5                              # beyond one wave of experts
    assert f(E=0) == 5
    assert f(k=9, E=16) == 5                         # k beyond 8
    assert f(k=5, E=4) == 5                          # k beyond E
    assert f(k=0) == 5
    assert f(d=12) == 2                              # not a multiple of 8
    assert f(T=-1) == 2
    assert f(dtype=7) == 3
    assert f(g=NULL) == 1
    assert f(x=NULL) == 1
    assert f(x=_fake(4100)) == 2                     # misaligned
    ws = lib.smoe_router_bwd_workspace_bytes(1000, 256, 8)
    assert ws >= 1000 * 8 * 4 + 256 * 8 * 4
    assert lib.smoe_router_bwd_workspace_bytes(0, 256, 8) > 0
    assert lib.smoe_router_bwd_workspace_bytes(-1, 256, 8) == 0

    def b(wsb=ws, E=8, dx=_fake()):
        return bwd(_fake(), _fake(), 1000, 256, E, 2, smoe.F32, _fake(), _fake(), _fake(), _fake(), dx, 0,
                   _fake(), wsb, NULL)

    assert b(wsb=ws - 1) == 4
    assert b(E=100) == 5
    assert b(dx=NULL) == 1


def test_attention_rejects_bad_arguments():
    fwd, bwd = lib.smoe_moa_attention_fwd, lib.smoe_moa_attention_bwd

    def f(T=256, k=2, S=128, hd=128, dtype=smoe.BF16, q=_fake()):
        return fwd(q, _fake(), _fake(), _fake(), T, k, S, hd, dtype, _fake(), _fake(), NULL)

    assert f(dtype=smoe.F32) == 5                    # bf16 only
    assert f(dtype=9) == 3
    assert f(hd=64) == 5                             # head_dim 128 only
    assert f(T=200, S=128) == 2                      # T not a multiple of seq_len
    assert f(S=0) == 2
    assert f(k=0) == 2
    assert f(q=NULL) == 1
    assert f(q=_fake(4104)) == 2                     # misaligned
    assert f(T=0) == 0                               # nothing to do
    ws = lib.smoe_moa_attention_bwd_workspace_bytes(256, 2, 128, 128)
    assert ws >= 256 * 2 * 4 + 2 * 256 * 128 * 4
    assert lib.smoe_moa_attention_bwd_workspace_bytes(256, 2, 128, 64) == 0

    def b(wsb=ws, dq=_fake()):
        return bwd(_fake(), _fake(), _fake(), _fake(), 256, 2, 128, 128, smoe.BF16, _fake(), _fake(), _fake(), dq,
                   _fake(), _fake(), _fake(), wsb, NULL)

    assert b(wsb=ws - 1) == 4
    assert b(dq=NULL) == 1


def test_fused_combine_workspace_holds_token_rows_only():
    """The fused-combine forward's workspace is smoe_mlp_fwd's less the
    fp32 per-assignment rows beyond T: (T*k - T) * d_model * 4 bytes."""
    for T, k, E, d, f in ((16384, 2, 8, 4096, 14336), (16384, 8, 64, 1024, 512), (7, 1, 4, 64, 64)):
        for act in (smoe.ACT_GELU, smoe.ACT_SWIGLU):
            for dt in (smoe.F32, smoe.BF16):
                a = lib.smoe_mlp_fwd_workspace_bytes(T, k, E, d, f, act, dt)
                b = lib.smoe_mlp_fwd_fused_combine_workspace_bytes(T, k, E, d, f, act, dt)
                assert a - b == (T * k - T) * d * 4
