"""smoe_route_noalloc (the routing entry point for callers that cannot
allocate) against smoe_route on the GPU, bit for bit, through the C ABI: two
calls in a row, the second smaller than the first, and a size beyond the
static scratch rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _route_both(smoe, idx, E):
    T, k = idx.shape
    M = T * k
    dev = idx.device
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outs = []
    for noalloc in (False, True):
        o = {n: torch.full((m,), -7, dtype=torch.int32, device=dev)
             for n, m in (("se", M), ("ss", M), ("cnt", E), ("off", E + 1))}
        if noalloc:
            rc = smoe.lib.smoe_route_noalloc(_p(idx), T, k, E, _p(o["se"]), _p(o["ss"]), _p(o["cnt"]), _p(o["off"]),
                                             st)
        else:
            ws = torch.empty(max(1, smoe.lib.smoe_route_workspace_bytes(T, k, E)), dtype=torch.uint8, device=dev)
            rc = smoe.lib.smoe_route(_p(idx), T, k, E, _p(o["se"]), _p(o["ss"]), _p(o["cnt"]), _p(o["off"]), _p(ws),
                                     ws.numel(), st)
        assert rc == 0, smoe.lib.smoe_last_error()
        outs.append(o)
    torch.cuda.synchronize()
    return outs


def test_route_noalloc_matches_route(smoe):
    rng = np.random.default_rng(71)
    for T, k, E in ((60000, 8, 64), (3001, 2, 7)):      # the second call smaller
        say(f"route noalloc T={T} k={k} E={E}")
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        idx[rng.random(T) < 0.01, 0] = -1                   # dropped choices
        a, b = _route_both(smoe, torch.from_numpy(idx).cuda(), E)
        for n in ("se", "ss", "cnt", "off"):
            assert torch.equal(a[n], b[n]), n
        assert int(b["off"][-1]) == int((idx >= 0).sum())


def test_route_noalloc_rejects_sizes_beyond_its_scratch(smoe):
    f = smoe.lib.smoe_route_noalloc
    fake = ctypes.c_void_p(4096)
    # ceil(T*k/4096) * E = 4097 * 1024 > 2^20 ints
    assert f(fake, 4097 * 4096, 1, 1024, fake, fake, fake, fake, None) == 2
    assert b"static" in smoe.lib.smoe_last_error()
