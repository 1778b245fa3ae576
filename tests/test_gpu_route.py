"""smoe_route on the GPU: bit-exact against the oracle for the workloads'
routings and the edge cases (k = E, E = 1, one hot expert, empty experts,
ragged sizes around the 4096-assignment chunk, T = 0, invalid ids)."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import say
from workloads import uniform_distinct_routing, zipf_routing, topk_softmax_routing

pytestmark = pytest.mark.gpu


def _run(smoe, idx, E):
    say(f"route T={idx.shape[0]} k={idx.shape[1] if idx.ndim == 2 else 0} E={E}")
    d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    r = smoe.smoe_route(d, E)
    torch.cuda.synchronize()
    return {n: v.cpu().numpy().astype(np.int64) for n, v in r.items()}


def _exact(smoe, idx, E):
    got = _run(smoe, idx, E)
    ref = oracle.route(idx, E)
    for n in ("counts", "offsets", "sorted_scattered_idxs", "sorted_expert_idxs"):
        np.testing.assert_array_equal(got[n], ref[n], err_msg=n)


@pytest.mark.parametrize("T,E,k", [(256, 8, 2), (8192, 16, 2), (16384, 8, 2), (8192, 16, 4),
                                   (1, 1, 1), (4095, 3, 1), (4097, 7, 3), (2049, 64, 2),
                                   (5000, 1024, 2), (1000, 5, 5)])
def test_route_uniform(smoe, T, E, k):
    _exact(smoe, uniform_distinct_routing(T, E, k, (300, T, E, k)), E)


def test_route_zipf_full_size(smoe):
    idx, _ = zipf_routing(16384, 64, 8, 1.1, 8, (4, 4))
    _exact(smoe, idx, 64)


def test_route_softmax_topk(smoe):
    logits = np.random.default_rng(31).standard_normal((3000, 16))
    idx, _ = topk_softmax_routing(logits, 4)
    _exact(smoe, idx, 16)


def test_route_one_hot_expert_and_repeats(smoe):
    _exact(smoe, np.full((9000, 2), 5, dtype=np.int32), 8)
    rng = np.random.default_rng(32)
    _exact(smoe, rng.integers(0, 3, size=(7000, 4)).astype(np.int32), 3)   # repeats allowed


def test_route_empty(smoe):
    got = _run(smoe, np.zeros((0, 2), dtype=np.int32), 6)
    assert got["offsets"].tolist() == [0] * 7
    assert got["counts"].tolist() == [0] * 6


def test_route_invalid_ids_are_dropped(smoe):
    idx = uniform_distinct_routing(500, 6, 2, (33, 0)).copy()
    bad = idx.copy()
    bad[3, 1] = 6
    bad[10, 0] = -1
    got = _run(smoe, bad, 6)
    valid = [p for p, e in enumerate(bad.reshape(-1)) if 0 <= e < 6]
    assert got["offsets"][6] == len(valid) == 998
    flat = bad.reshape(-1)
    s = got["sorted_scattered_idxs"][:998]
    np.testing.assert_array_equal(s, np.array(valid)[np.argsort(flat[valid], kind="stable")])


def test_route_deterministic(smoe):
    idx, _ = zipf_routing(16384, 64, 8, 1.1, 8, (4, 4))
    a = _run(smoe, idx, 64)
    b = _run(smoe, idx, 64)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])
