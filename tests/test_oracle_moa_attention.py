"""Pins for oracle.moa_attention_fwd / moa_attention_bwd.

* One expert, k = 1 (grouped order = token order): torch's own causal
  scaled-dot-product attention, per sequence, in fp64 on the CPU, and its
  autograd gradients.
* Several experts: a dense masked formula in torch fp64 (every grouped row
  against every key, keys outside the row's sequence prefix set to -inf)
  with autograd for the gradients; the normaliser against torch.logsumexp.
* Permuting the grouped rows permutes o and dq and leaves dK and dV alone;
  a row at its sequence's first position returns that position's value.
* The backward given the forward's exact o (D_r = do_r . o_r) equals the
  backward that forms D_r = sum p dp itself.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _setup(B=2, S=24, hd=16, E=4, k=2, seed=0):
    rng = np.random.default_rng([seed, 77])
    T = B * S
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    # grouped order: assignments p = t*k + j sorted by expert, stable in p
    sidx = np.argsort(ids.reshape(-1), kind="stable").astype(np.int32)
    M = T * k
    q = rng.standard_normal((M, hd))
    kk = rng.standard_normal((T, hd))
    v = rng.standard_normal((T, hd))
    do = rng.standard_normal((M, hd))
    return q, kk, v, do, sidx, k, S


def _dense(q, kk, v, sidx, k, S):
    """Dense masked attention in torch fp64 (autograd-ready tensors in)."""
    hd = q.shape[1]
    tok = torch.as_tensor(np.asarray(sidx) // k, dtype=torch.int64)
    lo = (tok // S) * S
    j = torch.arange(kk.shape[0], dtype=torch.int64)
    ok = (j[None, :] >= lo[:, None]) & (j[None, :] <= tok[:, None])
    z = (q @ kk.T) / math.sqrt(hd)
    z = z.masked_fill(~ok, float("-inf"))
    return torch.softmax(z, dim=1) @ v, torch.logsumexp(z, dim=1)


def test_single_expert_matches_torch_causal_sdpa():
    B, S, hd = 3, 20, 8
    rng = np.random.default_rng(5)
    T = B * S
    q, kk, v, do = (rng.standard_normal((T, hd)) for _ in range(4))
    sidx = np.arange(T, dtype=np.int32)
    f = oracle.moa_attention_fwd(q, kk, v, sidx, 1, S)
    b = oracle.moa_attention_bwd(q, kk, v, sidx, 1, S, do)
    qt, kt, vt = (torch.tensor(a.reshape(B, 1, S, hd), requires_grad=True) for a in (q, kk, v))
    ot = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    ot.backward(torch.tensor(do.reshape(B, 1, S, hd)))
    np.testing.assert_allclose(f["o"], ot.detach().numpy().reshape(T, hd), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b["dq"], qt.grad.numpy().reshape(T, hd), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["dk"], kt.grad.numpy().reshape(T, hd), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["dv"], vt.grad.numpy().reshape(T, hd), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_grouped_rows_match_dense_masked_autograd(seed):
    q, kk, v, do, sidx, k, S = _setup(seed=seed)
    f = oracle.moa_attention_fwd(q, kk, v, sidx, k, S)
    b = oracle.moa_attention_bwd(q, kk, v, sidx, k, S, do)
    qt, kt, vt = (torch.tensor(a, requires_grad=True) for a in (q, kk, v))
    ot, lse = _dense(qt, kt, vt, sidx, k, S)
    ot.backward(torch.tensor(do))
    np.testing.assert_allclose(f["o"], ot.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f["lse"], lse.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b["dq"], qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["dk"], kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["dv"], vt.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_row_permutation_and_first_position():
    q, kk, v, do, sidx, k, S = _setup(seed=3)
    M = q.shape[0]
    perm = np.random.default_rng(9).permutation(M)
    f = oracle.moa_attention_fwd(q, kk, v, sidx, k, S)
    b = oracle.moa_attention_bwd(q, kk, v, sidx, k, S, do)
    fp = oracle.moa_attention_fwd(q[perm], kk, v, sidx[perm], k, S)
    bp = oracle.moa_attention_bwd(q[perm], kk, v, sidx[perm], k, S, do[perm])
    np.testing.assert_allclose(fp["o"], f["o"][perm], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(bp["dq"], b["dq"][perm], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(bp["dk"], b["dk"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(bp["dv"], b["dv"], rtol=1e-11, atol=1e-12)
    # rows of tokens at position 0 of their sequence see one key: o = v
    for r in range(M):
        t = int(sidx[r]) // k
        if t % S == 0:
            np.testing.assert_array_equal(f["o"][r], v[t])


def test_backward_from_exact_stored_output_is_the_same():
    q, kk, v, do, sidx, k, S = _setup(seed=4)
    f = oracle.moa_attention_fwd(q, kk, v, sidx, k, S)
    a = oracle.moa_attention_bwd(q, kk, v, sidx, k, S, do)
    b = oracle.moa_attention_bwd(q, kk, v, sidx, k, S, do, o=f["o"])
    for n in ("dq", "dk", "dv"):
        np.testing.assert_allclose(b[n], a[n], rtol=1e-10, atol=1e-12)
