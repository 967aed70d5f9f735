"""Pins the oracle's dense backward: finite differences, autograd, invariants."""
import math

import numpy as np
import pytest
import torch

from oracle import attn_bwd_dense, attn_fwd


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def _loss(q, k, v, dout, scale, causal):
    o, _ = attn_fwd(q, k, v, scale, causal)
    return float(np.sum(o * dout))


@pytest.mark.parametrize("causal", [True, False])
def test_dense_bwd_finite_differences(causal):
    # L = sum(dO * O): its gradient wrt Q, K, V is exactly (dQ, dK, dV).
    B, Hq, Hkv, N, d = 1, 4, 2, 12, 6
    q, k, v = _rand((B, Hq, N, d), 10), _rand((B, Hkv, N, d), 11), _rand((B, Hkv, N, d), 12)
    dout = _rand((B, Hq, N, d), 13)
    scale = 0.45
    dq, dk, dv = attn_bwd_dense(q, k, v, dout, scale, causal)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, dout, scale, causal)
            x[idx] = old - h
            lm = _loss(q, k, v, dout, scale, causal)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7, err_msg=name)


@pytest.mark.parametrize("causal", [True, False])
def test_dense_bwd_matches_torch_autograd(causal):
    B, Hq, Hkv, N, d = 2, 8, 2, 64, 16
    q, k, v = _rand((B, Hq, N, d), 20), _rand((B, Hkv, N, d), 21), _rand((B, Hkv, N, d), 22)
    dout = _rand((B, Hq, N, d), 23)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = attn_bwd_dense(q, k, v, dout, scale, causal)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=True)
    o.backward(torch.from_numpy(dout))
    for name, a, t in (("dq", dq, tq), ("dk", dk, tk), ("dv", dv, tv)):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)


@pytest.mark.parametrize("causal", [True, False])
def test_dense_bwd_invariants(causal):
    # Every row of dS sums to zero, so sum_j dK_j = 0; sum_j dV_j = sum_i dO_i
    # (each probability row sums to one), summed over the heads of a group.
    B, Hq, Hkv, N, d = 1, 6, 3, 32, 8
    q, k, v = _rand((B, Hq, N, d), 30), _rand((B, Hkv, N, d), 31), _rand((B, Hkv, N, d), 32)
    dout = _rand((B, Hq, N, d), 33)
    _, dk, dv = attn_bwd_dense(q, k, v, dout, 0.3, causal)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-11)
    grouped = dout.reshape(B, Hkv, Hq // Hkv, N, d).sum(axis=(2, 3))
    np.testing.assert_allclose(dv.sum(axis=2), grouped, rtol=1e-12, atol=1e-11)
