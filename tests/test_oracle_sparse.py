"""Pins the oracle's sparse backward against its dense backward.

* delta = 0 keeps every block with w = 1: the sparse gradient is the dense one;
* for any keep set, the sparse gradient equals the dense gradient of the
  re-weighted output gradient dO' = keep * w * dO (the backward is linear in
  dO, and so is D = rowsum(dO * O));
* averaged over many draws the sparse gradient converges to the dense one
  with the variance of an unbiased 1/p estimator.
"""
import math

import numpy as np
import pytest

from oracle import attn_bwd_dense, attn_bwd_sparse, attn_fwd, block_masses, select


def _inputs(B, Hq, Hkv, N, d, seed, sigma=1.5):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    dout = rng.standard_normal((B, Hq, N, d)) * np.exp(sigma * rng.standard_normal((B, Hq, N, 1)))
    return q, k, v, dout


@pytest.mark.parametrize("causal", [True, False])
def test_sparse_delta_zero_equals_dense(causal):
    q, k, v, dout = _inputs(2, 4, 2, 64, 8, 40)
    scale = 1 / math.sqrt(8)
    sel = select(block_masses(dout, 16), 0.0, seed=5)
    assert sel["keep"].all() and np.all(sel["w"] == 1.0)
    sp = attn_bwd_sparse(q, k, v, dout, 16, sel["keep"], sel["w"], scale, causal)
    de = attn_bwd_dense(q, k, v, dout, scale, causal)
    for a, b in zip(sp, de):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_sparse_equals_dense_of_reweighted_dout(causal):
    q, k, v, dout = _inputs(1, 4, 1, 64, 8, 41)
    block, scale = 8, 0.3
    sel = select(block_masses(dout, block), 0.3, seed=9)
    assert 0 < sel["keep"].sum() < sel["keep"].size
    o, lse = attn_fwd(q, k, v, scale, causal)
    factor = np.repeat(sel["keep"] * sel["w"].astype(np.float64), block, axis=2)[..., None]
    de = attn_bwd_dense(q, k, v, dout * factor, scale, causal, o=o, lse=lse)
    sp = attn_bwd_sparse(q, k, v, dout, block, sel["keep"], sel["w"], scale, causal)
    for a, b in zip(sp, de):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)
    # skipped rows of dq are exact zeros
    skipped = np.repeat(~sel["keep"], block, axis=2)
    assert np.all(sp[0][skipped] == 0.0)


def test_sparse_head_subset_matches_full():
    q, k, v, dout = _inputs(1, 4, 2, 32, 8, 42)
    sel = select(block_masses(dout, 8), 0.2, seed=2)
    full = attn_bwd_sparse(q, k, v, dout, 8, sel["keep"], sel["w"], 0.35, True)
    part = attn_bwd_sparse(q, k, v, dout, 8, sel["keep"], sel["w"], 0.35, True,
                           heads=[(0, 2), (0, 3)])
    np.testing.assert_array_equal(part[0][0, 2:], full[0][0, 2:])
    np.testing.assert_allclose(part[1][0, 1], full[1][0, 1], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(part[2][0, 1], full[2][0, 1], rtol=1e-13, atol=1e-13)


@pytest.mark.slow
def test_sparse_mean_over_seeds_is_unbiased():
    # Per element, the estimator is sum_b (keep_b / p_b) c_b with c_b block b's
    # own dense contribution, so Var = sum_b (1 - p_b) / p_b * c_b**2.
    q, k, v, dout = _inputs(1, 2, 1, 64, 4, 43, sigma=1.0)
    block, scale, causal, delta = 8, 0.5, True, 0.3
    mass = block_masses(dout, block)
    sel0 = select(mass, delta, seed=0)
    p = sel0["p"]
    assert np.any((p > 0.05) & (p < 0.9))
    nqb = mass.shape[2]
    contrib = []                    # dense contribution of each (h, block)
    for h in range(2):
        for i in range(nqb):
            one = np.zeros_like(sel0["keep"])
            one[0, h, i] = True
            contrib.append((p[0, h, i], attn_bwd_sparse(q, k, v, dout, block, one,
                                                        np.ones_like(sel0["w"]), scale, causal)))
    dense = attn_bwd_dense(q, k, v, dout, scale, causal)
    K = 3000
    acc = [np.zeros_like(x) for x in dense]
    for s in range(K):
        keep = select(mass, delta, seed=s)["keep"]
        wts = [(keep[0, h, i] / p[0, h, i]) if keep[0, h, i] else 0.0
               for h in range(2) for i in range(nqb)]
        for (pb, c), wt in zip(contrib, wts):
            if wt:
                for a, x in zip(acc, c):
                    a += wt * x
    for t, (a, de) in enumerate(zip(acc, dense)):
        var = sum(((1 - pb) / pb) * c[t] ** 2 for pb, c in contrib)
        mean = a / K
        ok = var > 1e-20
        z = (mean[ok] - de[ok]) / np.sqrt(var[ok] / K)
        assert np.abs(z).max() < 5.5, t
        assert 0.6 < np.mean(z ** 2) < 1.5, t
        np.testing.assert_allclose(mean[~ok], de[~ok], atol=1e-9)
