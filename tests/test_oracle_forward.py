"""Pins the oracle's forward: a library routine and closed forms."""
import math

import numpy as np
import pytest
import torch

from oracle import attn_fwd


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (8, 2)])
def test_fwd_matches_torch_sdpa_fp64(causal, hq, hkv):
    B, N, d = 2, 48, 16
    q, k, v = _rand((B, hq, N, d), 1), _rand((B, hkv, N, d), 2), _rand((B, hkv, N, d), 3)
    scale = 1.0 / math.sqrt(d)
    o, lse = attn_fwd(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=(hq != hkv)).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    # logsumexp of the masked scores, from torch's own reduction
    rep = hq // hkv
    s = scale * (tq @ tk.repeat_interleave(rep, 1).transpose(-1, -2))
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_fwd_closed_form_zero_queries(causal):
    # Q = 0: every unmasked score is 0, so LSE_i = log(#keys seen) and O_i is
    # the plain mean of the visible value rows.
    B, H, N, d = 1, 2, 40, 8
    q = np.zeros((B, H, N, d))
    k = _rand((B, H, N, d), 4)
    v = _rand((B, H, N, d), 5)
    o, lse = attn_fwd(q, k, v, 0.3, causal)
    n_seen = np.arange(1, N + 1) if causal else np.full(N, N)
    np.testing.assert_allclose(lse[0, 0], np.log(n_seen), rtol=0, atol=1e-14)
    if causal:
        mean = np.cumsum(v, axis=2) / n_seen[None, None, :, None]
    else:
        mean = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    np.testing.assert_allclose(o, mean, rtol=1e-13, atol=1e-13)


def test_fwd_first_causal_row_copies_first_value():
    B, H, N, d = 1, 1, 16, 4
    q, k, v = _rand((B, H, N, d), 6), _rand((B, H, N, d), 7), _rand((B, H, N, d), 8)
    o, lse = attn_fwd(q, k, v, 0.5, True)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0])
    assert lse[0, 0, 0] == pytest.approx(0.5 * float(q[0, 0, 0] @ k[0, 0, 0]), abs=1e-15)
