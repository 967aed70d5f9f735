"""The pins are sharp: plausible mistakes planted in the oracle (on the CPU,
through monkeypatching) make the corresponding pin fail."""
import math

import numpy as np
import pytest
import torch

import oracle.lazyflash_oracle as orc


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def _autograd_gap(causal=True):
    B, Hq, Hkv, N, d = 1, 4, 2, 32, 8
    q, k, v = _rand((B, Hq, N, d), 1), _rand((B, Hkv, N, d), 2), _rand((B, Hkv, N, d), 3)
    dout = _rand((B, Hq, N, d), 4)
    dq, dk, dv = orc.attn_bwd_dense(q, k, v, dout, 0.35, causal)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, scale=0.35, enable_gqa=True).backward(torch.from_numpy(dout))
    return max(np.abs(a - t.grad.numpy()).max() for a, t in ((dq, tq), (dk, tk), (dv, tv)))


def test_clean_oracle_passes_autograd_pin():
    assert _autograd_gap() < 1e-10


def test_dropped_row_term_is_caught(monkeypatch):
    good = orc._row_grads

    def bad(qh, kg, vg, doh, o_rows, lse_rows, scale, causal, rows):
        return good(qh, kg, vg, doh, np.zeros_like(o_rows), lse_rows, scale, causal, rows)
    monkeypatch.setattr(orc, "_row_grads", bad)
    assert _autograd_gap() > 1e-3


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    def bad_fwd(q, k, v, scale, causal):
        B, Hq, N, _ = q.shape
        Hkv = k.shape[1]
        o, lse = np.empty_like(q), np.empty((B, Hq, N))
        for b in range(B):
            for h in range(Hq):
                o[b, h], lse[b, h] = orc.attn_fwd_rows(q[b, h], k[b, h % Hkv], v[b, h % Hkv],
                                                       scale, causal, np.arange(N))
        return o, lse
    q, k, v = _rand((1, 4, 16, 4), 5), _rand((1, 2, 16, 4), 6), _rand((1, 2, 16, 4), 7)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), is_causal=True, scale=0.5, enable_gqa=True)
    assert np.abs(bad_fwd(q, k, v, 0.5, True)[0] - ref.numpy()).max() > 1e-3
    assert np.abs(orc.attn_fwd(q, k, v, 0.5, True)[0] - ref.numpy()).max() < 1e-12


def test_sequential_mass_sum_is_caught():
    dout = np.array([3.0, 2.0**-25, 0.0, 2.0**-25]).reshape(1, 1, 2, 2)
    seq = 0.0
    for x in dout.ravel() ** 2:
        seq += x
    assert orc.block_masses(dout, 2)[0, 0, 0] == 9.0 + 2.0**-49
    assert seq != 9.0 + 2.0**-49


def test_philox_round_mistakes_are_caught():
    from tests.test_oracle_philox import _numpy_block
    ctr, key = (3, 1, 4, 1), (5, 9)
    want = _numpy_block(ctr, key)
    assert orc.philox4x64_10(ctr, key) == want

    def nine_rounds(counter, k):
        # the same structure with one round fewer
        m0, m1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
        c, k0, k1 = list(counter), k[0], k[1]
        for r in range(9):
            if r:
                k0, k1 = (k0 + 0x9E3779B97F4A7C15) & orc.MASK64, (k1 + 0xBB67AE8584CAA73B) & orc.MASK64
            p0, p1 = m0 * c[0], m1 * c[2]
            c = [((p1 >> 64) ^ c[1] ^ k0) & orc.MASK64, p1 & orc.MASK64,
                 ((p0 >> 64) ^ c[3] ^ k1) & orc.MASK64, p0 & orc.MASK64]
        return c
    assert nine_rounds(ctr, key) != want


def test_smallest_tau_reading_is_caught():
    # "the smallest tau within budget" taken literally keeps everything; the
    # closed form p = 1 - delta for equal masses rejects it.
    m = np.full(10, 3.0)
    literal_tau = m.min()
    assert min(1.0, 3.0 / literal_tau) != pytest.approx(0.7)
    assert min(1.0, 3.0 / orc.solve_tau(m, 0.3)) == pytest.approx(0.7, rel=1e-14)

