"""Pins the oracle where N is not a multiple of the block (a partial last query
block): the mass of the partial block sums only its rows, and the sparse
backward over its rows is the dense gradient's."""
import math

import numpy as np
import pytest

from oracle import attn_bwd_dense, attn_bwd_sparse, block_masses, halving_tree_sum


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


@pytest.mark.parametrize("N,block,d", [(13, 4, 2), (200, 64, 8), (1000, 128, 4)])
def test_partial_block_mass_sums_its_rows(N, block, d):
    x = np.round(_rand((1, 2, N, d), N), 3)
    m = block_masses(x, block)
    nqb = -(-N // block)
    assert m.shape == (1, 2, nqb)
    for h in range(2):
        for i in range(nqb):
            rows = x[0, h, i * block:min((i + 1) * block, N)]
            assert m[0, h, i] == pytest.approx(math.fsum((rows.ravel() ** 2).tolist()), rel=1e-14)
    # the tree over the zero-padded block, written out independently
    last = np.zeros((block, d))
    last[:N - (nqb - 1) * block] = x[0, 1, (nqb - 1) * block:]
    assert m[0, 1, -1] == halving_tree_sum((last * last).ravel())


@pytest.mark.parametrize("causal", [True, False])
def test_sparse_all_kept_equals_dense_on_ragged_length(causal):
    B, Hq, Hkv, N, d, block = 1, 4, 2, 23, 4, 8   # blocks of 8, 8, 7 rows
    q, k, v = _rand((B, Hq, N, d), 1), _rand((B, Hkv, N, d), 2), _rand((B, Hkv, N, d), 3)
    dout = _rand((B, Hq, N, d), 4)
    nqb = 3
    keep = np.ones((B, Hq, nqb), dtype=bool)
    w = np.ones((B, Hq, nqb))
    sp = attn_bwd_sparse(q, k, v, dout, block, keep, w, 0.4, causal)
    de = attn_bwd_dense(q, k, v, dout, 0.4, causal)
    for a, b in zip(sp, de):
        assert np.abs(a - b).max() < 1e-12


def test_sparse_partial_block_weight_scales_only_its_rows():
    B, Hq, Hkv, N, d, block = 1, 2, 1, 20, 4, 8   # last block: rows 16..19
    q, k, v = _rand((B, Hq, N, d), 5), _rand((B, Hkv, N, d), 6), _rand((B, Hkv, N, d), 7)
    dout = _rand((B, Hq, N, d), 8)
    keep = np.zeros((B, Hq, 3), dtype=bool)
    keep[0, 1, 2] = True
    w = np.zeros((B, Hq, 3))
    w[0, 1, 2] = 2.5
    dq, dk, dv = attn_bwd_sparse(q, k, v, dout, block, keep, w, 0.5, True)
    dO = np.zeros_like(dout)
    dO[0, 1, 16:] = 2.5 * dout[0, 1, 16:]
    rq, rk, rv = attn_bwd_dense(q, k, v, dO, 0.5, True)
    assert np.abs(dq - rq).max() < 1e-12
    assert np.abs(dk - rk).max() < 1e-12 and np.abs(dv - rv).max() < 1e-12
