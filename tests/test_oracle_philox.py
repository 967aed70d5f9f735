"""Pins the oracle's Philox4x64-10 against numpy's independent implementation.

numpy.random.Philox is the 4x64 variant with 10 rounds.  It advances its
counter by one *before* producing the first block, so the block for counter c
is the first output of a generator started at c - 1 (established by running
numpy, not by reading its source).
"""
import numpy as np
import pytest

from oracle import block_uniform, philox4x64_10

M64 = (1 << 64) - 1


def _numpy_block(counter, key):
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    c = (c - 1) % (1 << 256)
    words = np.array([(c >> (64 * i)) & M64 for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=words, key=np.array(key, dtype=np.uint64))
    return [int(x) for x in bg.random_raw(4)]


def test_philox_matches_numpy_many_counters():
    rng = np.random.Generator(np.random.PCG64(1234))
    n = 10000
    ctrs = rng.integers(0, 2**64, size=(n, 4), dtype=np.uint64, endpoint=False)
    keys = rng.integers(0, 2**64, size=(n, 2), dtype=np.uint64, endpoint=False)
    # structured counters of the form used for block draws, plus carries
    ctrs[:64] = [[i, h, b, 0] for i, h, b in zip(range(64), range(64)[::-1], [0, 1] * 32)]
    ctrs[64] = [M64, 7, 0, 0]
    for j in range(n):
        c = [int(x) for x in ctrs[j]]
        kk = [int(x) for x in keys[j]]
        assert philox4x64_10(c, kk) == _numpy_block(c, kk), j


@pytest.mark.parametrize("seed", [0, 1, 2**63 + 5])
def test_block_uniform_is_top_53_bits(seed):
    for (b, h, i) in [(0, 0, 0), (0, 3, 17), (2, 15, 255), (0, 31, 511)]:
        x0 = _numpy_block((i, h, b, 0), (seed, 0))[0]
        u = block_uniform(seed, b, h, i)
        assert u == (x0 >> 11) / 2.0**53
        assert 0.0 <= u < 1.0


def test_uniform_looks_uniform():
    u = np.array([block_uniform(7, 0, h, i) for h in range(8) for i in range(512)])
    # mean and a coarse histogram: a wrong shift or mask is visibly non-uniform
    assert abs(u.mean() - 0.5) < 0.02
    hist, _ = np.histogram(u, bins=16, range=(0, 1))
    assert hist.min() > 180 and hist.max() < 340
