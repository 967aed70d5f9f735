"""Reporting arithmetic of the benchmark: Amdahl whole-job gains against the
worked example printed on the FlashAttention course page, FLOP counts against
brute-force pair counting."""
import json
import os

import numpy as np
import pytest

from block_sparse_backward_amd import metrics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "amdahl_voce.json")


def test_amdahl_matches_printed_worked_example():
    data = json.load(open(GOLDEN))
    for c in data["cases"]:
        new, gain, cap = metrics.amdahl(c["total"], c["part"], c["speedup"])
        assert new == pytest.approx(c["new"], abs=0.05)
        assert gain == pytest.approx(c["gain"], abs=0.005)
        assert cap == pytest.approx(c["cap"], abs=1e-9)


def test_lazyflash_ratios_are_consistent():
    # the LazyFlash entry: 1429.8 -> 507.4 ms is the 2.82x quoted for Qwen3-8B
    assert 1429.8 / 507.4 == pytest.approx(2.82, abs=0.005)


@pytest.mark.parametrize("causal", [True, False])
def test_flop_counts_by_brute_force(causal):
    N, d, block = 96, 8, 16
    q = np.arange(N)[:, None]
    k = np.arange(N)[None, :]
    vis = (k <= q) if causal else np.ones((N, N), bool)
    assert metrics.pairs_dense(N, causal) == vis.sum()
    assert metrics.bwd_flops_dense(2, 3, N, d, causal) == 10 * d * 6 * vis.sum()
    keep = np.zeros((2, 3, N // block), bool)
    keep[0, 1, [0, 3, 5]] = True
    keep[1, 2, 2] = True
    want = 0
    for b, h, i in zip(*np.nonzero(keep)):
        want += vis[i * block:(i + 1) * block].sum()
    assert metrics.bwd_flops_kept(keep, N, d, block, causal) == 10 * d * want
    assert metrics.bwd_flops_kept(np.ones_like(keep), N, d, block, causal) == \
        metrics.bwd_flops_dense(2, 3, N, d, causal)


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU; asked for more it stops before any GPU
    work with a message and a nonzero status."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=root)
    assert r.returncode != 0
    assert "one GPU" in r.stderr + r.stdout
    assert not r.stdout.strip().startswith("{")  # no JSON line
