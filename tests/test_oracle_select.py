"""Pins the oracle's selection: masses, tau, draw, weights, compaction."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.optimize import brentq

from oracle import (block_masses, block_uniform, budget_discarded, halving_tree_sum,
                    select, solve_tau)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _val(expr):
    # fixtures write exact binary fractions as tiny float expressions
    return float(eval(expr, {"__builtins__": {}}, {}))


# ---------------------------------------------------------------- masses ----
def test_tree_golden_cases():
    for case in _golden("halving_tree_cases.json")["tree_cases"]:
        x = np.array([_val(e) for e in case["x"]])
        assert halving_tree_sum(x) == _val(case["tree"]), case["why"]
        seq = 0.0
        for e in x:
            seq += e
        assert seq == _val(case["sequential"]), case["why"]


def test_mass_golden_cases():
    for case in _golden("halving_tree_cases.json")["mass_cases"]:
        blk = np.array([[_val(e) for e in row] for row in case["dout_block"]])
        dout = blk.reshape(1, 1, case["block"], case["d"])
        assert block_masses(dout, case["block"])[0, 0, 0] == _val(case["mass"]), case["why"]


@pytest.mark.parametrize("block,d", [(64, 64), (128, 128), (64, 128)])
def test_masses_close_to_exact_sum(block, d):
    rng = np.random.Generator(np.random.PCG64(5))
    N = 4 * block
    dout = (rng.standard_normal((2, 3, N, d)) * np.exp(2 * rng.standard_normal((2, 3, N, 1))))
    dout = dout.astype(np.float32).astype(np.float64)
    m = block_masses(dout, block)
    assert m.shape == (2, 3, 4)
    L = block * d
    for idx in np.ndindex(m.shape):
        b, h, i = idx
        x = dout[b, h, i * block:(i + 1) * block].ravel() ** 2
        exact = math.fsum(x)
        # a pairwise tree of depth log2(L) errs by at most log2(L) * eps * sum
        assert abs(m[idx] - exact) <= math.log2(L) * 2**-53 * exact * 1.01
    # each block is its own rows only: a wrong reshape mixes rows across blocks
    np.testing.assert_allclose(m.sum(axis=2), (dout ** 2).sum(axis=(2, 3)), rtol=1e-12)


def test_masses_constant_block_exact():
    dout = np.full((1, 2, 128, 64), 0.75)
    dout[0, 1] = 0.0
    m = block_masses(dout, 64)
    assert np.all(m[0, 0] == 64 * 64 * 0.5625)
    assert np.all(m[0, 1] == 0.0)


# ------------------------------------------------------------------ tau -----
def test_tau_golden_cases():
    for case in _golden("tau_cases.json")["cases"]:
        m = np.array(case["m"])
        tau = solve_tau(m, case["delta"])
        exact = Fraction(case["tau_num"], case["tau_den"])
        assert abs(Fraction(tau) - exact) <= abs(exact) * Fraction(2) ** -52, case["why"]
        p = np.where(m > 0, np.minimum(1.0, m / tau), 0.0)
        want = np.array([float(Fraction(s)) for s in case["p"]])
        np.testing.assert_allclose(p, want, rtol=1e-15, atol=0, err_msg=case["why"])


def test_tau_delta_zero_keeps_every_positive_block():
    m = np.array([3.0, 0.0, 1e-30, 7.5, 2.0])
    tau = solve_tau(m, 0.0)
    assert tau == 1e-30
    assert np.all(np.minimum(1.0, m[m > 0] / tau) == 1.0)


@pytest.mark.parametrize("delta", [0.05, 0.1, 0.3, 0.6, 0.95])
def test_tau_all_equal_closed_form(delta):
    m = np.full(17, 2.5)
    tau = solve_tau(m, delta)
    assert tau == pytest.approx(2.5 / (1 - delta), rel=1e-14)


@pytest.mark.parametrize("delta", [0.01, 0.1, 0.5, 0.9])
def test_tau_single_positive_block(delta):
    m = np.array([0.0, 0.0, 4.25, 0.0])
    tau = solve_tau(m, delta)
    assert min(1.0, 4.25 / tau) == pytest.approx(1 - delta, rel=1e-14)


def test_tau_degenerate_heads():
    assert solve_tau(np.zeros(8), 0.1) == math.inf
    assert math.isnan(solve_tau(np.array([1.0, np.nan, 2.0]), 0.1))
    assert math.isnan(solve_tau(np.array([1.0, np.inf, 2.0]), 0.0))


def _heavy(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.exp(3 * rng.standard_normal(n)) * (rng.random(n) > 0.1)


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("delta", [0.02, 0.1, 0.2, 0.5])
def test_tau_is_root_of_budget_by_bisection(seed, delta):
    m = _heavy(64 + 37 * seed, seed)
    S = math.fsum(m)
    tau = solve_tau(m, delta)
    f = lambda t: budget_discarded(m, t) - delta * S  # noqa: E731
    lo, hi = m[m > 0].min() * 0.5, m.max() * 1e6 / (1 - delta)
    ref = brentq(f, lo, hi, xtol=1e-300, rtol=1e-15, maxiter=500)
    assert tau == pytest.approx(ref, rel=1e-12)
    assert budget_discarded(m, tau) == pytest.approx(delta * S, rel=1e-11)


@pytest.mark.parametrize("seed", range(6))
def test_tau_brute_force_interval_enumeration(seed):
    # Independent route: for every k compute the exact rational candidate
    # Q_k / (A_k - delta S) with Fractions and keep the one that lies in its
    # own interval [m_(k), m_(k+1)].
    m = _heavy(9 + seed, 100 + seed)
    delta = [0.05, 0.15, 0.3, 0.45, 0.7, 0.9][seed]
    pos = sorted(Fraction(x) for x in m if x > 0)
    S = sum(pos)
    dS = Fraction(delta) * S
    found = []
    for k in range(1, len(pos) + 1):
        A, Q = sum(pos[:k]), sum(x * x for x in pos[:k])
        if A - dS <= 0:
            continue
        t = Q / (A - dS)
        hi = pos[k] if k < len(pos) else None
        if pos[k - 1] <= t and (hi is None or t <= hi):
            found.append(t)
    assert len(found) >= 1
    assert all(abs(t - found[0]) <= found[0] * Fraction(1, 10**12) for t in found)
    assert solve_tau(m, delta) == pytest.approx(float(found[0]), rel=1e-12)


def test_tau_monotone_in_delta():
    m = _heavy(200, 3)
    taus = [solve_tau(m, dl) for dl in (0.0, 0.01, 0.05, 0.1, 0.2, 0.5, 0.9)]
    assert all(a <= b for a, b in zip(taus, taus[1:]))


# ------------------------------------------------------------- draw ---------
def test_select_fields_and_weights():
    rng = np.random.Generator(np.random.PCG64(9))
    mass = np.exp(2 * rng.standard_normal((2, 3, 40)))
    mass[0, 1, 5] = 0.0
    sel = select(mass, 0.2, seed=11)
    for b in range(2):
        for h in range(3):
            tau = solve_tau(mass[b, h], 0.2)
            assert sel["tau"][b, h] == tau
            for i in range(40):
                p = 0.0 if mass[b, h, i] == 0 else min(1.0, mass[b, h, i] / tau)
                u = block_uniform(11, b, h, i)
                assert sel["p"][b, h, i] == p and sel["u"][b, h, i] == u
                assert sel["keep"][b, h, i] == (u < p)
                assert sel["w"][b, h, i] == (np.float32(1.0 / p) if u < p else 0.0)
            idx = np.nonzero(sel["keep"][b, h])[0]
            n = sel["kept_count"][b, h]
            assert n == idx.size
            assert np.array_equal(sel["kept_idx"][b, h, :n], idx)
            assert np.all(sel["kept_idx"][b, h, n:] == -1)
    assert not sel["keep"][0, 1, 5]


def test_select_keep_frequency_is_binomial():
    rng = np.random.Generator(np.random.PCG64(12))
    mass = np.exp(1.5 * rng.standard_normal((1, 2, 48)))
    K = 400
    counts = np.zeros((1, 2, 48))
    for s in range(K):
        sel = select(mass, 0.3, seed=1000 + s)
        counts += sel["keep"]
    p = sel["p"]
    assert np.any((p > 0.05) & (p < 0.95))
    var = K * p * (1 - p)
    z = (counts - K * p) / np.sqrt(np.where(var > 0, var, 1.0))
    assert np.all(counts[p == 1.0] == K)
    assert np.abs(z).max() < 4.5
    assert 0.5 < np.mean(z[(p > 0) & (p < 1)] ** 2) < 1.6


def test_select_nesting_across_budgets():
    rng = np.random.Generator(np.random.PCG64(13))
    mass = np.exp(2 * rng.standard_normal((2, 4, 64)))
    prev = None
    for dl in (0.0, 0.05, 0.1, 0.2, 0.4, 0.8):
        keep = select(mass, dl, seed=3)["keep"]
        if prev is not None:
            assert np.all(prev | ~keep)        # kept(larger delta) within kept(smaller)
        prev = keep


def test_select_delta_zero_keeps_all_nonzero():
    mass = np.array([[[1.0, 0.0, 5.0, 1e-9]]])
    sel = select(mass, 0.0, seed=0)
    assert list(sel["keep"][0, 0]) == [True, False, True, True]
    assert np.all(sel["w"][0, 0][sel["keep"][0, 0]] == 1.0)


def test_select_nonfinite_head_falls_back_to_dense():
    mass = np.array([[[1.0, np.nan, 0.0], [1.0, 2.0, 3.0]]])
    sel = select(mass, 0.5, seed=1)
    assert math.isnan(sel["tau"][0, 0])
    assert np.all(sel["keep"][0, 0]) and np.all(sel["w"][0, 0] == 1.0)
    assert sel["kept_count"][0, 0] == 3


def test_select_rejects_bad_delta():
    for dl in (-0.1, 1.0, 1.5, math.nan):
        with pytest.raises(ValueError):
            select(np.ones((1, 1, 4)), dl, seed=0)
