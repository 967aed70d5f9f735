"""Pins the oracle's other selection rules (fixed fraction, top-k), the rules
the budget is compared with at equal backward time (LazyFlash entry on gyom.fr,
section "Le choix des blocs pèse plus que la quantité sautée")."""
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.optimize import brentq

import oracle.lazyflash_oracle as orc
from oracle import (RULE_BUDGET, RULE_FRACTION, RULE_TOPK, expected_kept, select, select_rule,
                    solve_tau_fraction, topk_keep)


def _heavy(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    m = np.exp(2.0 * rng.standard_normal(n)) * rng.chisquare(8, n)
    m[rng.random(n) < 0.1] = 0.0
    return m


# ------------------------------------------------------------ fraction ------
@pytest.mark.parametrize("f", [0.05, 0.3, 0.5, 0.99])
def test_fraction_all_equal_closed_form(f):
    # n equal masses mu: g(tau) = n mu / tau = f n  =>  tau = mu / f, p = f
    mu = 3.25
    tau = solve_tau_fraction(np.full(40, mu), f)
    assert tau == pytest.approx(mu / f, rel=1e-15)
    assert min(1.0, mu / tau) == pytest.approx(f, rel=1e-15)


def test_fraction_one_keeps_every_positive_block():
    m = np.array([0.0, 2.0, 5.0, 1e-12])
    assert solve_tau_fraction(m, 1.0) == 1e-12
    sel = select_rule(m.reshape(1, 1, 4), RULE_FRACTION, 1.0, seed=4)
    assert list(sel["keep"][0, 0]) == [False, True, True, True]
    assert np.all(sel["w"][0, 0][1:] == 1.0)


def test_fraction_degenerate_heads():
    assert solve_tau_fraction(np.zeros(8), 0.3) == math.inf
    assert math.isnan(solve_tau_fraction(np.array([1.0, math.inf]), 0.3))
    sel = select_rule(np.array([[[1.0, math.nan, 2.0], [0.0, 0.0, 0.0]]]), RULE_FRACTION, 0.5, 0)
    assert math.isnan(sel["tau"][0, 0]) and np.all(sel["w"][0, 0] == 1.0)
    assert sel["kept_count"][0, 1] == 0 and sel["tau"][0, 1] == math.inf


@pytest.mark.parametrize("seed,f", [(0, 0.1), (1, 0.25), (2, 0.5), (3, 0.8)])
def test_fraction_is_root_of_expected_count_by_bisection(seed, f):
    m = _heavy(80 + 23 * seed, 40 + seed)
    n = int((m > 0).sum())
    tau = solve_tau_fraction(m, f)
    ref = brentq(lambda t: expected_kept(m, t) - f * n, m[m > 0].min() * 0.5,
                 m.sum() / (f * n) * 2, xtol=1e-300, rtol=1e-15, maxiter=500)
    assert tau == pytest.approx(ref, rel=1e-12)
    assert expected_kept(m, tau) == pytest.approx(f * n, rel=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_fraction_brute_force_over_saturated_sets(seed):
    # Independent route in exact rationals: for every number j of saturated
    # (largest) blocks, tau_j = (sum of the others) / (c - j); keep the one
    # that separates the saturated masses from the rest.
    m = _heavy(10 + seed, 200 + seed)
    f = [0.07, 0.2, 0.35, 0.5, 0.65, 0.9][seed]
    pos = sorted(Fraction(x) for x in m if x > 0)
    n = len(pos)
    c = Fraction(f) * n
    found = []
    for j in range(n):
        if c - j <= 0:
            continue
        rest, sat = pos[:n - j], pos[n - j:]
        t = sum(rest) / (c - j)
        if rest[-1] <= t and (not sat or t <= sat[0]):
            found.append(t)
    assert found
    assert solve_tau_fraction(m, f) == pytest.approx(float(found[0]), rel=1e-12)


def test_fraction_monotone_and_nested():
    rng = np.random.Generator(np.random.PCG64(21))
    mass = np.exp(2 * rng.standard_normal((2, 3, 64)))
    prev = None
    taus = []
    for f in (0.05, 0.1, 0.2, 0.4, 0.8, 1.0):
        sel = select_rule(mass, RULE_FRACTION, f, seed=5)
        taus.append(sel["tau"])
        if prev is not None:
            assert np.all(~prev | sel["keep"])     # kept(f small) within kept(f large)
        prev = sel["keep"]
    assert all(np.all(a >= b) for a, b in zip(taus, taus[1:]))


def test_fraction_draw_is_unbiased():
    rng = np.random.Generator(np.random.PCG64(22))
    mass = np.exp(1.5 * rng.standard_normal((1, 2, 40)))
    K = 400
    counts = np.zeros((1, 2, 40))
    wsum = np.zeros((1, 2, 40))
    for s in range(K):
        sel = select_rule(mass, RULE_FRACTION, 0.3, seed=3000 + s)
        counts += sel["keep"]
        wsum += sel["w"]
    p = sel["p"]
    assert p.sum(axis=-1) == pytest.approx(0.3 * 40, rel=1e-12)
    var = K * p * (1 - p)
    z = (counts - K * p) / np.sqrt(np.where(var > 0, var, 1.0))
    assert np.abs(z).max() < 4.5
    # E[keep * w] = 1 for every positive block (the estimator is unbiased);
    # keep * w is 1/p with probability p, so its variance is (1 - p) / p
    sd = np.sqrt((1 - p) / np.where(p > 0, p, 1.0) / K)
    zw = (wsum / K - 1.0) / np.where(sd > 0, sd, 1.0)
    assert np.all(wsum[p == 1.0] == K)
    assert np.abs(zw).max() < 4.5
    assert 0.5 < np.mean(zw[(p > 0) & (p < 1)] ** 2) < 1.6


def test_fraction_uses_the_budget_draw():
    # same uniforms, same p -> w rule as the budget: with f set to the kept
    # expectation the budget's tau produces, the two rules agree exactly
    rng = np.random.Generator(np.random.PCG64(23))
    mass = np.exp(2 * rng.standard_normal((1, 1, 50)))
    b = select(mass, 0.2, seed=9)
    f = float(b["p"].sum()) / 50
    r = select_rule(mass, RULE_FRACTION, f, seed=9)
    assert r["tau"][0, 0] == pytest.approx(b["tau"][0, 0], rel=1e-9)
    assert np.array_equal(r["u"], b["u"])


# ----------------------------------------------------------------- top-k ----
@pytest.mark.parametrize("seed", range(5))
def test_topk_matches_a_full_sort(seed):
    rng = np.random.Generator(np.random.PCG64(300 + seed))
    m = np.round(np.exp(rng.standard_normal(57)), 1)   # rounding makes ties
    m[rng.random(57) < 0.15] = 0.0
    f = [0.01, 0.1, 0.33, 0.5, 1.0][seed]
    pos = np.nonzero(m > 0)[0]
    k = math.ceil(f * pos.size)
    order = np.lexsort((pos, -m[pos]))                  # by mass desc, index asc
    want = np.zeros(57, dtype=bool)
    want[pos[order[:k]]] = True
    assert np.array_equal(topk_keep(m, f), want)
    assert topk_keep(m, f).sum() == k


def test_topk_ties_go_to_lower_indices_and_zeros_never():
    m = np.array([2.0, 0.0, 5.0, 2.0, 2.0, 0.0])
    assert list(topk_keep(m, 0.5)) == [True, False, True, False, False, False]
    assert list(topk_keep(m, 0.75)) == [True, False, True, True, False, False]
    assert list(topk_keep(m, 1.0)) == [True, False, True, True, True, False]


def test_topk_select_fields_are_deterministic():
    rng = np.random.Generator(np.random.PCG64(31))
    mass = np.exp(rng.standard_normal((2, 2, 30)))
    a = select_rule(mass, RULE_TOPK, 0.2, seed=1)
    b = select_rule(mass, RULE_TOPK, 0.2, seed=999)
    for key in ("keep", "w", "kept_idx", "kept_count", "tau"):
        assert np.array_equal(a[key], b[key])
    assert np.all(a["kept_count"] == 6)
    assert np.all(a["w"][a["keep"]] == 1.0) and np.all(a["w"][~a["keep"]] == 0.0)
    kept_min = np.where(a["keep"], mass, np.inf).min(axis=-1)
    assert np.array_equal(a["tau"], kept_min)


# --------------------------------------------------------------- common -----
def test_budget_rule_is_select():
    rng = np.random.Generator(np.random.PCG64(41))
    mass = np.exp(rng.standard_normal((1, 3, 20)))
    a, b = select_rule(mass, RULE_BUDGET, 0.15, seed=7), select(mass, 0.15, seed=7)
    for key in a:
        assert np.array_equal(a[key], b[key], equal_nan=True)


def test_rules_reject_bad_parameters():
    for f in (0.0, -0.1, 1.5, math.nan):
        for rule in (RULE_FRACTION, RULE_TOPK):
            with pytest.raises(ValueError):
                select_rule(np.ones((1, 1, 4)), rule, f, seed=0)
    with pytest.raises(ValueError):
        select_rule(np.ones((1, 1, 4)), 7, 0.5, seed=0)


# --------------------------------------------------- the pins are sharp -----
def test_off_by_one_saturated_count_is_caught(monkeypatch):
    # a plausible mistake: counting the interval's own block as saturated
    def bad(m, f):
        m = np.asarray(m, dtype=np.float64)
        pos = np.sort(m[m > 0.0])
        n = pos.shape[0]
        c = f * float(n)
        a = 0.0
        for k in range(n):
            a = a + float(pos[k])
            hi = float(pos[k + 1]) if k + 1 < n else math.inf
            sat = float(n - k)
            if sat + a / hi <= c:
                return a / (c - sat) if c > sat else math.inf
        return math.inf
    m = _heavy(60, 77)
    n = int((m > 0).sum())
    assert abs(expected_kept(m, bad(m, 0.3)) - 0.3 * n) > 0.5
    assert expected_kept(m, solve_tau_fraction(m, 0.3)) == pytest.approx(0.3 * n, rel=1e-12)


def test_topk_tie_order_mistake_is_caught():
    m = np.array([1.0, 3.0, 3.0, 3.0])
    bad = np.zeros(4, dtype=bool)
    bad[np.argsort(-m, kind="stable")[::-1][:2]] = True   # wrong end of the tie
    assert not np.array_equal(bad, topk_keep(m, 0.5))
    assert list(topk_keep(m, 0.5)) == [False, True, True, False]
