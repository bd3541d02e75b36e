"""Pins of the oracle's production (asynchronous) scheduler step.

DSpark page, section 7: the current candidates are still ranked by the
latest confidences, while the number verified (a dynamic top-K) comes from
the scheduler's output two steps earlier, so the admission capacity does not
depend on the current tokens.  Pinned by
  - exhaustive enumeration: for R <= 4, gamma <= 4 and every K, the top-K
    selection maximises the expected accepted mass sum_r sum_{j<=l_r} a_rj
    over all allocations with sum_r l_r = K (the maximum is the value to
    1e-12; l is equal when the best allocation is unique);
  - the history ring: no history -> exactly the synchronous scheduler; the
    ring advances {h0, h1} -> {h1, K*}; K is capped at R*gamma;
  - nesting: l(K) <= l(K+1) elementwise and sum l(K) = min(K, R*gamma).
"""
import itertools

import numpy as np
import pytest

import oracle


def _best_mass(c, K):
    """Largest sum of a over allocations with sum(l) = K, and the argmax
    allocations (all of them), by direct enumeration."""
    a = np.cumprod(c.astype(np.float64), axis=1)
    R, g = c.shape
    csum = np.concatenate([np.zeros((R, 1)), np.cumsum(a, axis=1)], axis=1)
    best, args = -np.inf, []
    for ell in itertools.product(range(g + 1), repeat=R):
        if sum(ell) != K:
            continue
        m = sum(csum[r, ell[r]] for r in range(R))
        if m > best * (1 + 1e-13) + 1e-300:
            best, args = m, [ell]
        elif abs(m - best) <= 1e-13 * abs(best):
            args.append(ell)
    return best, [np.array(x) for x in args]


def test_top_k_maximises_accepted_mass_by_enumeration():
    rng = np.random.default_rng(11)
    checked = unique = 0
    for trial in range(400):
        R = int(rng.integers(1, 5))
        g = int(rng.integers(1, 5))
        c = (1 / (1 + np.exp(-rng.normal(1.5, 1.0, (R, g))))).astype(np.float32)
        if trial % 5 == 0:
            c[rng.random((R, g)) < 0.3] = 1.0      # ties
        sps = np.ones(R * (g + 1), np.float32)
        for K in range(R * g + 1):
            out = oracle.schedule_async(c, sps, [K, -1])
            assert out["K_used"] == K
            ell = out["ell"]
            assert ell.sum() == K and (ell >= 0).all() and (ell <= g).all()
            a = np.cumprod(c.astype(np.float64), axis=1)
            mass = sum(a[r, :ell[r]].sum() for r in range(R))
            best, args = _best_mass(c, K)
            assert mass == pytest.approx(best, rel=1e-12, abs=1e-300)
            if len(args) == 1:
                np.testing.assert_array_equal(ell, args[0])
                unique += 1
            checked += 1
    assert checked > 2000 and unique > 1000


def test_no_history_is_the_synchronous_scheduler():
    rng = np.random.default_rng(3)
    for _ in range(200):
        R = int(rng.integers(1, 7))
        g = int(rng.integers(1, 7))
        c = (1 / (1 + np.exp(-rng.normal(1.5, 1.0, (R, g))))).astype(np.float32)
        sps = rng.uniform(0.2, 1.0, R * (g + 1)).astype(np.float32)
        sync = oracle.schedule(c, sps)
        out = oracle.schedule_async(c, sps, [-1, -1])
        assert out["K_used"] == sync["K_star"] == out["K_star"]
        np.testing.assert_array_equal(out["ell"], sync["ell"])
        np.testing.assert_array_equal(out["a"], sync["a"])
        assert out["theta_star"] == sync["theta_star"]
        np.testing.assert_array_equal(out["K_hist"], [-1, sync["K_star"]])


def test_history_ring_and_two_step_lag():
    """Over a sequence of steps, the K applied at step t is the optimum the
    scheduler found at step t-2 (the first two steps use their own)."""
    rng = np.random.default_rng(9)
    R, g = 5, 6
    sps = (1000.0 / (20 + 0.25 * np.ceil(np.arange(1, R * (g + 1) + 1) / 64)
                     + 0.01 * np.arange(1, R * (g + 1) + 1))).astype(np.float32)
    hist = [-1, -1]
    stars = []
    for t in range(12):
        c = (1 / (1 + np.exp(-rng.normal(1.0, 1.5, (R, g))))).astype(np.float32)
        out = oracle.schedule_async(c, sps, hist)
        stars.append(out["K_star"])
        want = stars[t - 2] if t >= 2 else out["K_star"]
        assert out["K_used"] == want
        assert out["ell"].sum() == want
        hist = list(out["K_hist"])
        assert hist == ([stars[t - 1], stars[t]] if t >= 1 else [-1, stars[0]])


def test_cap_and_nesting():
    rng = np.random.default_rng(4)
    c = (1 / (1 + np.exp(-rng.normal(1.5, 1.0, (6, 5))))).astype(np.float32)
    sps = np.ones(36, np.float32)
    prev = np.zeros(6, np.int32)
    for K in range(0, 31):
        ell = oracle.schedule_async(c, sps, [K, 0])["ell"]
        assert (ell >= prev).all() and ell.sum() == K
        prev = ell
    out = oracle.schedule_async(c, sps, [1000, 0])
    assert out["K_used"] == 30 and (out["ell"] == 5).all()
    out = oracle.schedule_async(c, sps, [0, 0])
    assert out["K_used"] == 0 and (out["ell"] == 0).all()
