"""Pins of the oracle's hardware-aware prefix scheduler.

DSpark page, section 6: a_{r,j} = prod_{i<=j} c_{r,i}; B = sum_r (1 + l_r);
tau = sum_r (1 + sum_{j<=l_r} a_{r,j}); maximise Theta = tau * SPS(B).
Pinned by exhaustive enumeration of all (gamma+1)^R allocations for
R <= 4, gamma <= 4 (Theta* equal to 1e-12 relative; l equal when the optimum
is unique), and by the special cases constant SPS (verify everything) and an
SPS that collapses beyond B = R (verify nothing).
"""
import itertools

import numpy as np
import pytest

import oracle


def _enumerate(c, sps):
    """Best Theta over every allocation l in {0..gamma}^R, by direct evaluation."""
    c = c.astype(np.float64)
    R, g = c.shape
    a = np.cumprod(c, axis=1)
    csum = np.concatenate([np.zeros((R, 1)), np.cumsum(a, axis=1)], axis=1)
    best, second, arg = -np.inf, -np.inf, None
    for ell in itertools.product(range(g + 1), repeat=R):
        B = R + sum(ell)
        if B > sps.size:
            continue
        tau = sum(1.0 + csum[r, ell[r]] for r in range(R))
        th = tau * float(sps[B - 1])
        if th > best:
            best, second, arg = th, best, ell
        elif th > second:
            second = th
    return best, second, np.array(arg)


def _random_instance(rng):
    R = int(rng.integers(1, 5))
    g = int(rng.integers(1, 5))
    c = (1 / (1 + np.exp(-rng.normal(1.5, 1.0, (R, g))))).astype(np.float32)
    n = R * (g + 1) + int(rng.integers(-R * g, 3))
    n = max(n, R)
    kind = rng.integers(0, 3)
    if kind == 0:
        sps = rng.uniform(0.2, 1.0, n)
    elif kind == 1:
        sps = np.sort(rng.uniform(0.2, 1.0, n))[::-1]
    else:
        sps = 1.0 / (1.0 + 0.3 * np.arange(n)) * rng.uniform(0.9, 1.1, n)
    return c, sps.astype(np.float32)


def test_matches_exhaustive_enumeration():
    rng = np.random.default_rng(2024)
    unique = 0
    for trial in range(3000):
        c, sps = _random_instance(rng)
        out = oracle.schedule(c, sps)
        best, second, arg = _enumerate(c, sps)
        assert out["theta_star"] == pytest.approx(best, rel=1e-12), trial
        # the returned allocation attains the optimum when evaluated directly
        a = np.cumprod(c.astype(np.float64), axis=1)
        ell = out["ell"]
        tau = sum(1.0 + a[r, : ell[r]].sum() for r in range(c.shape[0]))
        B = c.shape[0] + ell.sum()
        assert B == c.shape[0] + out["K_star"]
        assert tau * float(sps[B - 1]) == pytest.approx(best, rel=1e-12)
        if best - second > 1e-9 * abs(best):
            unique += 1
            np.testing.assert_array_equal(ell, arg)
    assert unique > 2000


def test_constant_sps_verifies_everything():
    rng = np.random.default_rng(1)
    c = rng.uniform(0.05, 0.99, (6, 5)).astype(np.float32)
    out = oracle.schedule(c, np.ones(6 * 6, np.float32))
    assert (out["ell"] == 5).all() and out["K_star"] == 30


def test_collapsing_sps_verifies_nothing():
    c = np.full((5, 4), 0.9, np.float32)
    sps = np.full(25, 1e-3, np.float32)
    sps[:5] = 1.0
    out = oracle.schedule(c, sps)
    assert (out["ell"] == 0).all() and out["K_star"] == 0
    assert out["theta_star"] == pytest.approx(5.0)


def test_ties_break_by_request_then_position():
    c = np.ones((3, 4), np.float32)            # every a = 1
    sps = np.ones(3 + 5, np.float32)           # room for K <= 5
    out = oracle.schedule(c, sps)
    assert out["K_star"] == 5
    np.testing.assert_array_equal(out["ell"], [4, 1, 0])


def test_prefix_closed_allocation():
    rng = np.random.default_rng(5)
    for _ in range(200):
        c = rng.uniform(0, 1, (8, 6)).astype(np.float32)
        c[rng.random((8, 6)) < 0.1] = 1.0      # create ties inside rows
        sps = np.sort(rng.uniform(0.1, 1.0, 8 * 7))[::-1].astype(np.float32)
        out = oracle.schedule(c, sps)
        a = out["a"]
        # every selected entry has a at least as large as every unselected one
        sel = np.zeros_like(a, bool)
        for r, l in enumerate(out["ell"]):
            sel[r, :l] = True
        if sel.any() and (~sel).any():
            assert a[sel].min() >= a[~sel].max()


def test_rejects_bad_arguments():
    with pytest.raises(oracle.OracleError):
        oracle.schedule(np.full((2, 2), 1.5, np.float32), np.ones(6, np.float32))
    with pytest.raises(oracle.OracleError):
        oracle.schedule(np.full((2, 2), np.nan, np.float32), np.ones(6, np.float32))
    with pytest.raises(oracle.OracleError):
        oracle.schedule(np.full((4, 2), 0.5, np.float32), np.ones(3, np.float32))
