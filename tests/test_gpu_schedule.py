"""GPU parity of the prefix scheduler against the (enumeration-pinned) oracle."""
import numpy as np
import pytest
import torch

import oracle
import draft_sampling_verify_amd as spec
from parity import MARGIN, log, np_

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(c, sps, ws=None):
    ell, a, K, th = spec.spec_schedule(torch.from_numpy(c).cuda(), torch.from_numpy(sps).cuda(), ws=ws)
    torch.cuda.synchronize()
    return np_(ell), np_(a), int(np_(K)[0]), float(np_(th)[0])


def _compare(c, sps, ws=None):
    ell, a, K, th = _run(c, sps, ws)
    o = oracle.schedule(c, sps)
    np.testing.assert_array_equal(a, o["a"])
    assert th == pytest.approx(o["theta_star"], rel=1e-12)
    if o["theta_margin"] >= MARGIN:
        assert K == o["K_star"]
        np.testing.assert_array_equal(ell, o["ell"])
        return 0
    return 1


def test_random_small_instances():
    rng = np.random.default_rng(77)
    excluded = 0
    for trial in range(300):
        R = int(rng.integers(1, 9))
        g = int(rng.integers(1, 9))
        c = (1 / (1 + np.exp(-rng.normal(1.5, 1.0, (R, g))))).astype(np.float32)
        if trial % 7 == 0:
            c[rng.random((R, g)) < 0.3] = 1.0          # ties
        n = max(R, R * (g + 1) + int(rng.integers(-R * g, 3)))
        sps = np.sort(rng.uniform(0.1, 1.0, n))[::-1].astype(np.float32) if trial % 2 else \
            rng.uniform(0.1, 1.0, n).astype(np.float32)
        excluded += _compare(c, sps)
    log("  excluded (theta margin < 1e-6):", excluded)


def test_large_and_edge_instances():
    rng = np.random.default_rng(5)
    for R, g in ((512, 16), (8192, 1), (1, 64), (100, 7), (333, 24)):
        c = (1 / (1 + np.exp(-rng.normal(1.5, 1.0, (R, g))))).astype(np.float32)
        B = np.arange(1, R * (g + 1) + 1)
        sps = (1000.0 / (20 + 0.25 * np.ceil(B / 64) + 0.001 * B)).astype(np.float32)
        _compare(c, sps)
    # constant SPS -> everything; collapsing SPS -> nothing; all-ties ordering
    c = np.full((4, 3), 0.7, np.float32)
    ell, a, K, th = _run(c, np.ones(16, np.float32))
    assert (ell == 3).all() and K == 12
    sps = np.full(16, 1e-3, np.float32)
    sps[:4] = 1.0
    ell, a, K, th = _run(c, sps)
    assert (ell == 0).all() and K == 0
    ell, a, K, th = _run(np.ones((3, 4), np.float32), np.ones(8, np.float32))
    np.testing.assert_array_equal(ell, [4, 1, 0])


def test_bad_confidence_sets_flag():
    ws = spec.Workspace(2, 2, 16, 16)
    c = np.array([[0.5, 1.5], [0.2, 0.1]], np.float32)
    ell, a, K, th = _run(c, np.ones(6, np.float32), ws)
    assert K == -1 and (ell == -1).all()
    assert spec.spec_device_status(ws, clear=True) & spec.SPEC_DEV_BAD_CONFIDENCE
