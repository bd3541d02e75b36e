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


def _sawtooth(R, g, rng):
    """The decreasing sawtooth SPS table of the scheduler-heavy workload."""
    B = np.arange(1, R * (g + 1) + 1)
    eps = rng.uniform(-1, 1, int(np.ceil(B[-1] / 64)) + 1)
    step = np.ceil(B / 64).astype(int)
    return (1000.0 * (1 + 0.08 * eps[step]) / (20 + 0.25 * step + 0.001 * B)).astype(np.float32)


@pytest.mark.parametrize("R,g", [(5, 6), (64, 8), (512, 16)])
def test_async_sequence_matches_oracle(R, g):
    """The production step over a sequence of calls on one device ring: the
    count verified at step t is the optimum of step t-2, the ranking is the
    current one; ell, K_used, K_star, a and the ring match the oracle."""
    rng = np.random.default_rng(R + g)
    sps = _sawtooth(R, g, rng)
    sps_d = torch.from_numpy(sps).cuda()
    ring = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    oring = [-1, -1]
    ws = spec.Workspace(R, g, 16, 1, B_max=sps.size)
    excluded = 0
    for t in range(10):
        c = (1 / (1 + np.exp(-rng.normal(1.5, 1.0, (R, g))))).astype(np.float32)
        ell, a, Ku, Ks, th = spec.spec_schedule_async(torch.from_numpy(c).cuda(), sps_d, ring, ws=ws)
        torch.cuda.synchronize()
        o = oracle.schedule_async(c, sps, oring)
        np.testing.assert_array_equal(np_(a), o["a"])
        assert int(np_(Ku)[0]) == o["K_used"]
        np.testing.assert_array_equal(np_(ell), o["ell"])
        if o["theta_margin"] >= MARGIN:
            assert int(np_(Ks)[0]) == o["K_star"]
        else:
            excluded += 1
        oring = list(np_(ring))        # follow the device ring (equal unless excluded)
        assert oring[0] == (o["K_hist"][0])
    log("  async steps excluded (theta margin < 1e-6):", excluded)
    assert spec.spec_device_status(ws) == 0


def test_async_graph_replay():
    """One captured production step, replayed with new confidences copied
    into its input between replays: every replay equals the oracle step."""
    R, g = 64, 8
    rng = np.random.default_rng(123)
    sps = _sawtooth(R, g, rng)
    sps_d = torch.from_numpy(sps).cuda()
    c_d = torch.zeros((R, g), dtype=torch.float32, device="cuda")
    ring = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    ws = spec.Workspace(R, g, 16, 1, B_max=sps.size)
    outs = [torch.empty(R, dtype=torch.int32, device="cuda"), torch.empty((R, g), dtype=torch.float64, device="cuda"),
            torch.empty(1, dtype=torch.int32, device="cuda"), torch.empty(1, dtype=torch.int32, device="cuda"),
            torch.empty(1, dtype=torch.float64, device="cuda")]
    c_d.fill_(0.5)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):  # warm-up outside the capture
        spec.spec_schedule_async(c_d, sps_d, ring, *outs, ws=ws, stream=s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        spec.spec_schedule_async(c_d, sps_d, ring, *outs, ws=ws, stream=s)
    ring.fill_(-1)
    torch.cuda.synchronize()
    oring = [-1, -1]
    for t in range(8):
        c = (1 / (1 + np.exp(-rng.normal(1.5, 1.0, (R, g))))).astype(np.float32)
        c_d.copy_(torch.from_numpy(c))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o = oracle.schedule_async(c, sps, oring)
        np.testing.assert_array_equal(np_(outs[0]), o["ell"])
        assert int(np_(outs[2])[0]) == o["K_used"]
        oring = list(np_(ring))
    assert spec.spec_device_status(ws) == 0


def test_async_bad_confidence_keeps_ring():
    ws = spec.Workspace(2, 2, 16, 16)
    ring = torch.tensor([3, 4], dtype=torch.int32, device="cuda")
    c = torch.tensor([[0.5, float("nan")], [0.2, 0.1]], dtype=torch.float32, device="cuda")
    ell, a, Ku, Ks, th = spec.spec_schedule_async(c, torch.ones(6, device="cuda"), ring, ws=ws)
    torch.cuda.synchronize()
    assert int(np_(Ku)[0]) == -1 and int(np_(Ks)[0]) == -1 and (np_(ell) == -1).all()
    np.testing.assert_array_equal(np_(ring), [3, 4])
    assert spec.spec_device_status(ws, clear=True) & spec.SPEC_DEV_BAD_CONFIDENCE
