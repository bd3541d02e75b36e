"""GPU parity at the limits the C ABI accepts.

- The longest draft chain, gamma = 64, on the fused propose (its tagged
  hand-over words count positions in 7 bits) and on the per-position
  kernels; every request checked against the oracle.
- The largest vocabulary, V = 2^24 (131072 granules); every request checked.
- Logit tensors of more than 2^31 elements (R = 264, gamma = 8, V = 2^20:
  U holds 2.2e9 and the target rows 2.5e9 floats), so every row offset must
  be 64-bit; the first and the last request checked against the oracle, the
  structural invariants on all, and the two verify sweeps bit-identical.
"""
import numpy as np
import pytest
import torch

import workloads
from workloads import Config
import draft_sampling_verify_amd as spec
from parity import check_propose, check_verify, log, np_, run_propose, run_verify, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spec.lib()


def _check_all(cfg, d, greedy, path=0):
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    x, pdx, pds = run_propose(t, cfg, greedy, ws=ws, path=path)
    log("  propose", check_propose(d, np_(x), np_(pdx), np_(pds), greedy))
    n_acc, y, pt_x, c_star = run_verify(t, cfg, x, pds, greedy, ws=ws)
    log("  verify", check_verify(d, np_(x), None, np_(n_acc), np_(y), np_(pt_x), np_(c_star), greedy))
    assert spec.spec_device_status(ws) == 0


GAMMA64 = Config("gamma64", 30, 5, 64, 3000, 64, True, 1.0, 2.0, 0.05, 0.5)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "per_position"])
@pytest.mark.parametrize("greedy", [False, True], ids=["sampled", "greedy"])
def test_longest_draft_chain(fused, greedy):
    log("case gamma=64", "fused" if fused else "per_position", "greedy" if greedy else "sampled")
    _check_all(GAMMA64, workloads.make(GAMMA64), greedy,
               path=spec.SPEC_PATH_AUTO if fused else spec.SPEC_PATH_NO_FUSED_PROPOSE)


VMAX = Config("vmax", 31, 2, 2, 1 << 24, 16, True, 1.0, 2.0, 0.05, 0.5)


def test_largest_vocabulary():
    log("case V=2^24")
    _check_all(VMAX, workloads.make(VMAX), False)


BIG = Config("big_rows", 32, 264, 8, 1 << 20, 128, True, 1.0, 2.0, 0.05, 0.5)


def test_more_than_2_31_elements():
    cfg = BIG
    assert cfg.R * cfg.gamma * cfg.V > 2 ** 31 and cfg.R * (cfg.gamma + 1) * cfg.V > 2 ** 31
    log("case R=264 gamma=8 V=2^20 r=128 (U and target rows past 2^31 elements)")
    U = torch.empty((cfg.R, cfg.gamma, cfg.V), dtype=torch.float32, device="cuda")
    Lt = torch.empty((cfg.R, cfg.gamma + 1, cfg.V), dtype=torch.float32, device="cuda")
    for lo in range(0, cfg.R, 32):                 # a slice of requests at a time
        hi = min(lo + 32, cfg.R)
        u, lt = workloads.request_rows(cfg, range(lo, hi))
        U[lo:hi].copy_(torch.from_numpy(u))
        Lt[lo:hi].copy_(torch.from_numpy(lt))
        del u, lt
    W1, W2 = workloads.weights(cfg)
    t = {"U": U, "Lt": Lt,
         "W1": torch.from_numpy(W1.view(np.int16)).cuda().view(torch.bfloat16),
         "W2": torch.from_numpy(W2.view(np.int16)).cuda().view(torch.bfloat16),
         "x0": torch.from_numpy(workloads.anchors(cfg)).cuda()}
    t["W2p"] = spec.spec_pack_w2(t["W2"])
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    x, pdx, pds = run_propose(t, cfg, False, ws=ws)
    out = run_verify(t, cfg, x, pds, False, ws=ws)
    out2 = run_verify(t, cfg, x, pds, False, ws=ws, path=spec.SPEC_PATH_NO_PIPELINED_SWEEP)  # the staged sweep
    assert spec.spec_device_status(ws) == 0
    n_acc, y, pt_x, c_star = (np_(a) for a in out)
    for a, b in zip(out, out2):
        np.testing.assert_array_equal(np_(a), np_(b))
    xa = np_(x)
    del U, Lt, t, out, out2
    torch.cuda.empty_cache()
    req = [0, cfg.R - 1]
    sub = workloads.make(cfg, requests=req)
    log("  propose", check_propose(sub, xa[req], np_(pdx)[req], np_(pds)[req], False))
    log("  verify", check_verify(sub, xa[req], None, n_acc[req], y[req], pt_x[req], c_star[req], False))
    assert ((xa >= 0) & (xa < cfg.V)).all()
    assert ((n_acc >= 0) & (n_acc <= cfg.gamma)).all()
    for i in range(cfg.R):
        assert (y[i, :n_acc[i]] == xa[i, :n_acc[i]]).all() and (y[i, n_acc[i] + 1:] == -1).all()
        assert 0 <= y[i, n_acc[i]] < cfg.V
    assert np.isfinite(c_star).all() and (c_star >= 0).all() and (c_star <= 1).all()
