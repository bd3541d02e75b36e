"""The allocation-free propose (spec_markov_propose_noalloc, through the C
ABI) against the workspace entry point spec_markov_propose: identical tokens,
probabilities and statistics on two calls in a row, the second smaller than
the first (the static array keeps the first call's contents), on both the
fused launch's shapes and the per-position kernels' shapes; the size limit is
refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from workloads import Config
import draft_sampling_verify_amd as spec
from parity import log, np_, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spec.lib()


def _noalloc(t, cfg, greedy, seed, rnd):
    """The C entry point called directly (ctypes), outputs preallocated."""
    R, g, V = t["U"].shape
    r = t["W1"].shape[1]
    x = torch.full((R, g), -7, dtype=torch.int32, device="cuda")
    pdx = torch.full((R, g), -7.0, dtype=torch.float32, device="cuda")
    pds = torch.full((R, g, 2), -7.0, dtype=torch.float32, device="cuda")
    flags = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    P = lambda a: ctypes.c_void_p(a.data_ptr())
    st = spec.lib().spec_markov_propose_noalloc(
        P(t["U"]), P(t["W1"]), P(t["W2p"]), spec.SPEC_BF16 if t["W1"].dtype == torch.bfloat16 else spec.SPEC_F32,
        P(t["x0"]), R, g, r, V, float(cfg.T), int(greedy), seed, rnd, P(x), P(pdx), P(pds), P(flags),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == spec.SPEC_OK, spec.status_str(st)
    torch.cuda.synchronize()
    return np_(x), np_(pdx), np_(pds), int(np_(flags)[0])


def _reference(t, cfg, greedy, seed, rnd):
    R, g, V = t["U"].shape
    ws = spec.Workspace(R, g, t["W1"].shape[1], V)
    x, pdx, pds = spec.spec_markov_propose(t["U"], t["W1"], t["W2p"], t["x0"], cfg.T, greedy, seed, rnd, ws=ws)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws) == 0
    return np_(x), np_(pdx), np_(pds)


BIG = Config("na_big", 70, 32, 5, 20000, 256, True, 1.0, 3.0, 0.02, 1.0)      # fused launch
SMALL = Config("na_small", 71, 9, 3, 3001, 256, True, 0.8, 2.0, 0.05, 0.5)  # fused, fewer requests
WIDE = Config("na_wide", 72, 48, 4, 5000, 64, True, 1.0, 2.0, 0.05, 0.5)     # per-position kernels


@pytest.mark.parametrize("greedy", [False, True], ids=["sampled", "greedy"])
@pytest.mark.parametrize("first,second", [(BIG, SMALL), (WIDE, SMALL), (BIG, BIG)],
                         ids=["fused_then_smaller", "per_position_then_fused", "same_twice"])
def test_noalloc_equals_workspace_entry_point(first, second, greedy):
    for i, cfg in enumerate((first, second)):
        t = to_dev(workloads.make(cfg))
        got = _noalloc(t, cfg, greedy, 3, 10 + i)
        want = _reference(t, cfg, greedy, 3, 10 + i)
        log("  call %d: %s R=%d V=%d" % (i, cfg.name, cfg.R, cfg.V))
        assert got[3] == 0
        np.testing.assert_array_equal(got[0], want[0])
        np.testing.assert_array_equal(got[1], want[1])
        np.testing.assert_array_equal(got[2], want[2])


def test_noalloc_flags_and_limit():
    cfg = SMALL
    t = to_dev(workloads.make(cfg))
    t["x0"][2] = cfg.V                      # an anchor outside [0, V)
    x, pdx, pds, flags = _noalloc(t, cfg, False, 1, 0)
    assert flags & spec.SPEC_DEV_BAD_TOKEN and (x[2] == -1).all()
    t["x0"][2] = 0
    assert _noalloc(t, cfg, False, 1, 0)[3] == 0       # the next call starts clear
    # a size whose propose workspace exceeds the static array is refused
    R, V = 1024, 129280
    need = spec.spec_workspace_bytes(spec.SPEC_OP_PROPOSE, R, 2, 16, V)
    assert need > spec.SPEC_NOALLOC_BYTES
    F = ctypes.c_void_p(4096)
    st = spec.lib().spec_markov_propose_noalloc(F, F, F, 1, F, R, 2, 16, V, 1.0, 0, 1, 0, F, F, F, F, None)
    assert st == spec.SPEC_EUNSUPPORTED
