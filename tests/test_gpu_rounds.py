"""Multi-round decoding on the device (spec_decode_rounds): each round must
match the oracle given that round's anchors (conditioned mode, as for single
calls); the anchors must chain through the last emitted tokens; and the
rounds captured in a HIP graph must replay exactly what the eager calls
produced, replay after replay."""
import numpy as np
import pytest
import torch

import workloads
from workloads import Config
import draft_sampling_verify_amd as spec
from parity import check_propose, check_verify, log, np_, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    # fused single-launch propose (r fills the k-steps, R <= 32)
    "tiny": workloads.CONFIGS["tiny"],
    "fused_r256": Config("fused_r256", 17, 29, 7, 5000, 256, True, 1.0, 3.0, 0.02, 1.0),
    # per-position propose (r = 32 does not fill the k-steps; R > 32)
    "ragged_bf16": Config("ragged_bf16", 11, 37, 3, 1000, 32, True, 0.8, 2.0, 0.05, 0.5),
}
ROUND0 = 5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spec.lib()


@pytest.mark.parametrize("greedy", [False, True], ids=["sampled", "greedy"])
@pytest.mark.parametrize("name", list(CASES))
def test_rounds_match_oracle_round_by_round(name, greedy):
    cfg = CASES[name]
    n = 4
    log("case rounds", name, "greedy" if greedy else "sampled", "R=%d g=%d V=%d r=%d" % (cfg.R, cfg.gamma, cfg.V, cfg.r))
    d = workloads.make(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    anchors, x, n_acc, y, cs = spec.spec_decode_rounds(t["U"], t["W1"], t["W2p"], t["x0"], t["Lt"], cfg.T, n,
                                                       greedy, seed=1, round0=ROUND0, want_c_star=True, ws=ws)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws) == 0
    A, X, N, Y, C = np_(anchors), np_(x), np_(n_acc), np_(y), np_(cs)
    np.testing.assert_array_equal(A[0], d["x0"])
    for i in range(n):
        # the next anchor is the token each request emitted last
        np.testing.assert_array_equal(A[i + 1], Y[i][np.arange(cfg.R), N[i]])
        di = dict(d)
        di["x0"] = A[i]
        sp = check_propose(di, X[i], None, None, greedy, rnd=ROUND0 + i)
        sv = check_verify(di, X[i], None, N[i], Y[i], None, C[i], greedy, rnd=ROUND0 + i)
        log("  round", i, "propose", sp, "verify", sv)


@pytest.mark.parametrize("name", ["fused_r256", "ragged_bf16"])
def test_rounds_graph_replays_match_eager(name):
    cfg = CASES[name]
    n = 3
    d = workloads.make(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    R, g = cfg.R, cfg.gamma
    bufs = dict(anchors=torch.empty((n + 1, R), dtype=torch.int32, device="cuda"),
                x=torch.empty((n, R, g), dtype=torch.int32, device="cuda"),
                n_acc=torch.empty((n, R), dtype=torch.int32, device="cuda"),
                y=torch.empty((n, R, g + 1), dtype=torch.int32, device="cuda"),
                c_star=torch.empty((n, R, g), dtype=torch.float32, device="cuda"))

    def run(stream=None):
        spec.spec_decode_rounds(t["U"], t["W1"], t["W2p"], t["x0"], t["Lt"], cfg.T, n, False, seed=1, round0=ROUND0,
                                ws=ws, stream=stream, **bufs)

    run()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in bufs.items()}
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(stream=side)              # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run(stream=torch.cuda.current_stream())
    for rep in range(3):
        for v in bufs.values():
            v.fill_(-7)               # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in bufs:
            assert torch.equal(bufs[k].isnan() if bufs[k].is_floating_point() else bufs[k],
                               eager[k].isnan() if eager[k].is_floating_point() else eager[k]), (rep, k)
            if bufs[k].is_floating_point():
                ok = ~eager[k].isnan()
                assert torch.equal(bufs[k][ok], eager[k][ok]), (rep, k)
    assert spec.spec_device_status(ws) == 0
    log("  graph replays identical to eager:", name)
