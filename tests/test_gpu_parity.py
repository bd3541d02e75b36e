"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases span several 128-id granules, ragged vocabularies (V % 128 != 0,
V % 4 != 0), ragged request counts (R % 32 != 0), rank padding, fp32 and bf16
weights, and degenerate sizes; the measured workloads run at full size, with
the oracle checking every request of c2, c3 and c5 and 64 requests of c4 (in
host processes, tests/oracle_pool.py).  The method's special cases run on
the GPU too: identical draft and target rows, a planted target peak, rows
without probability mass, and a rejection whose residual mass is zero in
fp32.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import Config
import draft_sampling_verify_amd as spec
from parity import (MARGIN, PROB_TOL, check_propose, check_verify, log, np_, run_propose, run_verify,
                    to_dev)
from oracle_pool import check_requests

FUSED, PER_POSITION = spec.SPEC_PATH_AUTO, spec.SPEC_PATH_NO_FUSED_PROPOSE
STAGED = spec.SPEC_PATH_NO_PIPELINED_SWEEP

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny": workloads.CONFIGS["tiny"],
    "tiny_T07": workloads.CONFIGS["tiny"].replace(name="tiny_T07", T=0.7),
    "ragged_bf16": Config("ragged_bf16", 11, 37, 3, 1000, 32, True, 0.8, 2.0, 0.05, 0.5),
    "odd_vocab": Config("odd_vocab", 12, 5, 2, 1001, 48, True, 1.0, 2.0, 0.1, 0.7),
    "rank512": Config("rank512", 13, 3, 2, 2048, 512, True, 1.0, 2.0, 0.05, 0.5),
    "fp32_r256": Config("fp32_r256", 14, 6, 3, 3000, 256, False, 1.0, 2.0, 0.05, 0.5),
    "tiny_vocab": Config("tiny_vocab", 15, 9, 5, 7, 16, True, 1.0, 1.0, 0.3, 0.5),
    "one_token": Config("one_token", 16, 2, 3, 1, 16, True, 1.0, 1.0, 0.3, 0.5),
    # shapes the fused (single launch) propose takes: r fills the
    # k-steps, R <= 32; a ragged request count; more requests than granules
    "fused_r256": Config("fused_r256", 17, 29, 7, 5000, 256, True, 1.0, 3.0, 0.02, 1.0),
    "fused_many_req": Config("fused_many_req", 18, 30, 4, 300, 64, True, 1.0, 2.0, 0.1, 0.7),
    # the pipelined verify sweep (bf16, r = 128 / 256): V % 4 != 0 with a
    # ragged last block; several 32-row blocks per workgroup
    "lds_r128_odd": Config("lds_r128_odd", 19, 37, 3, 1001, 128, True, 1.0, 2.0, 0.05, 0.5),
    "lds_multi": Config("lds_multi", 20, 40, 7, 40000, 256, True, 1.0, 3.0, 0.02, 1.0),
    # the pipelined per-position tile (more than 32 requests, bf16, r = 128 /
    # 256): ragged request count and vocabulary (V % 4 != 0)
    "piped_tile": Config("piped_tile", 21, 130, 3, 3001, 128, True, 1.0, 2.0, 0.05, 0.5),
    "piped_tile_v4": Config("piped_tile_v4", 22, 100, 4, 5000, 256, True, 0.8, 3.0, 0.02, 1.0),
    # the pipelined tile with three 32-row blocks per granule (the last
    # ragged), V % 4 != 0, r = 128
    "multi_block": Config("multi_block", 23, 70, 3, 9001, 128, True, 1.0, 2.0, 0.05, 0.5),
    # several 32-row blocks through the staged tile (r = 64 has too few
    # k-steps for the pipelined one): a ragged last block, V % 4 != 0
    "multi_block_staged": Config("multi_block_staged", 24, 70, 3, 9001, 64, True, 1.0, 2.0, 0.05, 0.5),
}


@pytest.fixture(params=[FUSED, PER_POSITION], ids=["fused", "per_position"])
def propose_path(request):
    """The propose path bits: the fused launch allowed, then forbidden."""
    return request.param


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spec.lib()


@pytest.mark.parametrize("greedy", [False, True], ids=["sampled", "greedy"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_propose_verify_confidence(name, greedy):
    cfg = SMALL[name]
    log("case", name, "greedy" if greedy else "sampled", "R=%d g=%d V=%d r=%d" % (cfg.R, cfg.gamma, cfg.V, cfg.r))
    d = workloads.make(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    x, pdx, pds = run_propose(t, cfg, greedy, ws=ws)
    st = check_propose(d, np_(x), np_(pdx), np_(pds), greedy)
    log("  propose", st)
    n_acc, y, pt_x, c_star = run_verify(t, cfg, x, pds, greedy, ws=ws)
    sv = check_verify(d, np_(x), None, np_(n_acc), np_(y), np_(pt_x), np_(c_star), greedy)
    log("  verify", sv)
    # scheduled (ragged) lengths, including 0 and gamma
    rng = np.random.default_rng(cfg.index)
    ell = rng.integers(0, cfg.gamma + 1, cfg.R).astype(np.int32)
    ell[0] = 0
    ell[-1] = cfg.gamma
    n2, y2, p2, c2 = run_verify(t, cfg, x, pds, greedy, ell=torch.from_numpy(ell).cuda(), ws=ws)
    sv2 = check_verify(d, np_(x), ell, np_(n2), np_(y2), np_(p2), np_(c2), greedy)
    log("  verify ragged", sv2)
    # confidence, with and without the propose statistics
    oc, oa = oracle.confidence(d["U"], d["W1"], d["W2"], d["x0"], np_(x), d["Lt"], np.float32(cfg.T))
    for stats in (pds, None):
        cs, a = spec.spec_confidence(t["U"], t["W1"], t["W2p"], t["x0"], x, t["Lt"], cfg.T, pd_stats=stats, ws=ws)
        torch.cuda.synchronize()
        np.testing.assert_allclose(np_(cs), oc, rtol=0, atol=PROB_TOL)
        np.testing.assert_allclose(np_(a), oa, rtol=0, atol=PROB_TOL * cfg.gamma)
    assert spec.spec_device_status(ws) == 0


@pytest.mark.parametrize("name", ["ragged_bf16", "fused_r256"])
def test_determinism_and_round_dependence(name, propose_path):
    cfg = SMALL[name]
    d = workloads.make(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    a = [np_(v) for v in run_propose(t, cfg, False, rnd=3, ws=ws, path=propose_path)]
    b = [np_(v) for v in run_propose(t, cfg, False, rnd=3, ws=ws, path=propose_path)]
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    c = np_(run_propose(t, cfg, False, rnd=4, ws=ws, path=propose_path)[0])
    assert (c != a[0]).any()
    st = check_propose(d, c, *[np_(v) for v in run_propose(t, cfg, False, rnd=4, ws=ws, path=propose_path)[1:]],
                       False, rnd=4)
    log("  round 4", st)
    xs = torch.from_numpy(a[0]).cuda()
    pds = torch.from_numpy(a[2]).cuda()
    v1 = [np_(v) for v in run_verify(t, cfg, xs, pds, False, rnd=3, ws=ws)]
    v2 = [np_(v) for v in run_verify(t, cfg, xs, pds, False, rnd=3, ws=ws)]
    for u, v in zip(v1, v2):
        np.testing.assert_array_equal(u, v)


def test_invalid_tokens_flag_and_blank_outputs(propose_path):
    cfg = SMALL["tiny"]
    d = workloads.make(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    x0 = t["x0"].clone()
    x0[1] = cfg.V        # out of range anchor
    x, pdx, pds = spec.spec_markov_propose(t["U"], t["W1"], t["W2p"], x0, 1.0, False, 1, 0, ws=ws,
                                           path=propose_path)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws, clear=True) & spec.SPEC_DEV_BAD_TOKEN
    assert (np_(x)[1] == -1).all() and np.isnan(np_(pdx)[1]).all()
    ok = [0, 2, 3]
    dd = workloads.make(cfg, requests=ok)
    check_propose(dd, np_(x)[ok], np_(pdx)[ok], np_(pds)[ok], False)
    n_acc, y, pt_x, c_star = spec.spec_verify(t["U"], t["W1"], t["W2p"], x0, x, pds, t["Lt"], 1.0, False,
                                              1, 0, ws=ws)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws, clear=True) & spec.SPEC_DEV_BAD_TOKEN
    assert np_(n_acc)[1] == -1 and (np_(y)[1] == -1).all()
    bad_ell = torch.tensor([1, 2, cfg.gamma + 1, 0], dtype=torch.int32, device="cuda")
    n_acc, y, pt_x, c_star = spec.spec_verify(t["U"], t["W1"], t["W2p"], t["x0"], x.clone().fill_(0),
                                              pds, t["Lt"], 1.0, False, 1, 0, ell=bad_ell, ws=ws)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws, clear=True) & spec.SPEC_DEV_BAD_LENGTH
    assert np_(n_acc)[2] == -1
    assert spec.spec_device_status(ws) == 0


@pytest.mark.parametrize("name", ["fused_r256", "fused_many_req", "tiny"])
def test_propose_paths_agree_with_oracle(name):
    """Both ways of running the propose match the oracle on the same inputs;
    their token streams agree except where a decision is within the margin."""
    cfg = SMALL[name]
    d = workloads.make(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    outs = {}
    for path in (FUSED, PER_POSITION):
        for greedy in (False, True):
            x, pdx, pds = run_propose(t, cfg, greedy, ws=ws, path=path)
            st = check_propose(d, np_(x), np_(pdx), np_(pds), greedy)
            log("  %s %s" % ("fused" if path == FUSED else "per_position", "greedy" if greedy else "sampled"), st)
            outs[path, greedy] = np_(x)
    assert spec.spec_device_status(ws) == 0
    for greedy in (False, True):
        same = (outs[FUSED, greedy] == outs[PER_POSITION, greedy]).mean()
        log("  token agreement between paths", "greedy" if greedy else "sampled", same)
        assert same > 0.9


@pytest.mark.parametrize("name", ["lds_multi", "rank512", "lds_r128_odd"])
def test_verify_sweep_paths_identical(name):
    """The pipelined sweep and the staged one compute the same products and
    sum them in the same order: verify (fixed lengths, scheduled lengths
    through the row tables, and every length zero; sampled and greedy) and
    confidence outputs are bit-identical, and match the oracle."""
    cfg = SMALL[name]
    d = workloads.make(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    x, pdx, pds = run_propose(t, cfg, False, ws=ws)
    rng = np.random.default_rng(cfg.index + 100)
    ell = rng.integers(0, cfg.gamma + 1, cfg.R).astype(np.int32)
    lens_cases = {"fixed": None, "scheduled": ell, "zero": np.zeros(cfg.R, np.int32)}
    outs = {}
    for lds in (True, False):
        path = 0 if lds else STAGED
        for greedy in (False, True):
            for kind, lens in lens_cases.items():
                ell_d = None if lens is None else torch.from_numpy(lens).cuda()
                res = run_verify(t, cfg, x, pds, greedy, ell=ell_d, ws=ws, path=path)
                res = [np_(v) for v in res]
                st = check_verify(d, np_(x), lens, *res, greedy)
                log("  %s %s %s" % ("pipelined" if lds else "staged", "greedy" if greedy else "sampled", kind), st)
                outs[lds, greedy, kind] = res
        cs, a = spec.spec_confidence(t["U"], t["W1"], t["W2p"], t["x0"], x, t["Lt"], cfg.T, pd_stats=pds, ws=ws,
                                     path=path)
        torch.cuda.synchronize()
        outs[lds, "conf"] = [np_(cs), np_(a)]
    assert spec.spec_device_status(ws) == 0
    for key in [k for k in outs if k[0]]:
        for got, want in zip(outs[key], outs[(False,) + key[1:]]):
            np.testing.assert_array_equal(got, want)


def test_empty_batch_is_a_no_op():
    """R = 0: every entry point returns success at once with empty outputs;
    the scheduler, whose batch must hold at least one request, rejects it."""
    g, V, r = 4, 1024, 16
    e = torch.empty((0, g, V), device="cuda")
    lt = torch.empty((0, g + 1, V), device="cuda")
    W = torch.zeros((V, r), device="cuda")
    x0 = torch.empty(0, dtype=torch.int32, device="cuda")
    Wp = spec.spec_pack_w2(W)
    ws = spec.Workspace(1, g, r, V, B_max=8)
    x, pdx, pds = spec.spec_markov_propose(e, W, Wp, x0, 1.0, ws=ws)
    assert x.shape == (0, g) and pdx.shape == (0, g) and pds.shape == (0, g, 2)
    n_acc, y, pt_x, c_star = spec.spec_verify(e, W, Wp, x0, x, pds, lt, 1.0, ws=ws)
    assert n_acc.shape == (0,) and y.shape == (0, g + 1) and pt_x.shape == (0, g) and c_star.shape == (0, g)
    cs, a_star = spec.spec_confidence(e, W, Wp, x0, x, lt, 1.0, pd_stats=pds, ws=ws)
    assert cs.shape == (0, g) and a_star.shape == (0, g)
    anchors, xr, nr, yr, cr = spec.spec_decode_rounds(e, W, Wp, x0, lt, 1.0, 3, want_c_star=True, ws=ws)
    assert anchors.shape == (4, 0) and xr.shape == (3, 0, g) and yr.shape == (3, 0, g + 1) and cr.shape == (3, 0, g)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws) == 0
    with pytest.raises(spec.SpecError):
        spec.spec_schedule(torch.empty((0, g), device="cuda"), torch.ones(8, device="cuda"), ws=ws)


def _chi2_case(V=16, r=16, rounds=16, R=65536, seed=21):
    rng = np.random.default_rng(seed)
    u = (rng.standard_normal((2, V)) * 1.5).astype(np.float32)
    lt = (u + rng.standard_normal((2, V)) * 0.8).astype(np.float32)
    W1 = (rng.standard_normal((V, r)) * 0.5).astype(np.float32)
    W2 = (rng.standard_normal((V, r)) * 0.5).astype(np.float32)
    U = torch.from_numpy(u[:1]).cuda().expand(R, 1, V).contiguous()
    Lt = torch.from_numpy(lt).cuda().expand(R, 2, V).contiguous()
    tW1, tW2 = torch.from_numpy(W1).cuda(), spec.spec_pack_w2(torch.from_numpy(W2).cuda())
    x0 = torch.full((R,), 2, dtype=torch.int32, device="cuda")
    ws = spec.Workspace(R, 1, r, V)
    first, acc1 = [], []
    for rnd in range(rounds):
        x, pdx, pds = spec.spec_markov_propose(U, tW1, tW2, x0, 1.0, False, 1, rnd, ws=ws)
        n_acc, y, _, c_star = spec.spec_verify(U, tW1, tW2, x0, x, pds, Lt, 1.0, False, 1, rnd, ws=ws)
        first.append(np_(y)[:, 0])
        acc1.append(np_(n_acc) >= 1)
    from scipy import special
    p_d = special.softmax(u[0].astype(np.float64) + W2.astype(np.float64) @ W1[2].astype(np.float64))
    p_t = special.softmax(lt[0].astype(np.float64))
    return np.concatenate(first), np.concatenate(acc1), p_d, p_t, np_(c_star)[0, 0]


def test_emitted_tokens_follow_target_chi_square():
    """2^20 verify calls' first emitted token at V = 16 must follow p_t (chi-square)."""
    from scipy import stats
    tok, acc, p_d, p_t, c1 = _chi2_case()
    n = tok.size
    counts = np.bincount(tok, minlength=p_t.size)
    pv = stats.chisquare(counts, p_t * n).pvalue
    log("  chi-square p-value", pv)
    assert pv > 1e-4
    c_exact = np.minimum(p_d, p_t).sum()
    assert abs(c1 - c_exact) < PROB_TOL
    se = np.sqrt(c_exact * (1 - c_exact) / n)
    assert abs(acc.mean() - c_exact) < 5 * se


@pytest.mark.parametrize("path", [FUSED, PER_POSITION], ids=["fused", "per_position"])
def test_drafts_follow_pd_across_granules_chi_square(path):
    """The GPU's inverse-CDF draw has the law p_d across granule boundaries:
    nine tokens of mass spread over three 128-id granules (all other logits
    -inf), W2 = 0 so that every position draws from the same p_d; 2^18
    draws per path (R = 32 takes the fused kernel, R = 64 the per-position
    kernels), chi-square against the exact softmax."""
    from scipy import special, stats
    V, r, g = 3 * 128, 64, 8
    R = 32 if path == FUSED else 64
    ids = np.array([3, 60, 127, 128, 200, 255, 256, 300, 383])
    rng = np.random.default_rng(31)
    z = (rng.standard_normal(ids.size) * 1.2).astype(np.float32)
    u_row = np.full(V, -np.inf, np.float32)
    u_row[ids] = z
    U = torch.from_numpy(u_row).cuda().expand(R, g, V).contiguous()
    W1 = torch.from_numpy((rng.standard_normal((V, r)) * 0.5).astype(np.float32)).cuda().to(torch.bfloat16)
    W2p = spec.spec_pack_w2(torch.zeros((V, r), dtype=torch.bfloat16, device="cuda"))
    x0 = torch.from_numpy(rng.integers(0, V, R).astype(np.int32)).cuda()
    ws = spec.Workspace(R, g, r, V)
    counts = np.zeros(V, np.int64)
    for rnd in range((1 << 18) // (R * g)):
        x, pdx, pds = spec.spec_markov_propose(U, W1, W2p, x0, 1.0, False, 7, rnd, ws=ws, path=path)
        counts += np.bincount(np_(x).ravel(), minlength=V)
    assert spec.spec_device_status(ws) == 0
    assert counts[np.setdiff1d(np.arange(V), ids)].sum() == 0
    p = special.softmax(z.astype(np.float64))
    pv = stats.chisquare(counts[ids], p * counts.sum()).pvalue
    log("  chi-square p-value", pv, "draws", int(counts.sum()))
    assert pv > 1e-4
    np.testing.assert_allclose(np_(pdx), p[np.searchsorted(ids, np_(x))], rtol=0, atol=1e-6)


# ------------------------------------------------------- measured workloads

def _gpu_out(x, pdx, pds, n_acc, y, pt_x, c_star):
    return dict(x=np_(x), pd_x=np_(pdx), pd_stats=np_(pds), n_acc=np_(n_acc), y=np_(y), pt_x=np_(pt_x),
                c_star=np_(c_star))


def _report(name, tot):
    p, v = tot["propose"], tot["verify"]
    log("  %s: %d drafts decided, %d within %.0e of a boundary (excluded from the exact comparison), "
        "%d of those differ; free-running chains equal to the oracle's: %d of %d; verify decisions "
        "differing within the margin: %d; mean n_acc %.3f" % (
            name, p["decisions"], p["low_margin"], MARGIN, p["mismatches"], p["chains_equal"], p["requests"],
            v["excluded"], v["n_acc_mean"]))
    # every disagreement is a low-margin decision (asserted per decision);
    # the excluded share is what fp32 arithmetic against a 1e-6 band allows
    assert p["mismatches"] <= p["low_margin"]
    assert p["low_margin"] <= 0.2 * p["decisions"]


@pytest.mark.parametrize("greedy", [False, True], ids=["sampled", "greedy"])
def test_c2_full(greedy):
    cfg = workloads.CONFIGS["c2"]
    log("case c2 full", "greedy" if greedy else "sampled")
    d = workloads.make(cfg)
    t = to_dev(d)
    del d
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    x, pdx, pds = run_propose(t, cfg, greedy, ws=ws)
    out = run_verify(t, cfg, x, pds, greedy, ws=ws)
    assert spec.spec_device_status(ws) == 0
    _report("c2", check_requests(cfg, range(cfg.R), _gpu_out(x, pdx, pds, *out), greedy))


@pytest.mark.parametrize("name,greedy", [("c3", False), ("c3", True), ("c5", False), ("c5", True)])
def test_large_every_request(name, greedy):
    """Every request of c3 and c5 against the oracle (conditioned mode)."""
    cfg = workloads.CONFIGS[name]
    log("case", name, "greedy" if greedy else "sampled", "every request")
    d = workloads.make(cfg)
    t = to_dev(d)
    del d
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    x, pdx, pds = run_propose(t, cfg, greedy, ws=ws)
    out = run_verify(t, cfg, x, pds, greedy, ws=ws)
    assert spec.spec_device_status(ws) == 0
    g = _gpu_out(x, pdx, pds, *out)
    del t
    _report(name, check_requests(cfg, range(cfg.R), g, greedy))


def test_c4_pipeline():
    """propose -> confidence (c* of the drafted rows) -> schedule(c) ->
    verify(l); the schedule exactly, 64 requests (every 8th) against the
    oracle."""
    cfg = workloads.CONFIGS["c4"]
    log("case c4 pipeline")
    d = workloads.make(cfg)
    t = to_dev(d)
    c_in, sps = d["c"], d["sps"]
    del d
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V, B_max=cfg.sps_len)
    x, pdx, pds = run_propose(t, cfg, False, ws=ws)
    c_star, a_star = spec.spec_confidence(t["U"], t["W1"], t["W2p"], t["x0"], x, t["Lt"], cfg.T, pd_stats=pds,
                                          ws=ws)
    ell, a, K, th = spec.spec_schedule(t["c"], t["sps"], ws=ws)
    n_acc, y, pt_x, cv = run_verify(t, cfg, x, pds, False, ell=ell, ws=ws)
    assert spec.spec_device_status(ws) == 0
    os_ = oracle.schedule(c_in, sps)
    log("  schedule K*", int(np_(K)[0]), "oracle", os_["K_star"], "theta margin", os_["theta_margin"])
    assert os_["theta_margin"] > MARGIN
    np.testing.assert_array_equal(np_(ell), os_["ell"])
    assert int(np_(K)[0]) == os_["K_star"]
    assert float(np_(th)[0]) == pytest.approx(os_["theta_star"], rel=1e-12)
    np.testing.assert_array_equal(np_(a), os_["a"])           # same fp64 products, same order
    ell_np = np_(ell)
    # the verify c* equals the confidence c* on verified positions
    for i in range(cfg.R):
        np.testing.assert_allclose(np_(cv)[i, :ell_np[i]], np_(c_star)[i, :ell_np[i]], rtol=0, atol=1e-6)
    g = _gpu_out(x, pdx, pds, n_acc, y, pt_x, cv)
    del t
    _report("c4", check_requests(cfg, range(0, cfg.R, 8), g, False, ell=ell_np, conf=np_(c_star)))


# --------------------------------------------------- the method's special cases

def _edge_inputs(R=6, g=5, V=700, r=32, seed=41, bf16=True):
    rng = np.random.default_rng(seed)
    U = (rng.standard_normal((R, g, V)) * 2.0).astype(np.float32)
    W1 = (rng.standard_normal((V, r)) * 0.1).astype(np.float32)
    W2 = (rng.standard_normal((V, r)) * 0.1).astype(np.float32)
    if bf16:
        W1 = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(W1))
        W2 = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(W2))
    x0 = rng.integers(0, V, R).astype(np.int32)
    return U, W1, W2, x0


def _dev_w(W, bf16=True):
    t = torch.from_numpy(W).cuda()
    return t.to(torch.bfloat16) if bf16 else t


@pytest.mark.parametrize("path", [FUSED, PER_POSITION], ids=["fused", "per_position"])
def test_identical_rows_accept_everything(path):
    """p_t = p_d at every position (W2 = 0 and Lt = U, bonus row its own):
    every draft is accepted (n_acc = gamma), c* = 1, and the bonus is the
    draw from target row gamma, as the oracle's."""
    U, W1, W2, x0 = _edge_inputs()
    R, g, V = U.shape
    W2[:] = 0.0
    rng = np.random.default_rng(42)
    Lt = np.concatenate([U, (rng.standard_normal((R, 1, V)) * 2.0).astype(np.float32)], axis=1)
    tU, tLt = torch.from_numpy(U).cuda(), torch.from_numpy(Lt).cuda()
    tW1, tW2p = _dev_w(W1), spec.spec_pack_w2(_dev_w(W2))
    tx0 = torch.from_numpy(x0).cuda()
    ws = spec.Workspace(R, g, W1.shape[1], V)
    for greedy in (False, True):
        x, pdx, pds = spec.spec_markov_propose(tU, tW1, tW2p, tx0, 1.0, greedy, 3, 0, ws=ws, path=path)
        n_acc, y, pt_x, c_star = spec.spec_verify(tU, tW1, tW2p, tx0, x, pds, tLt, 1.0, greedy, 3, 0, ws=ws)
        torch.cuda.synchronize()
        assert (np_(n_acc) == g).all()
        np.testing.assert_allclose(np_(c_star), 1.0, rtol=0, atol=PROB_TOL)
        np.testing.assert_allclose(np_(pt_x), np_(pdx), rtol=0, atol=PROB_TOL)
        o = oracle.verify(U, W1, W2, x0, np_(x), Lt, 1.0, greedy, 3, 0)
        assert (o["n_acc"] == g).all()
        bonus_ok = (np_(y)[:, g] == o["y"][:, g]) | (o["y_margin"][:, g] < MARGIN)
        assert bonus_ok.all()
        np.testing.assert_array_equal(np_(y)[:, :g], np_(x))
    assert spec.spec_device_status(ws) == 0


def test_planted_target_peak_rejects_at_once():
    """A target row with a one-hot peak (+40 logits) at a token other than
    the draft: the first draft is rejected and the correction is the peak,
    as in the oracle."""
    U, W1, W2, x0 = _edge_inputs(seed=43)
    R, g, V = U.shape
    tU, tW1, tW2p, tx0 = torch.from_numpy(U).cuda(), _dev_w(W1), spec.spec_pack_w2(_dev_w(W2)), \
        torch.from_numpy(x0).cuda()
    ws = spec.Workspace(R, g, W1.shape[1], V)
    for greedy in (False, True):
        x, pdx, pds = spec.spec_markov_propose(tU, tW1, tW2p, tx0, 1.0, greedy, 5, 0, ws=ws)
        torch.cuda.synchronize()
        xs = np_(x)
        peak = (xs[:, 0] + 1 + np.arange(R) * 37) % V
        Lt = np.concatenate([U, U[:, :1]], axis=1).copy()
        Lt[np.arange(R), 0, peak] += 40.0
        tLt = torch.from_numpy(Lt).cuda()
        n_acc, y, pt_x, c_star = spec.spec_verify(tU, tW1, tW2p, tx0, x, pds, tLt, 1.0, greedy, 5, 0, ws=ws)
        torch.cuda.synchronize()
        assert (np_(n_acc) == 0).all()
        np.testing.assert_array_equal(np_(y)[:, 0], peak)
        assert (np_(y)[:, 1:] == -1).all()
        o = oracle.verify(U, W1, W2, x0, xs, Lt, 1.0, greedy, 5, 0)
        np.testing.assert_array_equal(o["y"][:, 0], peak)
        np.testing.assert_allclose(np_(c_star), o["c_star"], rtol=0, atol=PROB_TOL)
    assert spec.spec_device_status(ws) == 0


@pytest.mark.parametrize("path", [FUSED, PER_POSITION], ids=["fused", "per_position"])
@pytest.mark.parametrize("greedy", [False, True], ids=["sampled", "greedy"])
def test_row_without_mass_drafts_nothing(path, greedy):
    """Every draft logit -inf at one position of one request: that position
    and the rest of its chain are -1 / NaN (the oracle's reading: softmax is
    0/0), SPEC_DEV_BAD_TOKEN is raised, and every other request matches the
    oracle."""
    U, W1, W2, x0 = _edge_inputs(seed=44, R=5, g=4)
    R, g, V = U.shape
    U[3, 1, :] = -np.inf
    tU, tW1, tW2p, tx0 = torch.from_numpy(U).cuda(), _dev_w(W1), spec.spec_pack_w2(_dev_w(W2)), \
        torch.from_numpy(x0).cuda()
    ws = spec.Workspace(R, g, W1.shape[1], V)
    x, pdx, pds = spec.spec_markov_propose(tU, tW1, tW2p, tx0, 1.0, greedy, 2, 0, ws=ws, path=path)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws, clear=True) & spec.SPEC_DEV_BAD_TOKEN
    xs = np_(x)
    assert (xs[3, 1:] == -1).all() and np.isnan(np_(pdx)[3, 1:]).all() and np.isnan(np_(pds)[3, 1:]).all()
    o = oracle.markov_propose(U, W1, W2, x0, 1.0, greedy, 2, 0, x_cond=xs, allow_blank=True)
    assert o["blanked"] and (o["x"][3, 1:] == -1).all()
    d = dict(U=U, W1=W1, W2=W2, x0=x0, req_ids=np.arange(R, dtype=np.int32), cfg=Config("edge", 0, R, g, V, 32,
                                                                                          False, 1.0, 0, 0, 0))
    st = check_propose(d, xs, np_(pdx), np_(pds), greedy, seed=2)
    log("  propose", st)


def test_zero_residual_mass_falls_back_to_target():
    """A rejection whose residual mass max(0, p_t - p_d) is exactly zero
    (reading R7: the draw then falls back to p_t).  T = fp32(log2 e), so the
    kernels' exponent scale is exactly 1, and the logits are integers: eight
    tokens at 0..-7 and the draft x_1 at -100, all else -inf, W2 = 0.  The
    target row is the draft row with x_1 removed: p_t(x_1) = 0 forces the
    rejection, and since 2^-100 vanishes against the other weights both
    normalisers are the same number in fp32 and fp64, so p_t = p_d on every
    other token and the residual mass is 0 on both sides.  The GPU and the
    oracle then draw the correction from p_t with the same uniform."""
    R, g, V, r = 8, 3, 500, 32
    T = float(np.float32(np.log2(np.e)))
    ids = np.array([3, 130, 131, 260, 300, 301, 450, 499])
    tok = 200
    U = np.full((R, g, V), -np.inf, np.float32)
    U[:, :, ids] = -np.arange(8, dtype=np.float32)
    U[:, :, tok] = -100.0
    rng = np.random.default_rng(45)
    W1 = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(rng.standard_normal((V, r)).astype(np.float32) * 0.1))
    W2 = np.zeros((V, r), np.float32)
    x0 = rng.integers(0, V, R).astype(np.int32)
    Lt = np.concatenate([U, U[:, :1]], axis=1).copy()
    Lt[:, 0, tok] = -np.inf
    x = np.full((R, g), tok, np.int32)
    tU, tW1, tW2p, tx0 = torch.from_numpy(U).cuda(), _dev_w(W1), spec.spec_pack_w2(_dev_w(W2)), \
        torch.from_numpy(x0).cuda()
    tx, tLt = torch.from_numpy(x).cuda(), torch.from_numpy(Lt).cuda()
    ws = spec.Workspace(R, g, r, V)
    o_p = oracle.markov_propose(U, W1, W2, x0, T, False, 1, 0, x_cond=x)
    pds = torch.from_numpy(o_p["pd_stats"].astype(np.float32)).cuda()     # (0, 1.9921875) exactly
    n_acc, y, pt_x, c_star = spec.spec_verify(tU, tW1, tW2p, tx0, tx, pds, tLt, T, False, 9, 0, ws=ws)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws) == 0
    o = oracle.verify(U, W1, W2, x0, x, Lt, T, False, 9, 0)
    assert (np_(n_acc) == 0).all() and (o["n_acc"] == 0).all()
    same = (np_(y)[:, 0] == o["y"][:, 0]) | (o["y_margin"][:, 0] < MARGIN)
    assert same.all(), (np_(y)[:, 0], o["y"][:, 0])
    assert np.isin(np_(y)[:, 0], ids).all()
    np.testing.assert_allclose(np_(c_star)[:, 0], 1.0, rtol=0, atol=PROB_TOL)
    log("  corrections", np_(y)[:, 0].tolist())


def test_philox_matches_the_oracle_on_ten_million_counters():
    """The kernels' Philox4x32-10 (through spec_philox_words, which calls the
    same device function as every draw) against the oracle's C
    implementation, bit for bit, on 10^7 counters."""
    n = 10_000_000
    seed, rnd = 0x0123456789ABCDEF, 0xFEDCBA9876543210
    got = np_(spec.spec_philox_words(seed, rnd, n)).view(np.uint32)
    want = oracle.philox_words(seed, rnd, n)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("bf16,r,V", [(True, 256, 1000), (True, 16, 33), (True, 512, 64),
                                      (False, 256, 70), (False, 16, 5)])
def test_pack_w2_layout(bf16, r, V):
    """The packed W2 equals a numpy re-derivation of the documented layout."""
    rng = np.random.default_rng(r + V)
    W = rng.standard_normal((V, r)).astype(np.float32)
    nblk = (V + 31) // 32
    Wpad = np.zeros((nblk * 32, r), np.float32)
    if bf16:
        bits = workloads.to_bf16_bits(W)
        Wt = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        Wpad[:V] = workloads.bf16_bits_to_f32(bits)
        got = workloads.bf16_bits_to_f32(np_(spec.spec_pack_w2(Wt)).view(np.uint16))
        got = got.reshape(nblk, r // 16, 2, 32, 8)            # block, k-step, half, row, element
        want = Wpad.reshape(nblk, 32, r // 16, 2, 8).transpose(0, 2, 3, 1, 4)
    else:
        Wt = torch.from_numpy(W).cuda()
        Wpad[:V] = W
        got = np_(spec.spec_pack_w2(Wt)).view(np.float32).reshape(nblk, r // 8, 2, 32, 4)
        # group t, half h, row n, component q  <-  W[32b + n, 8t + 2q + h]
        want = Wpad.reshape(nblk, 32, r // 8, 4, 2).transpose(0, 2, 4, 1, 3)
    np.testing.assert_array_equal(got, want)


def test_pack_w2_rv_equals_pack_w2():
    """spec_pack_w2_rv on the r x V matrix packs the same bytes as
    spec_pack_w2 on its [V, r] transpose."""
    rng = np.random.default_rng(51)
    for bf16 in (True, False):
        for r, V in ((256, 1000), (16, 33)):
            W = torch.from_numpy(rng.standard_normal((V, r)).astype(np.float32)).cuda()
            if bf16:
                W = W.to(torch.bfloat16)
            a = spec.spec_pack_w2(W)
            b = spec.spec_pack_w2_rv(W.t().contiguous())
            torch.cuda.synchronize()
            assert torch.equal(a, b)


def test_reused_workspace_memory_gives_correct_tokens():
    """A workspace allocated where a freed one with leftover hand-over words
    lived (the caching allocator hands the same block back): after
    spec_workspace_init the fused propose matches the per-position path and
    the oracle, for a short chain (gamma = 2) and a different seed."""
    cfg = SMALL["fused_r256"].replace(name="reuse", gamma=2)
    d = workloads.make(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    run_propose(t, cfg, False, seed=1, ws=ws)
    ptr = ws.tensor.data_ptr()
    del ws
    ws2 = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    log("  same block reused:", ws2.tensor.data_ptr() == ptr)
    x, pdx, pds = run_propose(t, cfg, False, seed=5, ws=ws2)
    xp = run_propose(t, cfg, False, seed=5, ws=ws2, path=PER_POSITION)[0]
    st = check_propose(d, np_(x), np_(pdx), np_(pds), False, seed=5)
    log("  propose", st)
    assert (np_(x) == np_(xp)).mean() > 0.9
    assert spec.spec_device_status(ws2) == 0


def test_fused_propose_abort_word_ends_the_call():
    """The fused propose's failure path, forced from the host: the abort word
    of the coming call is written into the workspace header before the call
    (as a workgroup that gave up waiting would write it).  Every workgroup
    leaves at once, the call returns promptly with SPEC_DEV_WAIT_FAILED
    raised, and the next call on the same workspace (a new call counter) is
    correct again."""
    import time
    cfg = SMALL["fused_r256"]
    d = workloads.make(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    run_propose(t, cfg, False, ws=ws)
    hdr = ws.tensor[:16].view(torch.int32)        # status, call counter, abort word, -
    epoch = int(hdr[1].item()) & 0x7FFFFFFF
    hdr[2] = epoch - (1 << 31)                     # the bits of epoch | 0x80000000
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    x, pdx, pds = run_propose(t, cfg, False, ws=ws)
    el = time.perf_counter() - t0
    flags = spec.spec_device_status(ws, clear=True)
    log("  aborted call: %.1f ms, flags %d" % (1e3 * el, flags))
    assert flags & spec.SPEC_DEV_WAIT_FAILED
    assert el < 0.5                                # no wait ran to its bound
    assert int(hdr[1].item()) & 0x7FFFFFFF == (epoch + 1) & 0x7FFFFFFF
    x, pdx, pds = run_propose(t, cfg, False, rnd=4, ws=ws)
    assert spec.spec_device_status(ws) == 0
    log("  next call", check_propose(d, np_(x), np_(pdx), np_(pds), False, rnd=4))

