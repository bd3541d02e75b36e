"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases span several 128-id granules, ragged vocabularies (V % 128 != 0,
V % 4 != 0), ragged request counts (R % 32 != 0), rank padding, fp32 and bf16
weights, and degenerate sizes; the measured workloads run at full size, with
the oracle checking every request (c2) or sampled requests (c3, c4, c5).
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
    # the verify sweep that gathers W1 straight into LDS (bf16, r = 128 /
    # 256 / 512): V % 4 != 0 with a ragged last block; several 32-row blocks
    # per workgroup (its double-buffered gather)
    "lds_r128_odd": Config("lds_r128_odd", 19, 37, 3, 1001, 128, True, 1.0, 2.0, 0.05, 0.5),
    "lds_multi": Config("lds_multi", 20, 40, 7, 40000, 256, True, 1.0, 3.0, 0.02, 1.0),
}


@pytest.fixture(params=[True, False], ids=["fused", "per_position"])
def propose_path(request):
    """Run the test with the fused propose allowed, then forbidden."""
    prev = spec.spec_set_propose_fused(request.param)
    yield request.param
    spec.spec_set_propose_fused(prev)


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
    a = [np_(v) for v in run_propose(t, cfg, False, rnd=3, ws=ws)]
    b = [np_(v) for v in run_propose(t, cfg, False, rnd=3, ws=ws)]
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    c = np_(run_propose(t, cfg, False, rnd=4, ws=ws)[0])
    assert (c != a[0]).any()
    st = check_propose(d, c, *[np_(v) for v in run_propose(t, cfg, False, rnd=4, ws=ws)[1:]], False, rnd=4)
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
    x, pdx, pds = spec.spec_markov_propose(t["U"], t["W1"], t["W2p"], x0, 1.0, False, 1, 0, ws=ws)
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
    prev = spec.spec_set_propose_fused(True)
    try:
        for fused in (True, False):
            spec.spec_set_propose_fused(fused)
            for greedy in (False, True):
                x, pdx, pds = run_propose(t, cfg, greedy, ws=ws)
                st = check_propose(d, np_(x), np_(pdx), np_(pds), greedy)
                log("  %s %s" % ("fused" if fused else "per_position", "greedy" if greedy else "sampled"), st)
                outs[fused, greedy] = np_(x)
    finally:
        spec.spec_set_propose_fused(prev)
    assert spec.spec_device_status(ws) == 0
    for greedy in (False, True):
        same = (outs[True, greedy] == outs[False, greedy]).mean()
        log("  token agreement between paths", "greedy" if greedy else "sampled", same)
        assert same > 0.9


@pytest.mark.parametrize("name", ["lds_multi", "rank512", "lds_r128_odd"])
def test_verify_sweep_paths_identical(name):
    """The sweep that gathers W1 rows straight into LDS and the one that
    stages them through registers compute the same products in the same
    order: verify (fixed and scheduled lengths, sampled and greedy) and
    confidence outputs are bit-identical, and match the oracle."""
    cfg = SMALL[name]
    d = workloads.make(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    x, pdx, pds = run_propose(t, cfg, False, ws=ws)
    rng = np.random.default_rng(cfg.index + 100)
    ell = rng.integers(0, cfg.gamma + 1, cfg.R).astype(np.int32)
    ell_d = torch.from_numpy(ell).cuda()
    outs = {}
    prev = spec.spec_set_verify_lds(True)
    try:
        for lds in (True, False):
            spec.spec_set_verify_lds(lds)
            for greedy in (False, True):
                for lens in (None, ell):
                    res = run_verify(t, cfg, x, pds, greedy, ell=None if lens is None else ell_d, ws=ws)
                    res = [np_(v) for v in res]
                    st = check_verify(d, np_(x), lens, *res, greedy)
                    log("  %s %s %s" % ("lds" if lds else "staged", "greedy" if greedy else "sampled",
                                        "fixed" if lens is None else "scheduled"), st)
                    outs[lds, greedy, lens is None] = res
            cs, a = spec.spec_confidence(t["U"], t["W1"], t["W2p"], t["x0"], x, t["Lt"], cfg.T, pd_stats=pds, ws=ws)
            torch.cuda.synchronize()
            outs[lds, "conf"] = [np_(cs), np_(a)]
    finally:
        spec.spec_set_verify_lds(prev)
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


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "per_position"])
def test_drafts_follow_pd_across_blocks_chi_square(fused):
    """The GPU's two-level draw has the law p_d: nine tokens of mass spread
    over three 128-id blocks (all other logits -inf), W2 = 0 so that every
    position draws from the same p_d; 2^18 draws per path (R = 32 takes the
    fused kernel, R = 64 the per-position kernels), chi-square against the
    exact softmax."""
    from scipy import special, stats
    V, r, g = 3 * 128, 64, 8
    R = 32 if fused else 64
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
    prev = spec.spec_set_propose_fused(fused)
    try:
        counts = np.zeros(V, np.int64)
        for rnd in range((1 << 18) // (R * g)):
            x, pdx, pds = spec.spec_markov_propose(U, W1, W2p, x0, 1.0, False, 7, rnd, ws=ws)
            counts += np.bincount(np_(x).ravel(), minlength=V)
    finally:
        spec.spec_set_propose_fused(prev)
    assert spec.spec_device_status(ws) == 0
    assert counts[np.setdiff1d(np.arange(V), ids)].sum() == 0
    p = special.softmax(z.astype(np.float64))
    pv = stats.chisquare(counts[ids], p * counts.sum()).pvalue
    log("  chi-square p-value", pv, "draws", int(counts.sum()))
    assert pv > 1e-4
    np.testing.assert_allclose(np_(pdx), p[np.searchsorted(ids, np_(x))], rtol=0, atol=1e-6)


# ------------------------------------------------------- measured workloads

def _sample(R):
    return sorted(set([0, 1, R // 2, R - 1]))


@pytest.mark.parametrize("greedy", [False, True], ids=["sampled", "greedy"])
def test_c2_full(greedy):
    cfg = workloads.CONFIGS["c2"]
    log("case c2 full", "greedy" if greedy else "sampled")
    d = workloads.make(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    x, pdx, pds = run_propose(t, cfg, greedy, ws=ws)
    log("  propose", check_propose(d, np_(x), np_(pdx), np_(pds), greedy))
    n_acc, y, pt_x, c_star = run_verify(t, cfg, x, pds, greedy, ws=ws)
    log("  verify", check_verify(d, np_(x), None, np_(n_acc), np_(y), np_(pt_x), np_(c_star), greedy))


@pytest.mark.parametrize("name,greedy", [("c3", False), ("c5", False), ("c5", True)])
def test_large_sampled_requests(name, greedy):
    cfg = workloads.CONFIGS[name]
    log("case", name, "greedy" if greedy else "sampled")
    d = workloads.make(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    x, pdx, pds = run_propose(t, cfg, greedy, ws=ws)
    n_acc, y, pt_x, c_star = run_verify(t, cfg, x, pds, greedy, ws=ws)
    req = _sample(cfg.R)
    sub = workloads.make(cfg, requests=req)
    del d
    log("  propose", check_propose(sub, np_(x)[req], np_(pdx)[req], np_(pds)[req], greedy))
    log("  verify", check_verify(sub, np_(x)[req], None, np_(n_acc)[req], np_(y)[req], np_(pt_x)[req],
                                 np_(c_star)[req], greedy))
    # every request: structural invariants
    xa, na, ya = np_(x), np_(n_acc), np_(y)
    assert ((xa >= 0) & (xa < cfg.V)).all()
    assert ((na >= 0) & (na <= cfg.gamma)).all()
    for i in range(cfg.R):
        assert (ya[i, :na[i]] == xa[i, :na[i]]).all() and (ya[i, na[i] + 1:] == -1).all()
        assert 0 <= ya[i, na[i]] < cfg.V


def test_c4_pipeline():
    """propose -> confidence (c* of the drafted rows) -> schedule(c) -> verify(l)."""
    cfg = workloads.CONFIGS["c4"]
    log("case c4 pipeline")
    d = workloads.make(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V, B_max=cfg.sps_len)
    x, pdx, pds = run_propose(t, cfg, False, ws=ws)
    c_star, a_star = spec.spec_confidence(t["U"], t["W1"], t["W2p"], t["x0"], x, t["Lt"], cfg.T, pd_stats=pds,
                                          ws=ws)
    ell, a, K, th = spec.spec_schedule(t["c"], t["sps"], ws=ws)
    n_acc, y, pt_x, cv = run_verify(t, cfg, x, pds, False, ell=ell, ws=ws)
    os_ = oracle.schedule(d["c"], d["sps"])
    log("  schedule K*", int(np_(K)[0]), "oracle", os_["K_star"], "theta margin", os_["theta_margin"])
    assert os_["theta_margin"] > MARGIN
    np.testing.assert_array_equal(np_(ell), os_["ell"])
    assert int(np_(K)[0]) == os_["K_star"]
    assert float(np_(th)[0]) == pytest.approx(os_["theta_star"], rel=1e-12)
    np.testing.assert_array_equal(np_(a), os_["a"])           # same fp64 products, same order
    req = _sample(cfg.R)
    sub = workloads.make(cfg, requests=req)
    del d
    log("  propose", check_propose(sub, np_(x)[req], np_(pdx)[req], np_(pds)[req], False))
    oc, oa = oracle.confidence(sub["U"], sub["W1"], sub["W2"], sub["x0"], np_(x)[req], sub["Lt"],
                               np.float32(cfg.T))
    np.testing.assert_allclose(np_(c_star)[req], oc, rtol=0, atol=PROB_TOL)
    ell_np = np_(ell)
    log("  verify", check_verify(sub, np_(x)[req], ell_np[req], np_(n_acc)[req], np_(y)[req],
                                 np_(pt_x)[req], np_(cv)[req], False))
    # the verify c* equals the confidence c* on verified positions
    for i in range(cfg.R):
        np.testing.assert_allclose(np_(cv)[i, :ell_np[i]], np_(c_star)[i, :ell_np[i]], rtol=0, atol=1e-6)


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
