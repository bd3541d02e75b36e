"""GPU parity of spec_draft_loss against the oracle (DSpark page, section 9).

The loss is teacher-forced on seeded uniform labels y with seeded
confidence-head logits q ~ N(0, 1.5^2).  Tolerances follow the fp32
arithmetic of the kernels:
  - l1: the same sum as c*, so 2 * PROB_TOL (c* = 1 - l1 / 2);
  - ce = log S - (z_y - M) / T: S is an fp32 sum of at most 2^24 terms in
    [0, 1] with a tree order (relative error ~1e-6, so ~1e-6 on log S),
    z_y an fp32 logit of size ~10: 4e-5 absolute covers both;
  - bce = softplus(q) - q c*: the c* error times |q| <= 8, plus fp32
    rounding of softplus: 2e-5 + 8 * PROB_TOL;
  - dq = w a_conf (sigmoid(q) - c*) / sum w: (PROB_TOL + 1e-6) a_conf / sum w;
  - the loss is a weighted mean of the terms, so its error is at most the
    coefficient-weighted sum of the term tolerances; against the GPU's own
    terms it is exact up to fp64 rounding (the coefficients pass as fp32).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import PROB_TOL, log, np_, to_dev
from test_gpu_parity import SMALL
import draft_sampling_verify_amd as spec

pytestmark = pytest.mark.gpu

CE_TOL = 4e-5
L1_TOL = 2 * PROB_TOL
BCE_TOL = 2e-5 + 8 * PROB_TOL
ALPHAS = (0.1, 0.9, 1.0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spec.lib()


def _inputs(cfg):
    d = workloads.make(cfg)
    d["y"] = workloads.loss_labels(cfg)
    d["q"] = workloads.confidence_logits(cfg)
    t = to_dev(d)
    t["y"] = torch.from_numpy(d["y"]).cuda()
    t["q"] = torch.from_numpy(d["q"]).cuda()
    return d, t


def _wsum(R, g):
    return R * sum(math.exp(-(k - 1) / g) for k in range(1, g + 1))


def _check(o, loss, terms, dq, R, g, alphas):
    terms = np_(terms)
    np.testing.assert_allclose(terms[..., 0], o["terms"][..., 0], rtol=0, atol=CE_TOL)
    np.testing.assert_allclose(terms[..., 1], o["terms"][..., 1], rtol=0, atol=L1_TOL)
    np.testing.assert_allclose(terms[..., 2], o["terms"][..., 2], rtol=0, atol=BCE_TOL)
    dq_tol = (PROB_TOL + 1e-6) * abs(alphas[2]) / _wsum(R, g)
    np.testing.assert_allclose(np_(dq), o["dq"], rtol=0, atol=dq_tol)
    loss_tol = abs(alphas[0]) * CE_TOL + abs(alphas[1]) * L1_TOL + abs(alphas[2]) * BCE_TOL
    assert abs(float(np_(loss)[0]) - o["loss"]) <= loss_tol
    return float(np.abs(terms - o["terms"]).max())


@pytest.mark.parametrize("name", ["tiny", "tiny_T07", "ragged_bf16", "odd_vocab", "rank512", "fp32_r256",
                                  "tiny_vocab", "one_token", "lds_r128_odd", "lds_multi"])
def test_loss_matches_oracle(name):
    cfg = SMALL[name]
    log("case", name, "R=%d g=%d V=%d r=%d" % (cfg.R, cfg.gamma, cfg.V, cfg.r))
    d, t = _inputs(cfg)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    loss, terms, dq = spec.spec_draft_loss(t["U"], t["W1"], t["W2p"], t["x0"], t["y"], t["Lt"], t["q"], cfg.T,
                                           ALPHAS, ws=ws)
    torch.cuda.synchronize()
    o = oracle.draft_loss(d["U"], d["W1"], d["W2"], d["x0"], d["y"], d["Lt"], d["q"], np.float32(cfg.T), ALPHAS)
    err = _check(o, loss, terms, dq, cfg.R, cfg.gamma, ALPHAS)
    log("  loss %.9f oracle %.9f, max term error %.2e" % (float(np_(loss)[0]), o["loss"], err))
    assert spec.spec_device_status(ws) == 0


def test_loss_coefficients_optional_outputs_and_repeat():
    """Other coefficients; terms/dq not requested; two calls give identical
    bits (fixed-order reduction)."""
    cfg = SMALL["ragged_bf16"]
    d, t = _inputs(cfg)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    al = (1.0, 0.0, 0.25)
    l1, te, dq = spec.spec_draft_loss(t["U"], t["W1"], t["W2p"], t["x0"], t["y"], t["Lt"], t["q"], cfg.T, al, ws=ws)
    l2, none_t, none_dq = spec.spec_draft_loss(t["U"], t["W1"], t["W2p"], t["x0"], t["y"], t["Lt"], t["q"], cfg.T,
                                               al, want_terms=False, want_dq=False, ws=ws)
    torch.cuda.synchronize()
    assert none_t is None and none_dq is None
    assert np_(l1)[0] == np_(l2)[0]
    o = oracle.draft_loss(d["U"], d["W1"], d["W2"], d["x0"], d["y"], d["Lt"], d["q"], np.float32(cfg.T), al)
    _check(o, l1, te, dq, cfg.R, cfg.gamma, al)


def test_loss_c2_shape():
    """The full vocabulary (V = 129280, bf16, r = 256) on a sample of the
    c2 requests: the loss path's launch configuration at that shape."""
    cfg = workloads.CONFIGS["c2"]
    d = workloads.make(cfg)
    y = workloads.loss_labels(cfg)
    q = workloads.confidence_logits(cfg)
    t = to_dev(d)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    loss, terms, dq = spec.spec_draft_loss(t["U"], t["W1"], t["W2p"], t["x0"], torch.from_numpy(y).cuda(),
                                           t["Lt"], torch.from_numpy(q).cuda(), cfg.T, ALPHAS, ws=ws)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws) == 0
    req = [0, 13, cfg.R - 1]
    sub = workloads.make(cfg, requests=req)
    o = oracle.draft_loss(sub["U"], sub["W1"], sub["W2"], sub["x0"], y[req], sub["Lt"], q[req], np.float32(cfg.T),
                          ALPHAS)
    te = np_(terms)[req]
    np.testing.assert_allclose(te[..., 0], o["terms"][..., 0], rtol=0, atol=CE_TOL)
    np.testing.assert_allclose(te[..., 1], o["terms"][..., 1], rtol=0, atol=L1_TOL)
    np.testing.assert_allclose(te[..., 2], o["terms"][..., 2], rtol=0, atol=BCE_TOL)
    # the loss is the weighted mean of all the terms the GPU reported
    g = cfg.gamma
    w = np.exp(-np.arange(g) / g)
    allt = np_(terms).astype(np.float64)
    want = float((w[None, :] * (allt @ np.array(ALPHAS, np.float32).astype(np.float64))).sum() / _wsum(cfg.R, g))
    assert abs(float(np_(loss)[0]) - want) <= 1e-9 * max(1.0, abs(want))
    log("  c2 loss %.6f" % float(np_(loss)[0]))


def test_bad_label_flags_and_drops_its_positions():
    """A label outside [0, V) poisons its own position and every later one of
    that request (the chain feeds the next bias); they report NaN, add
    nothing to the sum and raise SPEC_DEV_BAD_TOKEN.  Every other position
    is unchanged."""
    cfg = SMALL["ragged_bf16"]
    d, t = _inputs(cfg)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    _, te0, dq0 = spec.spec_draft_loss(t["U"], t["W1"], t["W2p"], t["x0"], t["y"], t["Lt"], t["q"], cfg.T, ALPHAS,
                                       ws=ws)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws) == 0
    y = d["y"].copy()
    y[4, 1] = cfg.V
    y[7, 0] = -3
    loss, te, dq = spec.spec_draft_loss(t["U"], t["W1"], t["W2p"], t["x0"], torch.from_numpy(y).cuda(), t["Lt"],
                                        t["q"], cfg.T, ALPHAS, ws=ws)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws, clear=True) & spec.SPEC_DEV_BAD_TOKEN
    bad = np.zeros((cfg.R, cfg.gamma), bool)
    bad[4, 1:] = True
    bad[7, :] = True
    te, dq, te0, dq0 = np_(te), np_(dq), np_(te0), np_(dq0)
    assert np.isnan(te[bad]).all() and np.isnan(dq[bad]).all()
    np.testing.assert_array_equal(te[~bad], te0[~bad])
    np.testing.assert_array_equal(dq[~bad], dq0[~bad])
    w = np.exp(-np.arange(cfg.gamma) / cfg.gamma)
    contrib = np.where(bad, 0.0, w[None, :] * (te0.astype(np.float64) @ np.array(ALPHAS, np.float32).astype(np.float64)))
    want = float(contrib.sum() / _wsum(cfg.R, cfg.gamma))
    assert abs(float(np_(loss)[0]) - want) <= 1e-9 * max(1.0, abs(want))


def test_loss_rejects_empty_batch():
    cfg = SMALL["tiny"]
    d, t = _inputs(cfg)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    with pytest.raises(spec.SpecError) as e:
        spec.spec_draft_loss(t["U"][:0], t["W1"], t["W2p"], t["x0"][:0], t["y"][:0], t["Lt"][:0], t["q"][:0],
                             cfg.T, ALPHAS, ws=ws)
    assert e.value.status == spec.SPEC_EINVAL


def test_loss_graph_replays_match_eager():
    cfg = SMALL["lds_multi"]
    d, t = _inputs(cfg)
    ws = spec.Workspace(cfg.R, cfg.gamma, cfg.r, cfg.V)
    outs = spec.spec_draft_loss(t["U"], t["W1"], t["W2p"], t["x0"], t["y"], t["Lt"], t["q"], cfg.T, ALPHAS, ws=ws)

    def run(stream):
        spec.spec_draft_loss(t["U"], t["W1"], t["W2p"], t["x0"], t["y"], t["Lt"], t["q"], cfg.T, ALPHAS,
                             loss=outs[0], terms=outs[1], dq=outs[2], ws=ws, stream=stream)

    run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run(torch.cuda.current_stream())
    for rep in range(3):
        for o in outs:
            o.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), (rep, i)
    assert spec.spec_device_status(ws) == 0
