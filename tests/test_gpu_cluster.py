"""GPU parity of the clustered draft head and its verification against the
oracle (the MTP survey page, zdszero.github.io "spec_mtp": Gemma 4 assistant
section; the FROZEN_KV_MTP path of its SGLang section).

Conditioned mode, as for the Markov head: the oracle takes the GPU's
cluster selection and tokens as given and re-takes each decision.
  - Selection: equal to the oracle's wherever the gap between the K_c-th and
    the next coarse logit exceeds CUT_TOL; elsewhere the GPU's clusters must
    all lie within CUT_TOL of the cut.  The coarse logits are fp32 MFMA sums
    of d bf16 products of size <= |h_i c_i|; for these inputs their error is
    below 1e-5, and CUT_TOL = 1e-4 leaves a margin of ten.
  - Tokens equal except where the oracle's margin is below MARGIN (then the
    GPU's token must be a valid near-boundary choice); p_d(x), p_t(x) and c*
    within PROB_TOL; the normaliser (M, Z) within PROB_TOL (relative for Z).
"""
import functools

import numpy as np
import pytest
import torch
from scipy import special

import oracle
import workloads
from parity import MARGIN, PROB_TOL, check_verify_against, log, near_boundary, np_
import draft_sampling_verify_amd as spec

pytestmark = pytest.mark.gpu

CUT_TOL = 1e-4
SMALL = ["cl_tiny", "cl_ragged", "cl_mid", "cl_rows", "cl_wide", "cl_max"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    spec.lib()


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _dev(d):
    return dict(H=_bf16(d["H"]), C=_bf16(d["C"]), E=_bf16(d["E"]),
                cl_off=torch.from_numpy(d["cl_off"]).cuda(), cl_tok=torch.from_numpy(d["cl_tok"]).cuda(),
                Lt=torch.from_numpy(d["Lt"]).cuda())


def _expansion(d, sel_row, h):
    """ids and fp64 fine logits of a row's expanded tokens (expansion order)."""
    off, tok = d["cl_off"], d["cl_tok"]
    ids = np.concatenate([tok[off[c]:off[c + 1]] for c in sel_row])
    return ids, workloads.bf16_bits_to_f32(d["E"][ids]).astype(np.float64) @ h


def check_cluster_propose(d, o, x, pd_x, sel, pd_stats, greedy, seed, rnd):
    cfg = d["cfg"]
    R, g, K = sel.shape
    Hf = workloads.bf16_bits_to_f32(d["H"]).astype(np.float64)
    Cf = workloads.bf16_bits_to_f32(d["C"]).astype(np.float64)
    near_cut = 0
    for r in range(R):
        for k in range(g):
            if (sel[r, k] != o["sel"][r, k]).any():
                assert o["cut"][r, k] < CUT_TOL, ("selection", r, k, o["cut"][r, k])
                s = Cf @ Hf[r, k]
                kth = np.sort(s)[::-1][K - 1]
                assert (s[sel[r, k]] >= kth - CUT_TOL).all()
                assert (np.diff(sel[r, k]) > 0).all()
                near_cut += 1
    # the draws, conditioned on the GPU's selection
    T = np.float64(np.float32(cfg.T))
    low = excluded = 0
    for r in range(R):
        for k in range(g):
            ids, z = _expansion(d, sel[r, k], Hf[r, k])
            p = special.softmax(z / T)
            assert x[r, k] in ids, (r, k)
            i = int(np.where(ids == x[r, k])[0][0])
            assert pd_x[r, k] == pytest.approx(p[i], abs=PROB_TOL)
            assert pd_stats[r, k, 0] == pytest.approx(z.max(), abs=PROB_TOL * max(1.0, abs(z.max())))
            Z = np.exp((z - z.max()) / T).sum()
            assert pd_stats[r, k, 1] == pytest.approx(Z, rel=PROB_TOL)
            if greedy:
                best = ids[z == z.max()].min()
                srt = np.sort(z)
                margin = srt[-1] - srt[-2] if z.size > 1 else np.inf
                if x[r, k] != best:
                    assert margin < MARGIN, (r, k, margin)
                    excluded += 1
                low += margin < MARGIN
            else:
                u = oracle.u24(int(oracle.draw(seed, rnd, r, k + 1)[0]))
                cdf = np.cumsum(p)
                want = min(int(np.searchsorted(cdf, u * cdf[-1], side="right")), ids.size - 1)
                lo = cdf[want - 1] if want > 0 else 0.0
                margin = min(cdf[want] - u, u - lo)
                if i != want:
                    assert margin < MARGIN and near_boundary(p, i, u), (r, k, i, want, margin)
                    excluded += 1
                low += margin < MARGIN
    return dict(rows=R * g, near_cut=near_cut, low_margin=int(low), excluded=excluded)


@functools.lru_cache(maxsize=2)
def _inputs(name):
    return workloads.make_cluster(name)


def _run(name, greedy, seed=1, rnd=0, ell=None):
    d = _inputs(name)
    cfg = d["cfg"]
    t = _dev(d)
    ws = spec.ClusterWorkspace(cfg.R, cfg.gamma, cfg.d, cfg.N_c, cfg.K_c, d["max_cl"], cfg.V)
    tok_slot = spec.spec_cluster_index(t["cl_off"], t["cl_tok"], ws=ws)
    x, pd_x, sel, zf, pds = spec.spec_cluster_propose(t["H"], t["C"], t["E"], t["cl_off"], t["cl_tok"], cfg.K_c,
                                                      d["max_cl"], cfg.T, greedy, seed, rnd, ws=ws)
    ell_t = None if ell is None else torch.from_numpy(ell).cuda()
    n_acc, y, pt_x, c_star = spec.spec_cluster_verify(tok_slot, sel, zf, pds, x, t["Lt"], cfg.T, cfg.N_c, greedy,
                                                      seed, rnd, ell=ell_t, ws=ws)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws) == 0
    return d, t, dict(tok_slot=np_(tok_slot), x=np_(x), pd_x=np_(pd_x), sel=np_(sel), zf=np_(zf), pds=np_(pds),
                      n_acc=np_(n_acc), y=np_(y), pt_x=np_(pt_x), c_star=np_(c_star))


@pytest.mark.parametrize("greedy", [False, True], ids=["sampled", "greedy"])
@pytest.mark.parametrize("name", SMALL)
def test_cluster_propose_and_verify_match_oracle(name, greedy):
    d, t, g = _run(name, greedy, seed=3, rnd=2)
    cfg = d["cfg"]
    log("case", name, "greedy" if greedy else "sampled", "R=%d g=%d d=%d V=%d N_c=%d K_c=%d" % (
        cfg.R, cfg.gamma, cfg.d, cfg.V, cfg.N_c, cfg.K_c))
    T = np.float32(cfg.T)
    o = oracle.cluster_propose(d["H"], d["C"], d["E"], d["cl_off"], d["cl_tok"], cfg.K_c, T, greedy, 3, 2)
    st = check_cluster_propose(d, o, g["x"], g["pd_x"], g["sel"], g["pds"], greedy, 3, 2)
    log("  propose", st)
    ov = oracle.cluster_verify(d["H"], d["E"], d["cl_off"], d["cl_tok"], g["sel"], g["x"], d["Lt"], T, greedy, 3, 2)
    sv = check_verify_against(ov, g["x"], None, g["n_acc"], g["y"], g["pt_x"], g["c_star"])
    log("  verify", sv)


def test_cluster_empty_batch_is_a_no_op():
    d = _inputs("cl_tiny")
    cfg = d["cfg"]
    t = _dev(d)
    ws = spec.ClusterWorkspace(1, cfg.gamma, cfg.d, cfg.N_c, cfg.K_c, d["max_cl"], cfg.V)
    tok_slot = spec.spec_cluster_index(t["cl_off"], t["cl_tok"], ws=ws)
    H = t["H"][:0]
    x, pd_x, sel, zf, pds = spec.spec_cluster_propose(H, t["C"], t["E"], t["cl_off"], t["cl_tok"], cfg.K_c,
                                                      d["max_cl"], cfg.T, ws=ws)
    assert x.shape == (0, cfg.gamma) and sel.shape == (0, cfg.gamma, cfg.K_c)
    n_acc, y, pt_x, c_star = spec.spec_cluster_verify(tok_slot, sel, zf, pds, x, t["Lt"][:0], cfg.T, cfg.N_c,
                                                      ws=ws)
    assert n_acc.shape == (0,) and y.shape == (0, cfg.gamma + 1) and c_star.shape == (0, cfg.gamma)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws) == 0


def test_cluster_index_is_the_inverse_of_the_clustering():
    d = workloads.make_cluster("cl_ragged")
    t = _dev(d)
    ws = spec.ClusterWorkspace(1, 1, 16, 1, 1, 1, 1)
    slot = np_(spec.spec_cluster_index(t["cl_off"], t["cl_tok"], ws=ws))
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws) == 0
    off, tok = d["cl_off"], d["cl_tok"]
    for c in range(off.size - 1):
        for i in range(off[c], off[c + 1]):
            assert slot[tok[i]] == (c << 16) | (i - off[c])


def test_cluster_index_flags_a_non_partition():
    d = workloads.make_cluster("cl_tiny")
    tok = d["cl_tok"].copy()
    tok[5] = tok[6]                                  # listed twice, another token missing
    ws = spec.ClusterWorkspace(1, 1, 16, 1, 1, 1, 1)
    spec.spec_cluster_index(torch.from_numpy(d["cl_off"]).cuda(), torch.from_numpy(tok).cuda(), ws=ws)
    torch.cuda.synchronize()
    assert spec.spec_device_status(ws) & spec.SPEC_DEV_BAD_CLUSTER


def test_scheduled_lengths_and_determinism():
    cfg = workloads.CLUSTER_CONFIGS["cl_ragged"]
    ell = np.random.default_rng(5).integers(0, cfg.gamma + 1, cfg.R).astype(np.int32)
    ell[0], ell[-1] = 0, cfg.gamma
    d, t, g = _run("cl_ragged", False, seed=7, rnd=1, ell=ell)
    _, _, g2 = _run("cl_ragged", False, seed=7, rnd=1, ell=ell)
    for key in g:
        np.testing.assert_array_equal(g[key], g2[key])
    T = np.float32(cfg.T)
    ov = oracle.cluster_verify(d["H"], d["E"], d["cl_off"], d["cl_tok"], g["sel"], g["x"], d["Lt"], T, False, 7, 1,
                               ell=ell)
    log("  verify ragged", check_verify_against(ov, g["x"], ell, g["n_acc"], g["y"], g["pt_x"], g["c_star"]))


def test_cluster_too_large_for_max_cl_blanks_the_row():
    d = workloads.make_cluster("cl_ragged")
    cfg = d["cfg"]
    t = _dev(d)
    small = d["max_cl"] - 1                           # the largest cluster does not fit
    ws = spec.ClusterWorkspace(cfg.R, cfg.gamma, cfg.d, cfg.N_c, cfg.K_c, small, cfg.V)
    x, pd_x, sel, zf, pds = spec.spec_cluster_propose(t["H"], t["C"], t["E"], t["cl_off"], t["cl_tok"], cfg.K_c,
                                                      small, cfg.T, ws=ws)
    torch.cuda.synchronize()
    sizes = np.diff(d["cl_off"])
    big = (sizes[np_(sel)] > small).any(axis=-1)
    xs = np_(x)
    assert (xs[big] == -1).all() and (xs[~big] >= 0).all()
    if big.any():
        assert spec.spec_device_status(ws) & spec.SPEC_DEV_BAD_CLUSTER


@pytest.mark.parametrize("greedy", [False, True], ids=["sampled", "greedy"])
def test_gemma_e2b_shape_sampled_rows(greedy):
    """The full head (V = 262144, d = 1536, 2048 centres, top 32) in the
    launch configuration the benchmark times; the oracle checks every row of
    the first request."""
    d, t, g = _run("gemma_e2b", greedy, seed=1, rnd=0)
    cfg = d["cfg"]
    sub = dict(d)
    sub["H"] = d["H"][:1]
    sub["Lt"] = d["Lt"][:1]
    T = np.float32(cfg.T)
    o = oracle.cluster_propose(sub["H"], d["C"], d["E"], d["cl_off"], d["cl_tok"], cfg.K_c, T, greedy, 1, 0)
    st = check_cluster_propose(sub, o, g["x"][:1], g["pd_x"][:1], g["sel"][:1], g["pds"][:1], greedy, 1, 0)
    log("  gemma_e2b propose", st)
    ov = oracle.cluster_verify(sub["H"], d["E"], d["cl_off"], d["cl_tok"], g["sel"][:1], g["x"][:1], sub["Lt"], T,
                               greedy, 1, 0)
    log("  gemma_e2b verify", check_verify_against(ov, g["x"][:1], None, g["n_acc"][:1], g["y"][:1], g["pt_x"][:1],
                                                  g["c_star"][:1]))
    assert (g["n_acc"] >= 0).all()


def test_cluster_graph_replays_match_eager():
    """propose + verify of the clustered head captured in one HIP graph:
    every replay (with eager work in between) equals the eager call."""
    d = _inputs("cl_mid")
    cfg = d["cfg"]
    t = _dev(d)
    mc = d["max_cl"]
    ws = spec.ClusterWorkspace(cfg.R, cfg.gamma, cfg.d, cfg.N_c, cfg.K_c, mc, cfg.V)
    slot = spec.spec_cluster_index(t["cl_off"], t["cl_tok"], ws=ws)
    po = spec.spec_cluster_propose(t["H"], t["C"], t["E"], t["cl_off"], t["cl_tok"], cfg.K_c, mc, cfg.T, ws=ws)
    vo = spec.spec_cluster_verify(slot, po[2], po[3], po[4], po[0], t["Lt"], cfg.T, cfg.N_c, ws=ws)
    outs = list(po) + list(vo)

    def run(stream):
        spec.spec_cluster_propose(t["H"], t["C"], t["E"], t["cl_off"], t["cl_tok"], cfg.K_c, mc, cfg.T, False, 5, 9,
                                  *po, ws=ws, stream=stream)
        spec.spec_cluster_verify(slot, po[2], po[3], po[4], po[0], t["Lt"], cfg.T, cfg.N_c, False, 5, 9, None, *vo,
                                 ws=ws, stream=stream)

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
