"""GPU-vs-oracle comparison helpers for the parity tests.

Protocol (conditioned mode): the oracle re-takes every GPU decision given the
GPU's own earlier tokens.  Token ids, accept lengths and schedules must be
identical, except at decisions whose margin in the oracle (fp64) is below
MARGIN (RACE_MARGIN for the race of the sampled draft draw); those are
counted, checked to be a valid near-boundary choice, and the GPU's choice is
adopted.  Probabilities and c* must agree within PROB_TOL
absolute (fp32 kernels vs the fp64 oracle).
"""
import numpy as np
import torch
from scipy import special

import oracle
import workloads
import draft_sampling_verify_amd as spec

MARGIN = 1e-6
PROB_TOL = 1e-5
# Race keys of the sampled draft draw (natural-log units): the GPU forms them
# in fp32 from a granule's max logit, its weight sum and the race term, good
# to a few 1e-6; decisions whose top-2 keys lie closer than this are excluded.
RACE_MARGIN = 2e-5
BLOCK = 128  # ids per block of the draft draw


def log(*a):
    print(*a, flush=True)


def to_dev(d):
    """numpy workload dict -> torch tensors on the GPU."""
    t = {}
    for k in ("U", "Lt"):
        t[k] = torch.from_numpy(np.ascontiguousarray(d[k])).cuda()
    for k in ("W1", "W2"):
        w = d[k]
        if w.dtype == np.uint16:
            t[k] = torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            t[k] = torch.from_numpy(w).cuda()
    t["W2p"] = spec.spec_pack_w2(t["W2"])
    t["x0"] = torch.from_numpy(d["x0"]).cuda()
    if "c" in d:
        t["c"] = torch.from_numpy(d["c"]).cuda()
    if "sps" in d:
        t["sps"] = torch.from_numpy(d["sps"]).cuda()
    return t


def _wf64(w):
    return (workloads.bf16_bits_to_f32(w) if w.dtype == np.uint16 else w).astype(np.float64)


def draft_dist(d, i, k, xprev, T):
    """fp64 draft distribution of row i, position k (1-based) given x_{k-1}."""
    z = d["U"][i, k - 1].astype(np.float64) + _wf64(d["W2"]) @ _wf64(d["W1"])[xprev]
    return special.softmax(z / np.float64(T))


def target_dist(d, i, row, T):
    return special.softmax(d["Lt"][i, row].astype(np.float64) / np.float64(T))


def near_boundary(p, tok, u, tol=MARGIN):
    """True if u lies within tol of token tok's inverse-CDF interval."""
    c = np.cumsum(p / p.sum())
    lo = c[tok - 1] if tok > 0 else 0.0
    return (lo - tol) <= u < (c[tok] + tol)


def block_draw_near(p, tok, e, u):
    """True if tok is a valid outcome of the two-level draft draw within the
    margins: its block's race key within RACE_MARGIN of the best, and tok
    the block's inverse-CDF pick up to MARGIN."""
    P = np.add.reduceat(p, np.arange(0, p.size, BLOCK))
    with np.errstate(divide="ignore"):
        keys = np.log(P) - np.log(-np.log(e[:P.size]))
    b = tok // BLOCK
    if keys[b] < keys.max() - RACE_MARGIN:
        return False
    return near_boundary(p[b * BLOCK:(b + 1) * BLOCK], tok - b * BLOCK, u[b])


def check_propose(d, x, pd_x, pd_stats, greedy, seed=1, rnd=0):
    """d: oracle-side inputs of the checked requests; x, pd_x, pd_stats: the
    GPU outputs of the same requests (numpy)."""
    T = np.float32(d["cfg"].T)
    o = oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], T, greedy, seed, rnd,
                              req_ids=d["req_ids"], x_cond=x)
    mism = o["x"] != x
    if greedy:
        low = o["margin"] < MARGIN
    else:
        low = (o["margin"] < RACE_MARGIN) | (o["margin_within"] < MARGIN)
    hard = mism & ~low
    assert not hard.any(), "propose token mismatch at %s (gpu %s, oracle %s, margins %s %s)" % (
        np.argwhere(hard)[:5].tolist(), x[hard][:5], o["x"][hard][:5], o["margin"][hard][:5],
        o["margin_within"][hard][:5])
    V = d["U"].shape[2]
    for i, k in np.argwhere(mism):
        if greedy:
            continue
        xprev = d["x0"][i] if k == 0 else x[i, k - 1]
        p = draft_dist(d, i, k + 1, xprev, T)
        e, u = oracle.block_uniforms(seed, rnd, int(d["req_ids"][i]), int(k) + 1, (V + BLOCK - 1) // BLOCK)
        assert block_draw_near(p, int(x[i, k]), e, u), (i, k)
    ok = ~mism
    if pd_x is None:                 # tokens only (callers that keep no probabilities)
        return dict(decisions=int(x.size), excluded=int(mism.sum()), low_margin=int(low.sum()))
    np.testing.assert_allclose(pd_x[ok], o["pd_x"][ok], rtol=0, atol=PROB_TOL)
    M, S = pd_stats[..., 0], pd_stats[..., 1]
    np.testing.assert_allclose(M[ok], o["pd_stats"][..., 0][ok], rtol=0,
                               atol=PROB_TOL * max(1.0, float(np.abs(M).max())))
    np.testing.assert_allclose(S[ok], o["pd_stats"][..., 1][ok], rtol=PROB_TOL)
    return dict(decisions=int(x.size), excluded=int(mism.sum()), low_margin=int(low.sum()))


def check_verify(d, x, ell, n_acc, y, pt_x, c_star, greedy, seed=1, rnd=0):
    """Conditioned comparison of one verify call (numpy in, numpy GPU outputs)."""
    T = np.float32(d["cfg"].T)
    o = oracle.verify(d["U"], d["W1"], d["W2"], d["x0"], x, d["Lt"], T, greedy, seed, rnd,
                      ell=ell, req_ids=d["req_ids"])
    return check_verify_against(o, x, ell, n_acc, y, pt_x, c_star)


def check_verify_against(o, x, ell, n_acc, y, pt_x, c_star):
    """GPU verify outputs against an oracle verify dict conditioned on the
    same drafts x."""
    R, g = x.shape
    excluded = 0
    for i in range(R):
        L = g if ell is None else int(ell[i])
        na = int(n_acc[i])
        assert 0 <= na <= L, (i, na, L)
        for k in range(na):                       # accepted at k+1
            if o["acc"][i, k] != 1:
                assert o["acc_margin"][i, k] < MARGIN, ("accept", i, k, o["acc_margin"][i, k])
                excluded += 1
        if na < L and o["acc"][i, na] != 0:        # rejected at na+1
            assert o["acc_margin"][i, na] < MARGIN, ("reject", i, na, o["acc_margin"][i, na])
            excluded += 1
        want = int(o["y_alt"][i, na])
        if int(y[i, na]) != want:
            assert o["y_margin"][i, na] < MARGIN, ("emit", i, na, int(y[i, na]), want, o["y_margin"][i, na])
            excluded += 1
        np.testing.assert_array_equal(y[i, :na], x[i, :na])
        assert (y[i, na + 1:] == -1).all()
        if pt_x is not None:
            np.testing.assert_allclose(pt_x[i, :L], o["pt_x"][i, :L], rtol=0, atol=PROB_TOL)
            assert np.isnan(pt_x[i, L:]).all()
        if c_star is not None:
            np.testing.assert_allclose(c_star[i, :L], o["c_star"][i, :L], rtol=0, atol=PROB_TOL)
            assert np.isnan(c_star[i, L:]).all()
    return dict(requests=R, excluded=excluded, n_acc_mean=float(np.mean(n_acc)),
                oracle_free_running_equal=int((o["n_acc"] == n_acc).sum()))


def run_propose(t, cfg, greedy, seed=1, rnd=0, ws=None):
    x, pdx, pds = spec.spec_markov_propose(t["U"], t["W1"], t["W2p"], t["x0"], cfg.T, greedy, seed, rnd,
                                           ws=ws)
    torch.cuda.synchronize()
    return x, pdx, pds


def run_verify(t, cfg, x, pds, greedy, ell=None, seed=1, rnd=0, ws=None):
    n_acc, y, pt_x, c_star = spec.spec_verify(t["U"], t["W1"], t["W2p"], t["x0"], x, pds, t["Lt"], cfg.T,
                                              greedy, seed, rnd, ell=ell, ws=ws)
    torch.cuda.synchronize()
    return n_acc, y, pt_x, c_star


def np_(t):
    return None if t is None else t.detach().cpu().numpy()
