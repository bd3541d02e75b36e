"""GPU-vs-oracle comparison helpers that need no GPU (numpy, scipy and the
oracle only), so that host worker processes can run them.

Protocol (conditioned mode): the oracle re-takes every GPU decision given the
GPU's own earlier tokens.  Token ids, accept lengths and schedules must be
identical, except at decisions whose margin in the oracle (fp64) is below
MARGIN; those are counted, checked to be a valid near-boundary choice, and
the GPU's choice is adopted.  Probabilities and c* must agree within PROB_TOL
absolute (fp32 kernels vs the fp64 oracle).
"""
import numpy as np
from scipy import special

import oracle
import workloads

MARGIN = 1e-6
PROB_TOL = 1e-5


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


def check_propose(d, x, pd_x, pd_stats, greedy, seed=1, rnd=0, free_running=False):
    """d: oracle-side inputs of the checked requests; x, pd_x, pd_stats: the
    GPU outputs of the same requests (numpy).  Returns the counts: decisions,
    low_margin (decisions within MARGIN of a boundary: excluded from the
    bit-exact comparison), mismatches (GPU and oracle disagree; each is a
    low-margin decision whose GPU choice is valid) and, with free_running,
    chains_equal (requests whose whole draft chain equals the oracle's run
    on its own tokens)."""
    T = np.float32(d["cfg"].T)
    o = oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], T, greedy, seed, rnd,
                              req_ids=d["req_ids"], x_cond=x, allow_blank=True)
    mism = o["x"] != x
    low = o["margin"] < MARGIN
    hard = mism & ~low
    assert not hard.any(), "propose token mismatch at %s (gpu %s, oracle %s, margin %s)" % (
        np.argwhere(hard)[:5].tolist(), x[hard][:5], o["x"][hard][:5], o["margin"][hard][:5])
    for i, k in np.argwhere(mism):
        if greedy:
            continue
        xprev = d["x0"][i] if k == 0 else x[i, k - 1]
        p = draft_dist(d, i, k + 1, xprev, T)
        u = oracle.u24(int(oracle.draw(seed, rnd, int(d["req_ids"][i]), int(k) + 1)[0]))
        assert near_boundary(p, int(x[i, k]), u), (i, k)
    ok = ~mism
    res = dict(decisions=int((x >= 0).sum()), low_margin=int((low & (x >= 0)).sum()), mismatches=int(mism.sum()),
               excluded=int(mism.sum()))
    if free_running:
        f = oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], T, greedy, seed, rnd, req_ids=d["req_ids"],
                                  allow_blank=True)
        res["chains_equal"] = int((f["x"] == x).all(axis=1).sum())
        res["requests"] = int(x.shape[0])
    if pd_x is None:                 # tokens only (callers that keep no probabilities)
        return res
    np.testing.assert_allclose(pd_x[ok], o["pd_x"][ok], rtol=0, atol=PROB_TOL)
    M, S = pd_stats[..., 0], pd_stats[..., 1]
    fin = ok & np.isfinite(M)
    np.testing.assert_allclose(M[fin], o["pd_stats"][..., 0][fin], rtol=0,
                               atol=PROB_TOL * max(1.0, float(np.abs(M[fin]).max(initial=0.0))))
    np.testing.assert_allclose(S[ok], o["pd_stats"][..., 1][ok], rtol=PROB_TOL)
    return res


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
