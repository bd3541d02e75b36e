"""Pins of the oracle's lossless verification and confidence label.

DSpark page: section 1 diagram (longest accepted prefix plus one bonus
token), section 3 (exact draft probabilities make rejection sampling
possible), section 5 (c* = 1 - 1/2 ||p_d - p_t||_1, tied to the acceptance
rate).  The acceptance rule itself is the standard lossless one (accept with
min(1, p_t/p_d), resample from normalize(max(0, p_t - p_d)), bonus after a
full accept).  Pinned by: Monte Carlo chi-square of emitted tokens against
p_t at V = 16 over 10^6 requests; P(accept) = sum_v min(p_d, p_t) = c*;
E[n_acc] = sum_j prod_{i<=j} c*_i when W2 = 0; identical rows (c* = 1, all
accepted); a planted target peak (certain rejection, correction = the peak);
V = 2 closed form; greedy = target argmax decoding.
"""
import numpy as np
import pytest
from scipy import special, stats

import oracle
import workloads


def _bias_np(W1, W2, x):
    return W2.astype(np.float64) @ W1[x].astype(np.float64)


def _mc_setup(N, V=16, g=3, r=4, seed=5, w2_scale=0.5, target_noise=0.8):
    """N identical requests (same logits, same anchor), distinct Philox streams."""
    rng = np.random.default_rng(seed)
    u = (rng.standard_normal((g + 1, V)) * 1.5).astype(np.float32)
    lt = (u + rng.standard_normal((g + 1, V)) * target_noise).astype(np.float32)
    W1 = (rng.standard_normal((V, r)) * 0.5).astype(np.float32)
    W2 = (rng.standard_normal((V, r)) * w2_scale).astype(np.float32)
    U = np.ascontiguousarray(np.broadcast_to(u[:g], (N, g, V)))
    Lt = np.ascontiguousarray(np.broadcast_to(lt, (N, g + 1, V)))
    x0 = np.full(N, 2, np.int32)
    return U, Lt, W1, W2, x0, u, lt


@pytest.fixture(scope="module")
def mc():
    N = 1_000_000
    U, Lt, W1, W2, x0, u, lt = _mc_setup(N)
    prop = oracle.markov_propose(U, W1, W2, x0, 1.0, False, 1, 0)
    ver = oracle.verify(U, W1, W2, x0, prop["x"], Lt, 1.0, False, 1, 0)
    return dict(N=N, U=U, Lt=Lt, W1=W1, W2=W2, x0=x0, u=u, lt=lt, prop=prop, ver=ver)


@pytest.mark.slow
def test_emitted_tokens_follow_target_chi_square(mc):
    N, g, V = mc["N"], mc["U"].shape[1], mc["U"].shape[2]
    n_acc, y = mc["ver"]["n_acc"], mc["ver"]["y"]
    for k in range(1, g + 2):
        reached = n_acc >= k - 1          # position k was emitted
        tok = y[reached, k - 1]
        p_t = special.softmax(mc["lt"][k - 1].astype(np.float64))
        counts = np.bincount(tok, minlength=V)
        n = reached.sum()
        assert n > 10_000
        assert stats.chisquare(counts, p_t * n).pvalue > 1e-4, k


@pytest.mark.slow
def test_first_position_acceptance_rate_equals_c_star(mc):
    W1, W2, u, lt = mc["W1"], mc["W2"], mc["u"], mc["lt"]
    p_d = special.softmax(u[0].astype(np.float64) + _bias_np(W1, W2, 2))
    p_t = special.softmax(lt[0].astype(np.float64))
    c1 = np.minimum(p_d, p_t).sum()          # E[accept at 1]
    assert mc["ver"]["c_star"][0, 0] == pytest.approx(c1, abs=1e-12)
    rate = (mc["ver"]["acc"][:, 0] == 1).mean()
    se = np.sqrt(c1 * (1 - c1) / mc["N"])
    assert abs(rate - c1) < 5 * se


@pytest.mark.slow
def test_mean_accept_length_closed_form_w2_zero():
    N = 1_000_000
    U, Lt, W1, W2, x0, u, lt = _mc_setup(N, w2_scale=0.0, seed=9)
    prop = oracle.markov_propose(U, W1, W2, x0, 1.0, False, 1, 0)
    ver = oracle.verify(U, W1, W2, x0, prop["x"], Lt, 1.0, False, 1, 0)
    g = U.shape[1]
    c = [np.minimum(special.softmax(u[k].astype(np.float64)),
                    special.softmax(lt[k].astype(np.float64))).sum() for k in range(g)]
    want = sum(np.prod(c[: j + 1]) for j in range(g))
    got = ver["n_acc"].mean()
    se = ver["n_acc"].std() / np.sqrt(N)
    assert abs(got - want) < 5 * se
    # the oracle's own labels give the same closed form (the page's tau formula at c = c*)
    np.testing.assert_allclose(ver["c_star"][0], c, atol=1e-12)


def _identical_rows(cfg="tiny"):
    d = workloads.make(cfg)
    W2 = np.zeros_like(d["W2"])
    R, g, V = d["U"].shape
    Lt = d["Lt"].copy()
    Lt[:, :g] = d["U"]
    return d, W2, Lt


@pytest.mark.parametrize("greedy", [False, True])
def test_identical_distributions_accept_everything(greedy):
    d, W2, Lt = _identical_rows()
    R, g, V = d["U"].shape
    prop = oracle.markov_propose(d["U"], d["W1"], W2, d["x0"], 1.0, greedy, 1, 0)
    ver = oracle.verify(d["U"], d["W1"], W2, d["x0"], prop["x"], Lt, 1.0, greedy, 1, 0)
    assert (ver["n_acc"] == g).all()
    assert (ver["c_star"] == 1.0).all()
    np.testing.assert_array_equal(ver["y"][:, :g], prop["x"])
    # bonus = draw from the extra target row
    for r in range(R):
        p = special.softmax(Lt[r, g].astype(np.float64))
        if greedy:
            assert ver["y"][r, g] == int(np.argmax(Lt[r, g]))
        else:
            uu = oracle.u24(int(oracle.draw(1, 0, r, g + 1)[2]))
            assert ver["y"][r, g] == int(np.searchsorted(np.cumsum(p), uu, side="right"))


def test_planted_peak_forces_rejection_and_correction():
    d = workloads.make("tiny")
    prop = oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], 1.0, False, 1, 0)
    Lt = d["Lt"].copy()
    R, g, V = d["U"].shape
    peaks = []
    for r in range(R):
        t = (int(prop["x"][r, 0]) + 17) % V
        Lt[r, 0, t] += 60.0
        peaks.append(t)
    ver = oracle.verify(d["U"], d["W1"], d["W2"], d["x0"], prop["x"], Lt, 1.0, False, 1, 0)
    assert (ver["n_acc"] == 0).all()
    np.testing.assert_array_equal(ver["y"][:, 0], peaks)
    assert (ver["y"][:, 1:] == -1).all()


def test_two_token_vocabulary_closed_form():
    rng = np.random.default_rng(1)
    R, g, V, r = 50, 2, 2, 2
    U = rng.standard_normal((R, g, V)).astype(np.float32)
    Lt = rng.standard_normal((R, g + 1, V)).astype(np.float32)
    W1 = rng.standard_normal((V, r)).astype(np.float32)
    W2 = rng.standard_normal((V, r)).astype(np.float32)
    x0 = rng.integers(0, 2, R).astype(np.int32)
    x = rng.integers(0, 2, (R, g)).astype(np.int32)
    c, a = oracle.confidence(U, W1, W2, x0, x, Lt, 1.0)
    for i in range(R):
        xp = x0[i]
        for k in range(g):
            p = special.softmax(U[i, k].astype(np.float64) + _bias_np(W1, W2, xp))
            q = special.softmax(Lt[i, k].astype(np.float64))
            assert c[i, k] == pytest.approx(1 - abs(p[0] - q[0]), abs=1e-12)
            xp = x[i, k]
        assert a[i, 1] == pytest.approx(c[i, 0] * c[i, 1], rel=1e-15)


def test_c_star_is_the_overlap_mass_and_in_unit_interval():
    d = workloads.make("tiny")
    prop = oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], 1.0, False, 1, 0)
    ver = oracle.verify(d["U"], d["W1"], d["W2"], d["x0"], prop["x"], d["Lt"], 1.0, False, 1, 0)
    c, a = oracle.confidence(d["U"], d["W1"], d["W2"], d["x0"], prop["x"], d["Lt"], 1.0)
    np.testing.assert_array_equal(c, ver["c_star"])       # same label on both entry points
    assert ((c >= 0) & (c <= 1)).all()
    R, g, V = d["U"].shape
    for r in range(R):
        xp = int(d["x0"][r])
        for k in range(g):
            p = special.softmax(d["U"][r, k].astype(np.float64) + _bias_np(d["W1"], d["W2"], xp))
            q = special.softmax(d["Lt"][r, k].astype(np.float64))
            assert c[r, k] == pytest.approx(np.minimum(p, q).sum(), abs=1e-12)
            assert ver["pt_x"][r, k] == pytest.approx(q[prop["x"][r, k]], rel=1e-12)
            assert ver["pd_x"][r, k] == pytest.approx(p[prop["x"][r, k]], rel=1e-12)
            xp = int(prop["x"][r, k])
        np.testing.assert_allclose(a[r], np.cumprod(c[r]), rtol=1e-15)


def test_greedy_is_target_argmax_decoding():
    d = workloads.make("tiny")
    prop = oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], 1.0, True, 1, 0)
    x = prop["x"].copy()
    Lt = d["Lt"].copy()
    R, g, V = d["U"].shape
    # make the target agree with the first two drafts of every request
    for r in range(R):
        for k in range(2):
            Lt[r, k, x[r, k]] = Lt[r, k].max() + 5.0
        if np.argmax(Lt[r, 2]) == x[r, 2]:
            Lt[r, 2, x[r, 2]] -= 50.0
    ver = oracle.verify(d["U"], d["W1"], d["W2"], d["x0"], x, Lt, 1.0, True, 1, 0)
    assert (ver["n_acc"] == 2).all()
    for r in range(R):
        np.testing.assert_array_equal(ver["y"][r, :2], x[r, :2])
        assert ver["y"][r, 2] == int(np.argmax(Lt[r, 2]))
        assert (ver["y"][r, 3:] == -1).all()


def test_scheduled_lengths_limit_verification():
    d = workloads.make("tiny")
    prop = oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], 1.0, False, 1, 0)
    ell = np.array([0, 1, 4, 2], np.int32)
    ver = oracle.verify(d["U"], d["W1"], d["W2"], d["x0"], prop["x"], d["Lt"], 1.0, False, 1, 0,
                        ell=ell)
    g = d["U"].shape[1]
    assert (ver["n_acc"] <= ell).all()
    for r in range(4):
        assert np.isnan(ver["c_star"][r, ell[r]:]).all()
        assert not np.isnan(ver["c_star"][r, :ell[r]]).any()
        # the emitted token after a full accept comes from target row ell[r]
        if ver["n_acc"][r] == ell[r]:
            assert ver["y"][r, ell[r]] == ver["y_alt"][r, ell[r]]
        assert (ver["y"][r, ver["n_acc"][r] + 1:] == -1).all()
    assert ver["n_acc"][0] == 0
