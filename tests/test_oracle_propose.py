"""Pins of the oracle's Markov-head proposal.

DSpark page, section 3 (p_k = softmax(U_k + B_k)) and section 4
(B = W1[x_{k-1}] W2).  Pinned against library routines (numpy matmul,
scipy softmax, numpy searchsorted/argmax), the W2 = 0 reduction to the base
softmax, temperature scaling, brute-force inverse-CDF search and a
chi-square test of sampled tokens against p_d at V = 16.
"""
import numpy as np
import pytest
from scipy import special, stats

import oracle
import workloads


def _bias_np(W1, W2, x):
    if W1.dtype == np.uint16:
        W1 = workloads.bf16_bits_to_f32(W1)
        W2 = workloads.bf16_bits_to_f32(W2)
    return W2.astype(np.float64) @ W1[x].astype(np.float64)


@pytest.mark.parametrize("bf16", [False, True])
def test_bias_matches_numpy(bf16):
    cfg = workloads.CONFIGS["tiny"].replace(bf16=bf16, r=48, V=777)
    W1, W2 = workloads.weights(cfg)
    for x in (0, 5, 776):
        b = oracle.bias(W1, W2, x)
        np.testing.assert_allclose(b, _bias_np(W1, W2, x), rtol=0, atol=1e-12)


def test_inverse_cdf_brute_force():
    rng = np.random.default_rng(3)
    for trial in range(200):
        V = int(rng.integers(1, 40))
        w = rng.exponential(size=V) * (rng.random(V) < 0.7)
        if w.sum() == 0:
            w[0] = 1.0
        for u in np.linspace(0, 1 - 2 ** -24, 97):
            v, m = oracle.inverse_cdf(w, u)
            # plain linear search on the normalised CDF
            cdf, run, want = w / w.sum(), 0.0, None
            for i in range(V):
                prev = run
                run += cdf[i]
                if run > u:
                    want = i
                    break
            if want is None:
                continue  # rounding fallback; covered below
            if min(run - u, u - prev) > 1e-12:
                assert v == want, (trial, u)
                assert m == pytest.approx(min(run - u, u - prev), abs=1e-12)


def test_inverse_cdf_skips_zero_weights_and_falls_back():
    w = np.array([0.0, 1.0, 0.0, 1.0, 0.0])
    assert oracle.inverse_cdf(w, 0.0)[0] == 1
    assert oracle.inverse_cdf(w, 0.5)[0] == 3
    assert oracle.inverse_cdf(w, 1 - 2 ** -24)[0] == 3


def test_argmax_lowest_index_on_ties():
    z = np.array([1.0, 3.0, 2.0, 3.0])
    v, m = oracle.argmax(z)
    assert v == 1 and m == 0.0
    v, m = oracle.argmax(np.array([0.5, -1.0, 0.25]))
    assert v == 0 and m == pytest.approx(0.25)


def _brute_propose(d, greedy, T, x_cond=None):
    """Independent re-derivation with library routines (scipy softmax,
    numpy searchsorted/argmax) on the same Philox uniforms."""
    U, W1, W2, x0 = d["U"], d["W1"], d["W2"], d["x0"]
    R, g, V = U.shape
    xs = np.zeros((R, g), np.int32)
    pdx = np.zeros((R, g))
    for r in range(R):
        xp = int(x0[r])
        for k in range(1, g + 1):
            z = U[r, k - 1].astype(np.float64) + _bias_np(W1, W2, xp)
            p = special.softmax(z / np.float64(T))
            if greedy:
                tok = int(np.argmax(z))
            else:
                u = oracle.u24(int(oracle.draw(1, 0, int(d["req_ids"][r]), k)[0]))
                tok = int(np.searchsorted(np.cumsum(p), u, side="right"))
            xs[r, k - 1] = tok
            pdx[r, k - 1] = p[tok]
            xp = tok if x_cond is None else int(x_cond[r, k - 1])
    return xs, pdx


@pytest.mark.parametrize("greedy", [False, True])
@pytest.mark.parametrize("cfgname,T", [("tiny", 1.0), ("tiny", 0.7)])
def test_propose_matches_library_rederivation(cfgname, T, greedy):
    cfg = workloads.CONFIGS[cfgname].replace(T=T)
    d = workloads.make(cfg)
    out = oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], np.float32(T), greedy, 1, 0)
    xs, pdx = _brute_propose(d, greedy, np.float32(T))
    ok = out["margin"] > 1e-9
    assert ok.mean() > 0.9
    np.testing.assert_array_equal(out["x"][ok], xs[ok])
    np.testing.assert_allclose(out["pd_x"][ok], pdx[ok], rtol=1e-10, atol=1e-15)


def test_propose_stats_define_the_softmax():
    d = workloads.make("tiny")
    out = oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], 1.0, False, 1, 0)
    R, g, V = d["U"].shape
    for r in range(R):
        xp = int(d["x0"][r])
        for k in range(g):
            z = d["U"][r, k].astype(np.float64) + _bias_np(d["W1"], d["W2"], xp)
            M, S = out["pd_stats"][r, k]
            assert M == pytest.approx(z.max(), abs=1e-12)
            p = np.exp(z - M) / S
            assert p.sum() == pytest.approx(1.0, abs=1e-12)
            assert p[out["x"][r, k]] == pytest.approx(out["pd_x"][r, k], rel=1e-12)
            xp = int(out["x"][r, k])


def test_w2_zero_reduces_to_base_softmax():
    d = workloads.make("tiny")
    W2 = np.zeros_like(d["W2"])
    out = oracle.markov_propose(d["U"], d["W1"], W2, d["x0"], 1.0, False, 1, 0)
    R, g, V = d["U"].shape
    for r in range(R):
        for k in range(g):
            p = special.softmax(d["U"][r, k].astype(np.float64))
            assert out["pd_x"][r, k] == pytest.approx(p[out["x"][r, k]], rel=1e-12)
            np.testing.assert_allclose(out["pd_stats"][r, k, 0], d["U"][r, k].max())


def test_conditioned_mode_follows_given_prefix():
    d = workloads.make("tiny")
    rng = np.random.default_rng(0)
    xc = rng.integers(0, d["U"].shape[2], size=d["U"].shape[:2]).astype(np.int32)
    out = oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], 1.0, False, 1, 0, x_cond=xc)
    xs, pdx = _brute_propose(d, False, 1.0, x_cond=xc)
    ok = out["margin"] > 1e-9
    np.testing.assert_array_equal(out["x"][ok], xs[ok])


def test_request_ids_select_the_uniform_stream():
    d = workloads.make("tiny")
    full = oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], 1.0, False, 1, 0)
    sub = workloads.make("tiny", requests=[2, 0])
    part = oracle.markov_propose(sub["U"], sub["W1"], sub["W2"], sub["x0"], 1.0, False, 1, 0,
                                 req_ids=sub["req_ids"])
    np.testing.assert_array_equal(part["x"], full["x"][[2, 0]])


def test_sampled_tokens_follow_pd_chi_square():
    """10^6 proposals of one position at V = 16 from identical logits: the
    token frequencies must match p_d,1 (chi-square, fixed seed)."""
    V, r, N = 16, 4, 1_000_000
    rng = np.random.default_rng(11)
    u_row = (rng.standard_normal(V) * 1.5).astype(np.float32)
    U = np.broadcast_to(u_row, (N, 1, V))
    W1 = (rng.standard_normal((V, r)) * 0.5).astype(np.float32)
    W2 = (rng.standard_normal((V, r)) * 0.5).astype(np.float32)
    x0 = np.full(N, 3, np.int32)
    out = oracle.markov_propose(U, W1, W2, x0, 1.0, False, 1, 0)
    z = u_row.astype(np.float64) + _bias_np(W1, W2, 3)
    p = special.softmax(z)
    counts = np.bincount(out["x"][:, 0], minlength=V)
    assert stats.chisquare(counts, p * N).pvalue > 1e-4
    np.testing.assert_allclose(out["pd_x"][:, 0], p[out["x"][:, 0]], rtol=1e-12)


def test_rejects_bad_arguments():
    d = workloads.make("tiny")
    with pytest.raises(oracle.OracleError):
        oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], 0.0, False, 1, 0)
    bad = d["x0"].copy()
    bad[1] = d["U"].shape[2]
    with pytest.raises(oracle.OracleError):
        oracle.markov_propose(d["U"], d["W1"], d["W2"], bad, 1.0, False, 1, 0)


def _w2_zero_instance(u_row, R, g, r=4, seed=5):
    rng = np.random.default_rng(seed)
    V = u_row.size
    U = np.ascontiguousarray(np.broadcast_to(u_row.astype(np.float32), (R, g, V)))
    W1 = (rng.standard_normal((V, r)) * 0.5).astype(np.float32)
    W2 = np.zeros((V, r), np.float32)
    x0 = rng.integers(0, V, R).astype(np.int32)
    return U, W1, W2, x0


def test_sampled_tokens_follow_pd_across_granules_chi_square():
    """3 x 10^5 draws (W2 = 0 makes every position alike) over nine tokens
    spread across three 128-id granules, all other logits -inf: the one
    inverse CDF over the row has the law p_d across granule boundaries."""
    rng = np.random.default_rng(23)
    V = 3 * 128
    ids = np.array([3, 60, 127, 128, 200, 255, 256, 300, 383])
    u_row = np.full(V, -np.inf)
    u_row[ids] = rng.standard_normal(9) * 1.2
    U, W1, W2, x0 = _w2_zero_instance(u_row, 1000, 50)
    counts = np.zeros(V, np.int64)
    for rnd in range(6):
        out = oracle.markov_propose(U, W1, W2, x0, 1.0, False, 17, rnd)
        counts += np.bincount(out["x"].ravel(), minlength=V)
    assert counts.sum() == 300000 and counts[np.setdiff1d(np.arange(V), ids)].sum() == 0
    p = special.softmax(u_row[ids].astype(np.float32).astype(np.float64))
    assert stats.chisquare(counts[ids], p * counts.sum()).pvalue > 1e-4


def test_row_without_mass_has_no_sample():
    """Every logit -inf at one position: softmax is 0/0, so that position
    and the rest of its request's chain are -1 / NaN (status 'blanked');
    other requests are unaffected and equal a run without the blank row."""
    d = workloads.make("tiny")
    U = d["U"].copy()
    U[2, 1, :] = -np.inf
    for greedy in (False, True):
        out = oracle.markov_propose(U, d["W1"], d["W2"], d["x0"], 1.0, greedy, 1, 0, allow_blank=True)
        ref = oracle.markov_propose(d["U"], d["W1"], d["W2"], d["x0"], 1.0, greedy, 1, 0)
        assert out["blanked"] and not ref["blanked"]
        assert (out["x"][2, 1:] == -1).all() and out["x"][2, 0] == ref["x"][2, 0]
        assert np.isnan(out["pd_x"][2, 1:]).all() and np.isnan(out["pd_stats"][2, 1:]).all()
        keep = np.arange(U.shape[0]) != 2
        np.testing.assert_array_equal(out["x"][keep], ref["x"][keep])
        with pytest.raises(oracle.OracleError):
            oracle.markov_propose(U, d["W1"], d["W2"], d["x0"], 1.0, greedy, 1, 0)
