"""Pins of the oracle's clustered draft head and its verification.

The MTP survey page (zdszero.github.io "spec_mtp"), Gemma 4 assistant section
and the FROZEN_KV_MTP path of its SGLang section: coarse logits over cluster
centres, the top K_c clusters expanded, the draft distribution a softmax over
the expanded tokens.  Pinned against
  - numpy's lexicographic sort for the top-K selection (ties to the smaller
    cluster) and scipy's softmax over the expanded set;
  - full expansion over contiguous clusters: the draw is then the plain
    inverse CDF of the whole softmax (numpy searchsorted);
  - a chi-square test of sampled tokens against the sparse distribution;
  - verification: a chi-square test that emitted tokens follow p_t although
    the draft puts zero mass outside its clusters (the lossless property),
    P(accept at 1) = sum min(p_d, p_t) = c*, and, with exactly representable
    logits, the Markov oracle's verify with U = H E^T and W2 = 0.
"""
import numpy as np
import pytest
from scipy import special, stats

import oracle


def _instance(seed, R=3, g=2, d=12, N_c=10, V=60, sizes=None):
    rng = np.random.default_rng(seed)
    H = rng.normal(0, 1, (R, g, d)).astype(np.float32)
    C = rng.normal(0, 1, (N_c, d)).astype(np.float32)
    E = rng.normal(0, 0.5, (V, d)).astype(np.float32)
    if sizes is None:
        cuts = np.sort(rng.choice(np.arange(1, V), N_c - 1, replace=False))
        sizes = np.diff(np.concatenate([[0], cuts, [V]]))
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    tok = rng.permutation(V).astype(np.int32)
    return H, C, E, off, tok


def _expanded(H, E, off, tok, sel_row, h_idx):
    ids = np.concatenate([tok[off[c]:off[c + 1]] for c in sel_row])
    z = E[ids].astype(np.float64) @ H[h_idx].astype(np.float64)
    return ids, z


def test_selection_is_top_k_with_small_index_ties():
    for seed in range(20):
        H, C, E, off, tok = _instance(seed, N_c=16)
        C[5] = C[9]                                   # a tie between clusters 5 and 9
        K = 1 + seed % 15
        o = oracle.cluster_propose(H, C, E, off, tok, K, 1.0)
        R, g, _ = H.shape
        for r in range(R):
            for k in range(g):
                s = C.astype(np.float64) @ H[r, k].astype(np.float64)
                order = np.lexsort((np.arange(s.size), -s))   # s descending, then index ascending
                np.testing.assert_array_equal(o["sel"][r, k], np.sort(order[:K]))
                ss = s[order]
                assert o["cut"][r, k] == pytest.approx(ss[K - 1] - ss[K], abs=1e-12)


def test_draft_distribution_is_softmax_over_expanded_tokens():
    H, C, E, off, tok = _instance(7)
    T = 0.8
    o = oracle.cluster_propose(H, C, E, off, tok, 4, T)
    R, g, _ = H.shape
    for r in range(R):
        for k in range(g):
            ids, z = _expanded(H, E, off, tok, o["sel"][r, k], (r, k))
            p = special.softmax(z / np.float64(np.float32(T)))
            assert o["x"][r, k] in ids
            i = int(np.where(ids == o["x"][r, k])[0][0])
            assert o["pd_x"][r, k] == pytest.approx(p[i], rel=1e-12)
            assert o["pd_stats"][r, k, 0] == pytest.approx(z.max(), rel=1e-12)
            want_Z = np.exp((z - z.max()) / np.float64(np.float32(T))).sum()
            assert o["pd_stats"][r, k, 1] == pytest.approx(want_Z, rel=1e-12)


def test_full_expansion_of_contiguous_clusters_is_the_plain_inverse_cdf():
    V, N_c = 64, 8
    H, C, E, off, _ = _instance(11, R=5, g=3, N_c=N_c, V=V, sizes=[8] * N_c)
    tok = np.arange(V, dtype=np.int32)
    o = oracle.cluster_propose(H, C, E, off, tok, N_c, 1.0, seed=5, rnd=2)
    R, g, _ = H.shape
    for r in range(R):
        for k in range(g):
            p = special.softmax(E.astype(np.float64) @ H[r, k].astype(np.float64))
            u = oracle.u24(oracle.draw(5, 2, r, k + 1)[0])
            cdf = np.cumsum(p)
            want = int(np.searchsorted(cdf, u * cdf[-1], side="right"))
            assert o["x"][r, k] == want


def test_sampled_tokens_follow_the_sparse_distribution_chi_square():
    V, N_c, K = 16, 8, 3
    H, C, E, off, tok = _instance(13, R=1, g=1, d=6, N_c=N_c, V=V, sizes=[2] * N_c)
    n = 200000
    Hn = np.repeat(H, n, axis=0)                      # n i.i.d. rows (distinct Philox counters)
    o = oracle.cluster_propose(Hn, C, E, off, tok, K, 1.0, seed=3)
    ids, z = _expanded(H, E, off, tok, o["sel"][0, 0], (0, 0))
    p = np.zeros(V)
    p[ids] = special.softmax(z)
    counts = np.bincount(o["x"][:, 0], minlength=V)
    assert counts[p == 0].sum() == 0
    m = p > 0
    assert stats.chisquare(counts[m], p[m] * n).pvalue > 1e-4


def test_greedy_takes_the_largest_logit_smallest_id_on_ties():
    H, C, E, off, tok = _instance(17, V=40, N_c=5)
    E[tok[off[2]]] = E[tok[off[2] + 1]]               # two tokens of cluster 2 with equal logits
    o = oracle.cluster_propose(H, C, E, off, tok, 5, 1.0, greedy=True)
    R, g, _ = H.shape
    for r in range(R):
        for k in range(g):
            ids, z = _expanded(H, E, off, tok, o["sel"][r, k], (r, k))
            best = z.max()
            assert o["x"][r, k] == ids[z == best].min()


def _verify_instance(seed, n, V=16, N_c=8, K=3, g=2):
    H, C, E, off, tok = _instance(seed, R=1, g=g, d=6, N_c=N_c, V=V, sizes=[V // N_c] * N_c)
    rng = np.random.default_rng(seed + 100)
    Lt1 = rng.normal(0, 1, (1, g + 1, V)).astype(np.float32)
    Hn = np.repeat(H, n, axis=0)
    Lt = np.repeat(Lt1, n, axis=0)
    d = oracle.cluster_propose(Hn, C, E, off, tok, K, 1.0, seed=9)
    v = oracle.cluster_verify(Hn, E, off, tok, d["sel"], d["x"], Lt, 1.0, seed=9)
    return H, E, off, tok, Lt1, d, v


def test_emitted_tokens_follow_target_despite_sparse_draft_chi_square():
    n = 200000
    H, E, off, tok, Lt1, d, v = _verify_instance(21, n)
    p_t = special.softmax(Lt1[0, 0].astype(np.float64))
    counts = np.bincount(v["y"][:, 0], minlength=p_t.size)
    assert stats.chisquare(counts, p_t * n).pvalue > 1e-4


def test_first_position_acceptance_rate_equals_c_star():
    n = 200000
    H, E, off, tok, Lt1, d, v = _verify_instance(23, n)
    ids, z = _expanded(H, E, off, tok, d["sel"][0, 0], (0, 0))
    p_d = np.zeros(Lt1.shape[-1])
    p_d[ids] = special.softmax(z)
    p_t = special.softmax(Lt1[0, 0].astype(np.float64))
    c = np.minimum(p_d, p_t).sum()
    assert v["c_star"][0, 0] == pytest.approx(1 - 0.5 * np.abs(p_d - p_t).sum(), abs=1e-12)
    assert v["c_star"][0, 0] == pytest.approx(c, abs=1e-12)
    rate = (v["n_acc"] >= 1).mean()
    assert abs(rate - c) < 5 * np.sqrt(c * (1 - c) / n)


def test_full_expansion_equals_markov_verify_with_exact_logits():
    # quarter-integer H, E and d = 4: every dot product is exact in fp32, so
    # U = H E^T carries the same values into the Markov oracle
    rng = np.random.default_rng(31)
    R, g, d, V, N_c = 6, 3, 4, 24, 4
    H = (rng.integers(-4, 5, (R, g, d)) / 4).astype(np.float32)
    E = (rng.integers(-4, 5, (V, d)) / 4).astype(np.float32)
    C = rng.normal(0, 1, (N_c, d)).astype(np.float32)
    off = np.arange(0, V + 1, V // N_c, dtype=np.int32)
    tok = rng.permutation(V).astype(np.int32)
    Lt = rng.normal(0, 1, (R, g + 1, V)).astype(np.float32)
    for greedy in (False, True):
        dr = oracle.cluster_propose(H, C, E, off, tok, N_c, 0.9, greedy=greedy, seed=4)
        v = oracle.cluster_verify(H, E, off, tok, dr["sel"], dr["x"], Lt, 0.9, greedy=greedy, seed=4)
        U = np.einsum("rgd,vd->rgv", H.astype(np.float64), E.astype(np.float64)).astype(np.float32)
        W = np.zeros((V, 2), np.float32)
        m = oracle.verify(U, W, W, np.zeros(R, np.int32), dr["x"], Lt, 0.9, greedy, 4, 0)
        for key in ("n_acc", "y", "acc"):
            np.testing.assert_array_equal(v[key], m[key])
        for key in ("c_star", "pt_x", "pd_x"):
            np.testing.assert_allclose(v[key], m[key], rtol=0, atol=1e-13)


def test_bad_arguments_are_rejected():
    H, C, E, off, tok = _instance(41)
    bad = tok.copy()
    bad[3] = bad[4]                                    # a token listed twice: not a partition
    with pytest.raises(oracle.OracleError):
        oracle.cluster_propose(H, C, E, off, bad, 2, 1.0)
    with pytest.raises(oracle.OracleError):
        oracle.cluster_propose(H, C, E, off, tok, off.size, 1.0)   # K_c > N_c
    empty = off.copy()
    empty[1] = empty[0]                                # cluster 0 holds no token
    with pytest.raises(oracle.OracleError):
        oracle.cluster_propose(H, C, E, empty, tok, 2, 1.0)
    o = oracle.cluster_propose(H, C, E, off, tok, 3, 1.0)
    sel = o["sel"].copy()
    sel[0, 0] = sel[0, 0][::-1]                        # not ascending
    Lt = np.zeros((H.shape[0], H.shape[1] + 1, E.shape[0]), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.cluster_verify(H, E, off, tok, sel, o["x"], Lt, 1.0)
