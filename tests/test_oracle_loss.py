"""Pins of the oracle's training-side loss (DSpark page, section 9).

Per drafted position, teacher-forced on the labels y (the bias of position k
uses y_{k-1}, y_0 = the anchor): ce = -log p_d(y_k), l1 = ||p_d - p_t||_1,
bce = BCE-with-logits(q, c*); weights w_k = exp(-(k-1)/gamma); the loss is
the weighted mean of a_ce ce + a_tv l1 + a_conf bce.  Pinned by
  - the cross-entropy against scipy's log-softmax of the draft logits
    (U plus the separately pinned bias of the previous label);
  - l1 = 2 (1 - c*) against the oracle's confidence labels for the same
    tokens, and l1 = 0, c* = 1 (so bce = softplus(-q)) for identical rows;
  - dq against central finite differences of the loss in q;
  - linearity in the coefficients and the weights w_1 = 1, w_2 = e^-1/2.
"""
import numpy as np
import pytest
from scipy.special import log_softmax

import oracle


def _instance(seed, R=3, g=4, V=97, r=16, T=0.8):
    rng = np.random.default_rng(seed)
    U = rng.normal(0, 2, (R, g, V)).astype(np.float32)
    Lt = (np.concatenate([U, rng.normal(0, 2, (R, 1, V))], axis=1) + rng.normal(0, 0.7, (R, g + 1, V))).astype(np.float32)
    W1 = rng.normal(0, 0.2, (V, r)).astype(np.float32)
    W2 = rng.normal(0, 0.2, (V, r)).astype(np.float32)
    x0 = rng.integers(0, V, R).astype(np.int32)
    y = rng.integers(0, V, (R, g)).astype(np.int32)
    q = rng.normal(0, 1.5, (R, g)).astype(np.float32)
    return U, W1, W2, x0, y, Lt, q, T


def test_cross_entropy_matches_scipy_log_softmax():
    U, W1, W2, x0, y, Lt, q, T = _instance(1)
    o = oracle.draft_loss(U, W1, W2, x0, y, Lt, q, T)
    R, g, V = U.shape
    for r in range(R):
        prev = x0[r]
        for k in range(g):
            z = U[r, k].astype(np.float64) + oracle.bias(W1, W2, prev)
            want = -log_softmax(z / float(np.float32(T)))[y[r, k]]    # T passes as fp32
            assert o["terms"][r, k, 0] == pytest.approx(want, rel=1e-12)
            prev = y[r, k]


def test_l1_is_twice_one_minus_confidence_label():
    U, W1, W2, x0, y, Lt, q, T = _instance(2)
    o = oracle.draft_loss(U, W1, W2, x0, y, Lt, q, T)
    cs, _ = oracle.confidence(U, W1, W2, x0, y, Lt, np.float32(T))
    np.testing.assert_allclose(o["terms"][..., 1], 2.0 * (1.0 - cs), rtol=0, atol=1e-12)


def test_identical_rows_give_zero_l1_and_softplus_bce():
    U, W1, W2, x0, y, Lt, q, T = _instance(3)
    W2 = np.zeros_like(W2)                     # draft logits = U
    Lt[:, :-1] = U                             # target row k-1 = draft row k
    o = oracle.draft_loss(U, W1, W2, x0, y, Lt, q, T)
    np.testing.assert_allclose(o["terms"][..., 1], 0.0, atol=1e-13)
    np.testing.assert_allclose(o["terms"][..., 2], np.log1p(np.exp(-q.astype(np.float64))), rtol=1e-12)


def test_dq_matches_finite_differences():
    U, W1, W2, x0, y, Lt, q, T = _instance(4)
    o = oracle.draft_loss(U, W1, W2, x0, y, Lt, q, T)
    eps = 1e-3
    for (r, k) in [(0, 0), (1, 2), (2, 3)]:
        qp, qm = q.copy(), q.copy()
        qp[r, k] += eps
        qm[r, k] -= eps
        fd = (oracle.draft_loss(U, W1, W2, x0, y, Lt, qp, T)["loss"] -
              oracle.draft_loss(U, W1, W2, x0, y, Lt, qm, T)["loss"]) / (float(qp[r, k]) - float(qm[r, k]))
        assert o["dq"][r, k] == pytest.approx(fd, rel=1e-5, abs=1e-9)


def test_linearity_and_position_weights():
    U, W1, W2, x0, y, Lt, q, T = _instance(5)
    parts = [oracle.draft_loss(U, W1, W2, x0, y, Lt, q, T, alphas=a)["loss"]
             for a in ((1, 0, 0), (0, 1, 0), (0, 0, 1))]
    both = oracle.draft_loss(U, W1, W2, x0, y, Lt, q, T, alphas=(0.1, 0.9, 1.0))["loss"]
    a_ce, a_tv = float(np.float32(0.1)), float(np.float32(0.9))   # the coefficients pass as fp32
    assert both == pytest.approx(a_ce * parts[0] + a_tv * parts[1] + parts[2], rel=1e-12)
    # one request, two positions: weights 1 and e^-1/2
    U2, W12, W22, x02, y2, Lt2, q2, _ = _instance(6, R=1, g=2)
    o = oracle.draft_loss(U2, W12, W22, x02, y2, Lt2, q2, T, alphas=(1, 0, 0))
    t = o["terms"][0, :, 0]
    w2 = np.exp(-0.5)
    assert o["loss"] == pytest.approx((t[0] + w2 * t[1]) / (1 + w2), rel=1e-12)


def test_uniform_draft_has_log_v_cross_entropy():
    U, W1, W2, x0, y, Lt, q, T = _instance(7)
    U[:] = 0.25
    W2 = np.zeros_like(W2)
    o = oracle.draft_loss(U, W1, W2, x0, y, Lt, q, T)
    np.testing.assert_allclose(o["terms"][..., 0], np.log(U.shape[2]), rtol=1e-13)


def test_bad_label_is_rejected():
    U, W1, W2, x0, y, Lt, q, T = _instance(8)
    y[1, 2] = U.shape[2]
    with pytest.raises(oracle.OracleError):
        oracle.draft_loss(U, W1, W2, x0, y, Lt, q, T)
