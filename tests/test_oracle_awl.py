"""Pins of the AWL oracle (oracle/awl.py): weights against the verify oracle's survival products,
the P = Q closed form (every weight 1: the plain mean cross-entropy), the all-excluded case (0/eps),
a hand-worked block, and the analytic gradient against central finite differences of the loss with
the weights held fixed (the stop-gradient)."""

import numpy as np
import pytest

from oracle import awl, verify


def _problem(rng, n_blocks=3, n_pos=4, V=6):
    zt = rng.normal(0, 1.5, size=(n_blocks, n_pos, V))
    zd = zt + rng.normal(0, 1.0, size=zt.shape)
    tok = rng.integers(0, V, size=(n_blocks, n_pos))
    lab = rng.integers(0, V, size=(n_blocks, n_pos))
    inc = rng.random((n_blocks, n_pos)) < 0.8
    return zt, zd, tok, lab, inc


def test_weights_are_the_verify_survival_products():
    rng = np.random.default_rng(0)
    zt, zd, tok, lab, inc = _problem(rng)
    out = awl.awl_loss(zt, zd, tok, lab, inc)
    for r in range(zt.shape[0]):
        alpha = verify.acceptance_ratios(zt[r], zd[r], tok[r], 1.0)
        s, _tau = verify.survival(alpha)  # S(k) = prod_{j<k} alpha_j for k = 1..n
        np.testing.assert_allclose(out["weights"][r], np.concatenate([[1.0], s[:-1]]), rtol=0, atol=0)


def test_equal_distributions_give_the_mean_cross_entropy():
    rng = np.random.default_rng(1)
    zt, _zd, tok, lab, inc = _problem(rng)
    out = awl.awl_loss(zt, zt, tok, lab, inc)
    assert (out["weights"] == 1.0).all()
    p = np.exp(zt - zt.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    ce = -np.log(np.take_along_axis(p, lab[..., None], -1)[..., 0])
    assert out["loss"] == pytest.approx(ce[inc].sum() / (inc.sum() + 1e-6), rel=1e-12)


def test_nothing_included_gives_zero():
    rng = np.random.default_rng(2)
    zt, zd, tok, lab, _ = _problem(rng)
    out = awl.awl_loss(zt, zd, tok, lab, np.zeros(tok.shape, bool))
    assert out["loss"] == 0.0 and (out["grad"] == 0).all()


def test_hand_worked_block():
    # one block, two positions, V = 2. Position 0: P = softmax(0, ln 3) = (1/4, 3/4), Q = (1/2, 1/2),
    # draft token 1: alpha_0 = min(1, (3/4)/(1/2)) = 1. Position 1: P = (1/2, 1/2), Q = softmax(0, ln 3),
    # draft token 1: alpha_1 = (1/2)/(3/4) = 2/3 (not used: weights are w_0 = 1, w_1 = alpha_0 = 1).
    zt = np.array([[[0.0, np.log(3)], [0.0, 0.0]]])
    zd = np.array([[[0.0, 0.0], [0.0, np.log(3)]]])
    out = awl.awl_loss(zt, zd, np.array([[1, 1]]), np.array([[0, 1]]))
    np.testing.assert_allclose(out["weights"], [[1.0, 1.0]])
    np.testing.assert_allclose(out["ce"], [[np.log(2), np.log(4 / 3)]])
    assert out["loss"] == pytest.approx((np.log(2) + np.log(4 / 3)) / (2 + 1e-6), rel=1e-14)
    # flip the first draft token: alpha_0 = (1/4)/(1/2) = 1/2, so w_1 = 1/2
    out = awl.awl_loss(zt, zd, np.array([[0, 1]]), np.array([[0, 1]]))
    np.testing.assert_allclose(out["weights"], [[1.0, 0.5]])


def test_gradient_matches_finite_differences_with_weights_held():
    rng = np.random.default_rng(3)
    zt, zd, tok, lab, inc = _problem(rng, n_blocks=2, n_pos=3, V=5)
    out = awl.awl_loss(zt, zd, tok, lab, inc)
    w = out["weights"]

    def loss_fixed_w(z):
        p = np.exp(z - z.max(-1, keepdims=True))
        p /= p.sum(-1, keepdims=True)
        ce = -np.log(np.take_along_axis(p, lab[..., None], -1)[..., 0])
        return float(np.sum(inc * w * ce) / (np.sum(inc * w) + 1e-6))

    h = 1e-6
    num = np.zeros_like(zd)
    for idx in np.ndindex(zd.shape):
        zp, zm = zd.copy(), zd.copy()
        zp[idx] += h
        zm[idx] -= h
        num[idx] = (loss_fixed_w(zp) - loss_fixed_w(zm)) / (2 * h)
    np.testing.assert_allclose(out["grad"], num, atol=1e-8)
