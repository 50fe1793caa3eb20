"""Pins of the oracle's verification: losslessness by brute force, closed forms, special cases.

The reference distributions below come from scipy.special.softmax, not from the oracle."""

import itertools
from collections import defaultdict

import numpy as np
import pytest
from scipy import special, stats

from oracle import philox, verify


def _logits(rng, B, V, noise=0.7, scale=1.5):
    zp = rng.normal(0, scale, size=(B, V))
    zq = zp[:B - 1] + rng.normal(0, noise, size=(B - 1, V))
    return zp, zq


def _emission_law(zp, zq, T):
    """Exact law of the emitted tokens (accepted drafts + resampled/bonus token) of the oracle,
    integrating the draft y ~ prod Q_j, every acceptance uniform and the sampling uniform."""
    B, V = zp.shape
    nd = B - 1
    q_lib = special.softmax(zq / T, axis=-1)
    law = defaultdict(float)
    for y in itertools.product(range(V), repeat=nd):
        wy = float(np.prod([q_lib[j, y[j]] for j in range(nd)]))
        alpha = verify.verify_request(zp, zq, y, T, u_accept=np.zeros(nd), u_sample=0.0).alpha
        for pattern in itertools.product((True, False), repeat=nd):
            w = float(np.prod([alpha[j] if acc else 1.0 - alpha[j] for j, acc in enumerate(pattern)]))
            if w == 0.0:
                continue
            u = np.array([alpha[j] / 2 if acc else (1.0 + alpha[j]) / 2 for j, acc in enumerate(pattern)])
            first = verify.verify_request(zp, zq, y, T, u_accept=u, u_sample=0.0)
            c = np.cumsum(first.sample_mass) / first.sample_mass.sum()
            for v in np.nonzero(first.sample_mass > 0)[0]:
                lo = c[v - 1] if v > 0 else 0.0
                out = verify.verify_request(zp, zq, y, T, u_accept=u, u_sample=(lo + c[v]) / 2)
                assert out.next_token == v
                assert out.n_accepted == first.n_accepted
                law[tuple(y[:out.n_accepted]) + (int(v),)] += wy * w * (c[v] - lo)
    return law


@pytest.mark.parametrize("B,V,T,seed", [(4, 4, 1.0, 0), (3, 5, 0.75, 1), (2, 6, 1.0, 2), (4, 3, 1.25, 3)])
def test_lossless_brute_force(B, V, T, seed):
    """Each emitted token, given the emitted tokens before it, follows the target row P_j."""
    zp, zq = _logits(np.random.default_rng(seed), B, V)
    law = _emission_law(zp, zq, T)
    p_lib = special.softmax(zp / np.float64(np.float32(T)), axis=-1)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    for j in range(B):
        by_prefix = defaultdict(lambda: np.zeros(V))
        for seq, mass in law.items():
            if len(seq) > j:
                by_prefix[seq[:j]][seq[j]] += mass
        assert by_prefix
        for s, mass in by_prefix.items():
            np.testing.assert_allclose(mass / mass.sum(), p_lib[j], rtol=0, atol=1e-12)


def test_equal_distributions_accept_everything():
    """P = Q gives alpha = 1 on every row, n_accepted = B-1 and tau = B."""
    rng = np.random.default_rng(7)
    B, V = 16, 300
    zp = rng.normal(0, 2, size=(B, V))
    zq = zp[:B - 1].copy()
    y = rng.integers(0, V, size=B - 1)
    for r in range(20):
        out = verify.verify_request(zp, zq, y, 1.0, seed=11, round_=r)
        assert np.all(out.alpha == 1.0)
        assert out.n_accepted == B - 1
        assert out.tau == float(B)
        np.testing.assert_array_equal(out.survival, np.ones(B - 1))


def test_bonus_follows_last_target_row_when_all_accepted():
    rng = np.random.default_rng(8)
    B, V = 4, 8
    zp = rng.normal(0, 1, size=(B, V))
    zq = zp[:B - 1].copy()
    y = rng.integers(0, V, size=B - 1)
    n = 20000
    tok = np.array([verify.verify_request(zp, zq, y, 1.0, seed=5, round_=r).next_token for r in range(n)])
    expect = special.softmax(zp[B - 1]) * n
    assert stats.chisquare(np.bincount(tok, minlength=V), expect).pvalue > 1e-3


def test_expected_alpha_is_overlap_mass():
    """E_{y ~ Q_j}[alpha_j(y)] = sum_v min(P_j(v), Q_j(v)) (the acceptance rate of one row)."""
    rng = np.random.default_rng(9)
    B, V = 3, 40
    zp, zq = _logits(rng, B, V, noise=1.0)
    p, q = special.softmax(zp, axis=-1), special.softmax(zq, axis=-1)
    for j in range(B - 1):
        exp_alpha = 0.0
        for v in range(V):
            y = np.zeros(B - 1, dtype=int)
            y[j] = v
            exp_alpha += q[j, v] * verify.acceptance_ratios(zp, zq, y, 1.0)[j]
        assert abs(exp_alpha - np.minimum(p[j], q[j]).sum()) < 1e-13


def test_tau_is_mean_acceptance_length_monte_carlo():
    """The mean of the realised n_accepted + 1 over Philox rounds matches tau = 1 + sum_k S(k)."""
    rng = np.random.default_rng(10)
    B, V = 8, 64
    zp, zq = _logits(rng, B, V, noise=0.8)
    y = np.array([rng.choice(V, p=special.softmax(zq[j])) for j in range(B - 1)])
    alpha = verify.acceptance_ratios(zp, zq, y, 1.0)
    _, tau = verify.survival(alpha)
    n = 100000
    u = philox.uniforms(0xBEEF, np.arange(B - 1)[None, :], 0, np.arange(n)[:, None], 0)
    lengths = np.array([verify.first_rejection(alpha, u[r]) + 1 for r in range(n)])
    assert abs(lengths.mean() - tau) < 4 * lengths.std() / np.sqrt(n)
    # the closed form of tau itself: 1 + sum_k prod_{j<k} alpha_j
    assert abs(tau - (1 + sum(np.prod(alpha[:k]) for k in range(1, B)))) < 1e-12


def test_residual_token_differs_from_rejected_draft():
    rng = np.random.default_rng(11)
    B, V = 8, 50
    seen = 0
    for trial in range(200):
        zp, zq = _logits(rng, B, V, noise=1.5)
        y = rng.integers(0, V, size=B - 1)
        out = verify.verify_request(zp, zq, y, 1.0, seed=3, round_=trial)
        if out.n_accepted < B - 1:
            seen += 1
            j = out.n_accepted
            assert out.next_token != y[j]
            p, q = special.softmax(zp[j]), special.softmax(zq[j])
            assert p[out.next_token] > q[out.next_token]
    assert seen > 100


def test_greedy_reduces_to_argmax():
    rng = np.random.default_rng(12)
    B, V = 16, 100
    for trial in range(50):
        zp = rng.normal(0, 1, size=(B, V))
        y = np.argmax(zp[:B - 1], axis=-1)
        cut = int(rng.integers(0, B))
        if cut < B - 1:
            y[cut] = (y[cut] + 1) % V
        out = verify.verify_request(zp, np.zeros((B - 1, V)), y, 0.0, seed=1, round_=trial)
        assert out.n_accepted == cut if cut < B - 1 else out.n_accepted == B - 1
        assert out.next_token == int(np.argmax(zp[out.n_accepted]))
        assert set(np.unique(out.alpha)) <= {0.0, 1.0}
        assert out.flags == 0


def test_greedy_ties_take_lowest_id():
    zp = np.zeros((2, 6))
    zp[1, [2, 4]] = 5.0
    zp[0, [1, 3]] = 2.0
    out = verify.verify_request(zp, np.zeros((1, 6)), [3], 0.0)
    assert out.n_accepted == 0 and out.next_token == 1
    out = verify.verify_request(zp, np.zeros((1, 6)), [1], 0.0)
    assert out.n_accepted == 1 and out.next_token == 2


def test_greedy_masked_row_has_no_token():
    """A target row of -inf logits has no most likely token: its draft is rejected and the emitted
    token is -1; a row with any finite logit keeps the first argmax among them."""
    zp = np.full((3, 5), -np.inf)
    zp[0, 2] = 1.0
    zp[2, [1, 4]] = -3.0
    out = verify.verify_request(zp, np.zeros((2, 5)), [2, 0], 0.0)
    assert out.n_accepted == 1 and out.next_token == -1
    assert list(out.alpha) == [1.0, 0.0]
    out = verify.verify_request(zp, np.zeros((2, 5)), [0, 0], 0.0)
    assert out.n_accepted == 0 and out.next_token == 2
    zp[1, 3] = -1e30
    out = verify.verify_request(zp, np.zeros((2, 5)), [2, 3], 0.0)
    assert out.n_accepted == 2 and out.next_token == 1


def test_flags_mark_near_threshold_draws():
    rng = np.random.default_rng(13)
    zp, zq = _logits(rng, 4, 20)
    y = np.array([1, 2, 3])
    alpha = verify.acceptance_ratios(zp, zq, y, 1.0)
    u = np.array([alpha[0] - 5e-7, 0.999999, 0.5])
    out = verify.verify_request(zp, zq, y, 1.0, u_accept=u, u_sample=0.3)
    assert out.flags & verify.FLAG_NEAR_ACCEPT
    assert np.all(alpha > 1e-3)
    out = verify.verify_request(zp, zq, y, 1.0, u_accept=alpha / 2, u_sample=0.3)
    assert out.n_accepted == 3
    assert not out.flags & verify.FLAG_NEAR_ACCEPT
    # sampling exactly on a cumulative boundary
    base = verify.verify_request(zp, zq, y, 1.0, u_accept=np.ones(3) * 0.999999999, u_sample=0.0)
    c = np.cumsum(base.sample_mass)
    edge = c[5] / c[-1]
    out = verify.verify_request(zp, zq, y, 1.0, u_accept=np.ones(3) * 0.999999999, u_sample=edge)
    assert out.flags & verify.FLAG_NEAR_SAMPLE


def test_inverse_cdf_edges():
    r = np.array([0.0, 0.25, 0.0, 0.5, 0.25, 0.0])
    assert verify.inverse_cdf(r, 0.0)[0] == 1
    assert verify.inverse_cdf(r, 0.25)[0] == 3      # inclusive C(1) = 0.25 is not > 0.25
    assert verify.inverse_cdf(r, 1.0 - 2**-53)[0] == 4
    assert verify.inverse_cdf(r, 0.9999)[0] == 4
