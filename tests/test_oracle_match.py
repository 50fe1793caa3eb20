"""Pins of the oracle's cache match: a hand-worked table and the closed-form hit probability."""

import numpy as np
import pytest
from scipy import special

from oracle import match, packing, verify


def test_hand_worked_table():
    """B=4, C=3, F=2, anchors k=1 -> (10, 11), k=2 -> (20, 21), full accept -> 30."""
    blocks = packing.pack_blocks(4, 3, 2, 99, [10, 11, 20, 21, 30])
    table = {
        (0, 10): 1, (0, 11): 2, (0, 20): -1,
        (1, 20): 3, (1, 21): 4, (1, 10): -1,
        (2, 20): -1,                      # rejection at position 3 = C is not covered
        (3, 30): 5, (3, 31): -1,          # full accept: bonus token against the full-accept anchor
        (0, 99): -1,                      # block 0 is never a branch
    }
    for (n_acc, tok), want in table.items():
        assert match.match_request(blocks, n_acc, tok) == want


def test_duplicate_anchor_first_branch_wins():
    blocks = packing.pack_blocks(4, 3, 2, 0, [10, 10, 20, 20, 30])
    assert match.match_request(blocks, 0, 10) == 1
    assert match.match_request(blocks, 1, 20) == 3


def test_hit_rate_closed_form():
    """P(hit) = sum_{k=1}^{C-1} S(k-1)(1-alpha_{k-1}) sum_{g in anchors_k} r_{k-1}(g)/Z_{k-1}
                + S(B-1) P_{B-1}(g_full), with 0-based rows and S(0) = 1, computed from library
    softmaxes, against the empirical hit rate of oracle verify + match over Philox rounds."""
    rng = np.random.default_rng(21)
    B, C, F, V = 5, 4, 2, 10
    zp = rng.normal(0, 1.0, size=(B, V))
    zq = zp[:B - 1] + rng.normal(0, 0.6, size=(B - 1, V))
    q_lib = special.softmax(zq, axis=-1)
    p_lib = special.softmax(zp, axis=-1)
    y = np.array([int(np.argmax(q_lib[j])) for j in range(B - 1)])
    anchors = []
    for k in range(1, C):
        order = [v for v in np.argsort(-zq[k - 1], kind="stable") if v != y[k - 1]]
        anchors += [int(v) for v in order[:F]]
    anchors.append(int(np.argmax(zp[B - 1])))
    blocks = packing.pack_blocks(B, C, F, 0, anchors)

    alpha = np.minimum(1.0, p_lib[np.arange(B - 1), y] / q_lib[np.arange(B - 1), y])
    S = np.concatenate([[1.0], np.cumprod(alpha)])
    closed = 0.0
    for k in range(1, C):
        r = np.maximum(0.0, p_lib[k - 1] - q_lib[k - 1])
        closed += S[k - 1] * (1 - alpha[k - 1]) * sum(r[g] for g in anchors[(k - 1) * F:k * F]) / r.sum()
    closed += S[B - 1] * p_lib[B - 1][anchors[-1]]

    n = 30000
    hits = 0
    for rnd in range(n):
        out = verify.verify_request(zp, zq, y, 1.0, seed=0x5EED, round_=rnd)
        hits += match.match_request(blocks, out.n_accepted, out.next_token) >= 0
    rate = hits / n
    assert 0.05 < closed < 0.95
    assert abs(rate - closed) < 4 * np.sqrt(closed * (1 - closed) / n)
