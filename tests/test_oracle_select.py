"""Pins of the oracle's token selection (oracle/select.py) to what the pages and the definition fix,
by routes other than sorting: pairwise counting on small rows, NumPy's first-occurrence argmax, a
hand-worked row, and the invariant that ties the anchors to the verify step (the residual is zero at
the rejected draft token)."""

import numpy as np
import pytest

from oracle import select, verify


def _beats(z, a, b):
    return z[a] > z[b] or (z[a] == z[b] and a < b)


@pytest.mark.parametrize("seed", range(6))
def test_topk_equals_pairwise_rank(seed):
    """Token t is the i-th output exactly when i other candidates beat it (larger logit, or equal
    logit and lower id): a counting definition, no sort."""
    rng = np.random.default_rng(seed)
    V = int(rng.integers(1, 40))
    z = rng.integers(-3, 4, size=V).astype(np.float64)  # many ties
    if seed % 2:
        z[rng.integers(0, V)] = -np.inf
    ex = int(rng.integers(-1, V))
    k = int(rng.integers(1, 9))
    got = select.topk(z, k, exclude=ex)
    cands = [t for t in range(V) if t != ex]
    rank = {t: sum(_beats(z, u, t) for u in cands if u != t) for t in cands}
    want = [next(t for t in cands if rank[t] == i) for i in range(min(k, len(cands)))]
    assert got[:len(want)].tolist() == want
    assert (got[len(want):] == -1).all()


def test_k1_is_first_argmax():
    rng = np.random.default_rng(1)
    for _ in range(50):
        z = rng.integers(0, 5, size=int(rng.integers(1, 300))).astype(np.float32)
        assert select.topk(z, 1)[0] == int(np.argmax(z))


def test_hand_worked_row():
    # logits by id: 0:3, 1:7, 2:7, 3:1, 4:7, 5:-inf, 6:9; excluding id 1
    z = [3, 7, 7, 1, 7, -np.inf, 9]
    assert select.topk(z, 4, exclude=1).tolist() == [6, 2, 4, 0]
    assert select.topk(z, 8, exclude=1).tolist() == [6, 2, 4, 0, 3, 5, -1, -1]
    assert select.topk([np.nan, -np.inf], 2).tolist() == [0, 1]  # NaN counts as -inf, tie to the lower id


def test_anchor_is_never_the_rejected_draft_and_replacements_come_from_outside_it():
    """The excluded token is the rejected draft d_k. A rejection at k is possible only when
    alpha = P(d_k)/Q(d_k) < 1, and then the residual max(0, P - Q) is zero at d_k -- so d_k is never
    the replacement, and an anchor equal to it could never hit."""
    rng = np.random.default_rng(4)
    B, V, C, F = 6, 12, 4, 2
    zt = rng.normal(0, 1.5, size=(B, V))
    zd = zt[:B - 1] + rng.normal(0, 1.0, size=(B - 1, V))
    tok = np.array([int(np.argmax(zd[j])) for j in range(B - 1)])
    anchors = select.alt_anchors(zd, tok, rng.normal(size=V), C, F)
    assert anchors.size == (C - 1) * F + 1
    alpha = verify.acceptance_ratios(zt, zd, tok, 1.0)
    rejectable = 0
    for k in range(1, C):
        assert tok[k - 1] not in anchors[(k - 1) * F:k * F]
        if alpha[k - 1] < 1.0:
            rejectable += 1
            assert verify.residual_mass(zt[k - 1], zd[k - 1], 1.0)[tok[k - 1]] == 0.0
    assert rejectable > 0


def test_sampled_drafting_follows_the_softmax():
    """Gumbel-max over the counter-based uniforms draws from softmax(z / T): the token frequencies
    over 40000 rows (row indexes 0..39999) match the probabilities (chi-square, 5 cells)."""
    from oracle import select as sel
    z = np.array([1.0, 0.2, -0.5, 2.0, 0.0])
    T = 0.8
    p = np.exp(z / T) / np.exp(z / T).sum()
    n = 40000
    counts = np.bincount([sel.sample_token(z, T, 0x5EED, 3, r) for r in range(n)], minlength=5)
    chi2 = float(((counts - n * p) ** 2 / (n * p)).sum())
    assert chi2 < 20.5  # 4 degrees of freedom: p < 0.0004 under the right law


def test_sampled_drafting_special_cases():
    from oracle import select as sel
    from oracle import philox
    # the uniform map stays inside (0, 1) at the extreme words
    assert 0.0 < float(philox.uniform24(0)) and float(philox.uniform24(0xFFFFFFFF)) < 1.0
    # a very low temperature gives the argmax; -inf and NaN logits are never drawn
    z = np.array([0.1, 3.0, 2.9, -np.inf, np.nan])
    assert all(sel.sample_token(z, 1e-4, 7, 0, r) == 1 for r in range(50))
    draws = {sel.sample_token(z, 5.0, 7, 0, r) for r in range(300)}
    assert draws <= {0, 1, 2} and len(draws) == 3
    # the same counter draws the same token; another row index draws independently
    assert sel.sample_token(z, 1.0, 9, 4, 11) == sel.sample_token(z, 1.0, 9, 4, 11)
    # the scores are z / T plus a standard Gumbel variable: mean Euler's constant over many tokens
    g = sel.gumbel_scores(np.zeros(200000), 1.0, 1, 0, 0)
    assert abs(g.mean() - 0.5772156649) < 0.01 and abs(g.var() - np.pi ** 2 / 6) < 0.03
