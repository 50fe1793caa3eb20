"""Planted mistakes: each plausible error in the oracle must make at least one of its pins fail.

Every case below replaces one oracle function (in the oracle module itself, for the duration of the
case) with a copy that carries a single mistake -- a swapped operand, an off-by-one, a wrong index or
constant -- and runs the pins that are meant to catch it. The case passes when some pin raises an
AssertionError; a mistake that every pin accepts would mean the pins do not fix that part of the
oracle."""

import numpy as np
import pytest

import test_oracle_attention as t_attn
import test_oracle_awl as t_awl
import test_oracle_commit as t_commit
import test_oracle_match as t_match
import test_oracle_packing as t_pack
import test_oracle_philox as t_philox
import test_oracle_select as t_select
import test_oracle_train_attn as t_train
import test_oracle_verify as t_ver
from conftest import golden_rows
from oracle import attention, awl, commit, match, packing, philox, select, train_attn, verify


# ------------------------------------------------------------------------------------------------
# the mutants (each a copy of one oracle function with one mistake)
# ------------------------------------------------------------------------------------------------

def alpha_q_over_p(z_target, z_draft, tokens, temperature):
    """alpha = min(1, Q/P): target and draft swapped."""
    tokens = np.asarray(tokens, dtype=np.int64)
    n = tokens.size
    if verify.as_temperature(temperature) == 0.0:
        return np.array([float(verify.greedy_argmax(z_target[j]) == tokens[j]) for j in range(n)])
    rows = np.arange(n)
    p = verify.row_softmax(np.asarray(z_target)[:n], temperature)[rows, tokens]
    q = verify.row_softmax(z_draft, temperature)[rows, tokens]
    return np.minimum(1.0, q / p)


def residual_abs(z_target_row, z_draft_row, temperature):
    """|P - Q| instead of max(0, P - Q)."""
    return np.abs(verify.row_softmax(z_target_row, temperature) - verify.row_softmax(z_draft_row, temperature))


def first_rejection_flipped(alpha, u):
    """Accept while u >= alpha."""
    for j, (a, uj) in enumerate(zip(alpha, u)):
        if uj < a:
            return j
    return len(alpha)


def inverse_cdf_exclusive(r, u):
    """C(v) >= u Z instead of C(v) > u Z."""
    r = np.asarray(r, dtype=np.float64)
    c = np.cumsum(r)
    z = float(c[-1])
    hits = np.nonzero(c >= u * z)[0]
    v = int(hits[0]) if hits.size else int(np.nonzero(r > 0)[0][-1])
    return v, z, float(c[v]), float(c[v - 1]) if v > 0 else 0.0


def survival_inclusive_shift(alpha):
    """tau = 1 + sum of S(k) with the product starting one row late."""
    s = np.cumprod(np.concatenate([[1.0], np.asarray(alpha, dtype=np.float64)[1:]]))
    return s, 1.0 + float(s.sum())


def _mask_with(slice_extra=0, causal_extra=0):
    def visible_mask(B, blocks, prefix_len):
        n_q = len(blocks) * B
        L = int(prefix_len)
        mask = np.zeros((n_q, L + n_q), dtype=bool)
        mask[:, :L] = True
        for b, (r, _anchor, causal) in enumerate(blocks):
            own = L + b * B
            for i in range(B):
                t = b * B + i
                if b >= 1 and r > 0:
                    mask[t, L:L + min(r + slice_extra, B)] = True
                if causal:
                    mask[t, own:own + min(i + 1 + causal_extra, B)] = True
                else:
                    mask[t, own:own + B] = True
        return mask
    return visible_mask


def packed_attention_round_robin(q, k_prefix, v_prefix, k_new, v_new, mask, scale, rows=None):
    """Query head h reads key/value head h mod H_kv instead of h // (H_q / H_kv)."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.concatenate([np.asarray(k_prefix, np.float64), np.asarray(k_new, np.float64)], axis=0)
    vals = np.concatenate([np.asarray(v_prefix, np.float64), np.asarray(v_new, np.float64)], axis=0)
    n_q, h_q, d = q.shape
    h_kv = keys.shape[1]
    sel = np.arange(n_q) if rows is None else np.asarray(list(rows), dtype=np.int64)
    out = np.empty((sel.size, h_q, d))
    m = mask[sel]
    for h in range(h_q):
        g = h % h_kv
        s = np.where(m, (q[sel, h, :] @ keys[:, g, :].T) * float(scale), -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (p / p.sum(axis=1, keepdims=True)) @ vals[:, g, :]
    return out


def philox_weyl_swapped(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 with the two key-schedule increments exchanged."""
    m32 = np.uint64(0xFFFFFFFF)
    x0, x1, x2, x3 = (a.copy() for a in np.broadcast_arrays(*[np.asarray(c, dtype=np.uint64) & m32
                                                              for c in (c0, c1, c2, c3)]))
    k0, k1 = np.uint64(int(k0) & 0xFFFFFFFF), np.uint64(int(k1) & 0xFFFFFFFF)
    ma, mb = np.uint64(philox.PHILOX_M4x32[0]), np.uint64(philox.PHILOX_M4x32[1])
    wa, wb = np.uint64(philox.PHILOX_W32[1]), np.uint64(philox.PHILOX_W32[0])
    for _ in range(10):
        p0, p1 = ma * x0, mb * x2
        x0, x1, x2, x3 = ((p1 >> np.uint64(32)) ^ x1 ^ k0, p1 & m32, (p0 >> np.uint64(32)) ^ x3 ^ k1, p0 & m32)
        k0, k1 = (k0 + wa) & m32, (k1 + wb) & m32
    return tuple(a.astype(np.uint32) for a in (x0, x1, x2, x3))


def uniform53_words_swapped(x0, x1):
    """The 27 high bits taken from word 1 and the 26 low bits from word 0."""
    hi = np.asarray(x1, dtype=np.uint64) >> np.uint64(5)
    lo = np.asarray(x0, dtype=np.uint64) >> np.uint64(6)
    return (hi.astype(np.float64) * 67108864.0 + lo.astype(np.float64)) * (2.0 ** -53)


def uniforms_counter_swapped(seed, position, request, round_, purpose):
    """Counter words (request, position, ...) instead of (position, request, ...)."""
    seed = int(seed)
    x0, x1, _, _ = philox.philox4x32_10(request, position, round_, purpose, seed & 0xFFFFFFFF,
                                        (seed >> 32) & 0xFFFFFFFF)
    return philox.uniform53(x0, x1)


def uniforms_key_swapped(seed, position, request, round_, purpose):
    """Key words (high, low) instead of (low, high)."""
    seed = int(seed)
    x0, x1, _, _ = philox.philox4x32_10(position, request, round_, purpose, (seed >> 32) & 0xFFFFFFFF,
                                        seed & 0xFFFFFFFF)
    return philox.uniform53(x0, x1)


def awl_weights_inclusive(alpha):
    """w_k = prod_{j<=k} alpha_j: the position's own score included."""
    return np.cumprod(np.asarray(alpha, dtype=np.float64))


def match_last(blocks, n_accepted, next_token):
    """The last hit branch in pack order instead of the first."""
    found = -1
    for b in range(1, len(blocks)):
        r, anchor, _causal = blocks[b]
        if r == n_accepted + 1 and anchor == next_token:
            found = b
    return found


def match_rejection_index(blocks, n_accepted, next_token):
    """r = n_accepted instead of n_accepted + 1."""
    for b in range(1, len(blocks)):
        r, anchor, _causal = blocks[b]
        if r == n_accepted and anchor == next_token:
            return b
    return -1


def topk_ties_high(row, k, exclude=-1):
    """Ties go to the higher token id."""
    z = np.asarray(row, dtype=np.float64)
    z = np.where(np.isnan(z), -np.inf, z)
    order = np.lexsort((-np.arange(z.size), -z))
    order = order[order != exclude][:k]
    out = np.full(k, -1, dtype=np.int64)
    out[:order.size] = order
    return out


def train_mask_anchor_inclusive(L, anchors, B):
    """A block also sees the response token at its anchor position."""
    anchors = [int(a) for a in anchors]
    n = train_attn.n_rows(L, len(anchors), B)
    mask = np.zeros((n, n), dtype=bool)
    for p in range(L):
        mask[p, :p + 1] = True
    for i, a in enumerate(anchors):
        r0 = L + i * B
        mask[r0:r0 + B, :min(a + 1, L)] = True
        mask[r0:r0 + B, r0:r0 + B] = True
    return mask


def kv_commit_short(k_new, v_new, k_cache, v_cache, page_table, req_block_off, prefix_len, n_accepted, B):
    """Commits n_accepted rows (the anchor's row forgotten at the end of the slice)."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    page_size = kc.shape[1]
    new_len = np.array(prefix_len, dtype=np.int64, copy=True)
    for i in range(len(n_accepted)):
        n = min(max(int(n_accepted[i]), 0), B - 1)
        for j in range(n):
            t = int(prefix_len[i]) + j
            page = int(page_table[i, t // page_size])
            kc[page, t % page_size] = k_new[int(req_block_off[i]) * B + j]
            vc[page, t % page_size] = v_new[int(req_block_off[i]) * B + j]
        new_len[i] = int(prefix_len[i]) + n
    return kc, vc, new_len, np.zeros(len(n_accepted), dtype=np.int64)


# ------------------------------------------------------------------------------------------------
# cases: (name, module, attribute, mutant, pins)
# ------------------------------------------------------------------------------------------------

def _golden(name):
    return golden_rows(name)


CASES = [
    ("P and Q swapped in alpha", verify, "acceptance_ratios", alpha_q_over_p,
     [lambda: t_ver.test_expected_alpha_is_overlap_mass(), lambda: t_ver.test_lossless_brute_force(3, 5, 0.75, 1)]),
    ("residual |P - Q|", verify, "residual_mass", residual_abs,
     [lambda: t_ver.test_residual_token_differs_from_rejected_draft(),
      lambda: t_ver.test_lossless_brute_force(3, 5, 0.75, 1)]),
    ("acceptance test flipped", verify, "first_rejection", first_rejection_flipped,
     [lambda: t_ver.test_equal_distributions_accept_everything(),
      lambda: t_ver.test_tau_is_mean_acceptance_length_monte_carlo()]),
    ("inverse CDF not inclusive", verify, "inverse_cdf", inverse_cdf_exclusive,
     [lambda: t_ver.test_inverse_cdf_edges()]),
    ("survival product shifted", verify, "survival", survival_inclusive_shift,
     [lambda: t_ver.test_tau_is_mean_acceptance_length_monte_carlo(),
      lambda: t_ver.test_equal_distributions_accept_everything()]),
    ("accepted slice one row too long", packing, "visible_mask", _mask_with(slice_extra=1),
     [lambda: t_pack.test_hand_derived_mask(), lambda: t_pack.test_visible_pair_count_closed_form(63)]),
    ("causal block sees the next row", packing, "visible_mask", _mask_with(causal_extra=1),
     [lambda: t_pack.test_hand_derived_mask(), lambda: t_pack.test_visible_pair_count_closed_form(63)]),
    ("query heads grouped round-robin", attention, "packed_attention", packed_attention_round_robin,
     [lambda: t_attn.test_packed_matches_masked_library_attention_gqa()]),
    ("Philox key increments exchanged", philox, "philox4x32_10", philox_weyl_swapped,
     [lambda: t_philox.test_known_answer_vectors(_golden), lambda: t_philox.test_vectorised_matches_scalar()]),
    ("uniform built from the words in the wrong order", philox, "uniform53", uniform53_words_swapped,
     [lambda: t_philox.test_uniform53_grid_and_range()]),
    ("Philox counter words in the wrong order", philox, "uniforms", uniforms_counter_swapped,
     [lambda: t_philox.test_uniforms_layout_against_known_answers(_golden)]),
    ("Philox key words in the wrong order", philox, "uniforms", uniforms_key_swapped,
     [lambda: t_philox.test_uniforms_layout_against_known_answers(_golden)]),
    ("AWL weight includes its own position", awl, "awl_weights", awl_weights_inclusive,
     [lambda: t_awl.test_weights_are_the_verify_survival_products(), lambda: t_awl.test_hand_worked_block()]),
    ("match takes the last branch", match, "match_request", match_last,
     [lambda: t_match.test_duplicate_anchor_first_branch_wins()]),
    ("match off by one in the rejection position", match, "match_request", match_rejection_index,
     [lambda: t_match.test_hand_worked_table(), lambda: t_match.test_hit_rate_closed_form()]),
    ("top-k ties to the higher id", select, "topk", topk_ties_high,
     [lambda: t_select.test_topk_equals_pairwise_rank(0), lambda: t_select.test_k1_is_first_argmax()]),
    ("training block sees its anchor position", train_attn, "visible_mask", train_mask_anchor_inclusive,
     [lambda: t_train.test_visibility_table_by_hand()]),
    ("commit one row short", commit, "kv_commit", kv_commit_short,
     [lambda: t_commit.test_cache_reads_back_as_prefix_then_accepted_rows(0)]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_planted_mistake_fails_a_pin(case, monkeypatch):
    name, module, attr, mutant, pins = case
    assert callable(getattr(module, attr))
    monkeypatch.setattr(module, attr, mutant)
    caught = []
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught.append(pin)
    assert caught, f"no pin fails with the planted mistake: {name}"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pins_pass_without_the_mistake(case):
    """The same pins pass on the oracle as it stands (so a failure above is the mistake's doing)."""
    for pin in case[4]:
        pin()
