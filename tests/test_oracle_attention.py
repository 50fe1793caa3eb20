"""Pins of the oracle's packed attention against a library routine, closed forms and invariants."""

import numpy as np
import pytest
import torch

from oracle import attention, packing


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa(q, keys, vals, mask, scale):
    """torch's CPU scaled-dot-product attention in float64, grouped-query via enable_gqa."""
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]          # [1, Hq, n, d]
    tk = torch.from_numpy(keys).permute(1, 0, 2)[None]
    tv = torch.from_numpy(vals).permute(1, 0, 2)[None]
    tm = None if mask is None else torch.from_numpy(mask)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=tm, scale=scale, enable_gqa=tq.shape[1] != tk.shape[1])
    return out[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv,d,L", [(1, 1, 64, 128), (8, 2, 32, 37), (4, 4, 16, 0)])
def test_single_bidirectional_block_is_textbook_attention(hq, hkv, d, L):
    """A lone bidirectional block with r = 0 is plain attention of its B queries over [prefix; block]."""
    rng = np.random.default_rng(1)
    B = 16
    q, kn, vn = _rand(rng, B, hq, d), _rand(rng, B, hkv, d), _rand(rng, B, hkv, d)
    kp, vp = _rand(rng, L, hkv, d), _rand(rng, L, hkv, d)
    mask = packing.visible_mask(B, [(0, 1, False)], L)
    got = attention.packed_attention(q, kp, vp, kn, vn, mask, d ** -0.5)
    want = _sdpa(q, np.concatenate([kp, kn]), np.concatenate([vp, vn]), None, d ** -0.5)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_packed_matches_masked_library_attention_gqa():
    """Full async pack with grouped heads equals the library's masked GQA attention
    (the library groups consecutive query heads over one key/value head)."""
    rng = np.random.default_rng(2)
    B, C, F, L, hq, hkv, d = 8, 4, 2, 45, 8, 2, 32
    blocks = packing.pack_blocks(B, C, F, 0, [0] * ((C - 1) * F + 1))
    n = len(blocks) * B
    q, kn, vn = _rand(rng, n, hq, d), _rand(rng, n, hkv, d), _rand(rng, n, hkv, d)
    kp, vp = _rand(rng, L, hkv, d), _rand(rng, L, hkv, d)
    mask = packing.visible_mask(B, blocks, L)
    got = attention.packed_attention(q, kp, vp, kn, vn, mask, 0.3)
    want = _sdpa(q, np.concatenate([kp, kn]), np.concatenate([vp, vn]), mask, 0.3)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_zero_queries_average_visible_values_hand_mask():
    """q = 0 gives the mean of the visible values; with one-hot values per key the output row is
    the indicator of the visible set over its size (hand-derived sets at B=4, C=3, F=1, L=2)."""
    blocks = packing.pack_blocks(4, 3, 1, 9, [10, 20, 30])
    n, L = 16, 2
    keys = L + n
    q = np.zeros((n, 1, keys))
    kp = np.ones((L, 1, keys))
    kn = np.ones((n, 1, keys))
    eye = np.eye(keys)
    vp, vn = eye[:L, None, :], eye[L:, None, :]
    mask = packing.visible_mask(4, blocks, L)
    out = attention.packed_attention(q, kp, vp, kn, vn, mask, 1.0)[:, 0, :]
    row_sets = {0: [0, 1, 2], 7: [0, 1, 2, 6, 7, 8, 9], 9: [0, 1, 2, 3, 10, 11, 12, 13],
                15: [0, 1, 2, 3, 4, 5, 14, 15, 16, 17]}
    for t, vis in row_sets.items():
        want = np.zeros(keys)
        want[vis] = 1.0 / len(vis)
        np.testing.assert_allclose(out[t], want, atol=1e-15)


def test_branch_permutation_equivariance():
    """Permuting the branch blocks (and their rows) permutes the outputs the same way."""
    rng = np.random.default_rng(3)
    B, C, F, L, h, d = 4, 4, 2, 20, 2, 8
    blocks = packing.pack_blocks(B, C, F, 0, list(range((C - 1) * F + 1)))
    n = len(blocks) * B
    q, kn, vn = _rand(rng, n, h, d), _rand(rng, n, h, d), _rand(rng, n, h, d)
    kp, vp = _rand(rng, L, h, d), _rand(rng, L, h, d)
    base = attention.packed_attention(q, kp, vp, kn, vn, packing.visible_mask(B, blocks, L), 0.5)
    perm = [0] + list(1 + rng.permutation(len(blocks) - 1))
    rows = np.concatenate([np.arange(b * B, (b + 1) * B) for b in perm])
    pblocks = [blocks[b] for b in perm]
    out = attention.packed_attention(q[rows], kp, vp, kn[rows], vn[rows],
                                     packing.visible_mask(B, pblocks, L), 0.5)
    np.testing.assert_allclose(out, base[rows], rtol=1e-12, atol=1e-13)


def test_mha_reduces_headwise():
    """H_q = H_kv: every head is independent single-head attention."""
    rng = np.random.default_rng(4)
    B, L, h, d = 8, 10, 3, 16
    blocks = packing.pack_blocks(B, 3, 1, 0, [0, 0, 0])
    n = len(blocks) * B
    q, kn, vn = _rand(rng, n, h, d), _rand(rng, n, h, d), _rand(rng, n, h, d)
    kp, vp = _rand(rng, L, h, d), _rand(rng, L, h, d)
    mask = packing.visible_mask(B, blocks, L)
    full = attention.packed_attention(q, kp, vp, kn, vn, mask, 0.25)
    for i in range(h):
        one = attention.packed_attention(q[:, i:i + 1], kp[:, i:i + 1], vp[:, i:i + 1],
                                         kn[:, i:i + 1], vn[:, i:i + 1], mask, 0.25)
        np.testing.assert_allclose(full[:, i:i + 1], one, rtol=0, atol=0)


def test_row_subset_matches_full():
    rng = np.random.default_rng(5)
    B, L, h, d = 4, 9, 2, 8
    blocks = packing.pack_blocks(B, 3, 2, 0, [0] * 5)
    n = len(blocks) * B
    q, kn, vn = _rand(rng, n, h, d), _rand(rng, n, h, d), _rand(rng, n, h, d)
    kp, vp = _rand(rng, L, h, d), _rand(rng, L, h, d)
    mask = packing.visible_mask(B, blocks, L)
    full = attention.packed_attention(q, kp, vp, kn, vn, mask, 0.4)
    rows = [0, 3, 17, n - 1]
    np.testing.assert_array_equal(attention.packed_attention(q, kp, vp, kn, vn, mask, 0.4, rows=rows),
                                  full[rows])
