"""Pins of the oracle's packing: the printed budget, a hand-derived mask, a closed-form pair count."""

import numpy as np
import pytest

from oracle import packing


def test_budget_printed_on_page(golden):
    (B, C, F, covered, n), = [[int(x) for x in r] for r in golden("async_budget.txt")]
    assert packing.n_async(B, C, F) == n
    blocks = packing.pack_blocks(B, C, F, 7, list(range(100, 100 + (C - 1) * F + 1)))
    assert len(blocks) * B == n
    assert sorted({r for r, _, _ in blocks if 0 < r < B}) == list(range(1, covered + 1))


def test_long_horizon_budget():
    # B=32, C=16, F=5: 15 covered positions x 5 anchors + full-accept + current = 77 blocks.
    assert packing.n_async(32, 16, 5) == 32 * 77 == 2464


def test_block_order_and_modes():
    B, C, F = 16, 12, 2
    anchors = list(range(1000, 1000 + (C - 1) * F + 1))
    blocks = packing.pack_blocks(B, C, F, 5, anchors)
    assert blocks[0] == (0, 5, True)
    assert blocks[-1] == (B, anchors[-1], False)
    mid = blocks[1:-1]
    assert [r for r, _, _ in mid] == [k for k in range(1, C) for _ in range(F)]
    assert [a for _, a, _ in mid] == anchors[:-1]
    assert not any(c for _, _, c in mid)


def test_hand_derived_mask():
    """B=4, C=3, F=1, prefix L=2: blocks b0 (current, causal), b1 (r=1), b2 (r=2), b3 (full, r=4).

    Keys 0,1 are the prefix; key 2+t is packed row t. Visible sets written out by hand from the
    rules: prefix shared by all; block 0 causal; a branch sees block 0's first r rows and its own
    four rows.
    """
    blocks = packing.pack_blocks(4, 3, 1, 9, [10, 20, 30])
    m = packing.visible_mask(4, blocks, 2)
    expect = {
        0: {0, 1, 2}, 1: {0, 1, 2, 3}, 2: {0, 1, 2, 3, 4}, 3: {0, 1, 2, 3, 4, 5},
        4: {0, 1, 2, 6, 7, 8, 9}, 5: {0, 1, 2, 6, 7, 8, 9},
        6: {0, 1, 2, 6, 7, 8, 9}, 7: {0, 1, 2, 6, 7, 8, 9},
        8: {0, 1, 2, 3, 10, 11, 12, 13}, 9: {0, 1, 2, 3, 10, 11, 12, 13},
        10: {0, 1, 2, 3, 10, 11, 12, 13}, 11: {0, 1, 2, 3, 10, 11, 12, 13},
        12: {0, 1, 2, 3, 4, 5, 14, 15, 16, 17}, 13: {0, 1, 2, 3, 4, 5, 14, 15, 16, 17},
        14: {0, 1, 2, 3, 4, 5, 14, 15, 16, 17}, 15: {0, 1, 2, 3, 4, 5, 14, 15, 16, 17},
    }
    assert m.shape == (16, 18)
    for t, keys in expect.items():
        assert set(np.nonzero(m[t])[0].tolist()) == keys, t


@pytest.mark.parametrize("L", [0, 1, 63, 4096])
def test_visible_pair_count_closed_form(L):
    """At B=16, C=12, F=2 the visible (query, key) pairs are 384 L + 8392, by hand:
    block 0: 1+2+...+16 = 136; branches: sum_{k=1..11} 2*16*(k+16) = 32*(66+176) = 7744;
    full accept: 16*(16+16) = 512."""
    blocks = packing.pack_blocks(16, 12, 2, 0, [0] * 23)
    m = packing.visible_mask(16, blocks, L)
    assert int(m.sum()) == 384 * L + 8392


def test_rejects_bad_budget():
    with pytest.raises(ValueError):
        packing.pack_blocks(16, 17, 2, 0, [0] * 33)
    with pytest.raises(ValueError):
        packing.pack_blocks(16, 12, 2, 0, [0] * 22)
