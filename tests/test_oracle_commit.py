"""Pins of the oracle's KV commit and branch promotion (oracle/commit.py): the cache read back
through its page table, causal consistency with the attention oracle (the committed rows are
exactly the keys / values the accepted tokens would have as prefix tokens), the promoted block's
anchor against the match oracle, and the cache-full case."""

import numpy as np
import pytest

from oracle import attention, commit, match, packing


def _logical(cache, table_row, length):
    ps = cache.shape[1]
    return np.stack([cache[table_row[t // ps], t % ps] for t in range(length)]) if length else cache[:0, 0]


def _setup(rng, n_req=3, B=4, ps=3, hkv=2, d=8, lens=(5, 0, 7), blocks=(3, 2, 4)):
    off = np.concatenate([[0], np.cumsum(blocks)]).astype(np.int64)
    nq = int(off[-1]) * B
    k_new, v_new = rng.normal(size=(nq, hkv, d)), rng.normal(size=(nq, hkv, d))
    max_pages = 6
    pages = rng.permutation(n_req * max_pages)
    table = pages.reshape(n_req, max_pages)
    kc = rng.normal(size=(n_req * max_pages, ps, hkv, d))
    vc = rng.normal(size=kc.shape)
    return off, k_new, v_new, kc, vc, table, np.array(lens)


@pytest.mark.parametrize("seed", range(4))
def test_cache_reads_back_as_prefix_then_accepted_rows(seed):
    rng = np.random.default_rng(seed)
    B = 4
    off, k_new, v_new, kc, vc, table, lens = _setup(rng, B=B)
    n_acc = rng.integers(0, B, size=3)
    kc2, vc2, lens2, status = commit.kv_commit(k_new, v_new, kc, vc, table, off, lens, n_acc, B)
    assert (status == 0).all()
    assert (lens2 == lens + n_acc + 1).all()
    for i in range(3):
        before = _logical(kc, table[i], int(lens[i]))
        after = _logical(kc2, table[i], int(lens2[i]))
        rows = k_new[off[i] * B: off[i] * B + n_acc[i] + 1]
        assert np.array_equal(after, np.concatenate([before, rows]))
        assert np.array_equal(_logical(vc2, table[i], int(lens2[i]))[lens[i]:],
                              v_new[off[i] * B: off[i] * B + n_acc[i] + 1])


def test_committed_rows_are_what_block0_queries_attend_as_prefix():
    """A query of block 0 row j (causal) sees the prefix and rows 0..j of its own block; after the
    commit the same keys are the first L + j + 1 cache tokens: attention over them matches."""
    rng = np.random.default_rng(7)
    B, C, F, L, hq, hkv, d = 4, 3, 1, 5, 4, 2, 8
    blocks = packing.pack_blocks(B, C, F, 11, [21, 22, 23])
    nq = len(blocks) * B
    q = rng.normal(size=(nq, hq, d))
    k_new, v_new = rng.normal(size=(nq, hkv, d)), rng.normal(size=(nq, hkv, d))
    k_pre, v_pre = rng.normal(size=(L, hkv, d)), rng.normal(size=(L, hkv, d))
    ps, max_pages = 2, 8
    table = rng.permutation(max_pages)[None]
    kc, vc = np.zeros((max_pages, ps, hkv, d)), np.zeros((max_pages, ps, hkv, d))
    for t in range(L):
        kc[table[0, t // ps], t % ps], vc[table[0, t // ps], t % ps] = k_pre[t], v_pre[t]
    n_acc = 2
    kc2, vc2, lens2, _ = commit.kv_commit(k_new, v_new, kc, vc, table, [0, len(blocks)], [L], [n_acc], B)
    mask = packing.visible_mask(B, blocks, L)
    packed = attention.packed_attention(q, k_pre, v_pre, k_new, v_new, mask, d ** -0.5, rows=range(n_acc + 1))
    for j in range(n_acc + 1):
        n = L + j + 1
        kk, vv = _logical(kc2, table[0], n), _logical(vc2, table[0], n)
        plain = attention.packed_attention(q[j:j + 1], kk, vv, k_new[:0], v_new[:0], np.ones((1, n), bool), d ** -0.5)
        np.testing.assert_allclose(plain[0], packed[j], rtol=1e-12, atol=1e-12)


def test_promoted_block_starts_with_the_verified_next_token():
    B, C, F = 4, 3, 2
    anchors = [31, 32, 41, 42, 50]
    blocks = packing.pack_blocks(B, C, F, 7, anchors)
    tokens = np.concatenate([[anc] + [100 * b + p for p in range(1, B)] for b, (_r, anc, _c) in enumerate(blocks)])
    for n_acc, nxt in ((0, 32), (1, 41), (3, 50), (1, 99)):
        hit = match.match_request(blocks, n_acc, nxt)
        out = commit.promote(tokens, [0, len(blocks)], [hit], B)[0]
        if hit >= 0:
            assert out[0] == nxt and out[1:].tolist() == [100 * hit + p for p in range(1, B)]
        else:
            assert (out == -1).all()


def test_cache_full_keeps_the_leading_rows():
    rng = np.random.default_rng(3)
    B, ps = 4, 2
    off = np.array([0, 2])
    k_new, v_new = rng.normal(size=(2 * B, 1, 4)), rng.normal(size=(2 * B, 1, 4))
    kc, vc = np.zeros((3, ps, 1, 4)), np.zeros((3, ps, 1, 4))
    table = np.array([[2, 0, -1]])  # room for 4 tokens
    kc2, _vc2, lens2, status = commit.kv_commit(k_new, v_new, kc, vc, table, off, [3], [3], B)
    assert status[0] == 1 and lens2[0] == 4  # one of four rows fits
    assert np.array_equal(kc2[0, 1], k_new[0])
