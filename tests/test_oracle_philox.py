"""Pins of the oracle's Philox generator against its published definition and a library routine."""

import numpy as np
import pytest
from scipy import stats

from oracle import philox


def test_known_answer_vectors(golden):
    for row in golden("philox4x32_10_kat.txt"):
        words = [int(x, 16) for x in row]
        ctr, key, want = words[:4], words[4:6], tuple(words[6:])
        assert philox.philox4(ctr, key, bits=32) == want
        got = philox.philox4x32_10(*[np.array([c]) for c in ctr], key[0], key[1])
        assert tuple(int(g[0]) for g in got) == want


@pytest.mark.parametrize("key,start", [((3, 5), 7), ((0, 0), 0), ((2**64 - 1, 12345), 2**40)])
def test_philox4x64_matches_numpy(key, start):
    """The same round function and key schedule at 64-bit words is NumPy's Philox bit generator
    (which advances its 256-bit counter before producing each block)."""
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                          counter=np.array([start, 0, 0, 0], dtype=np.uint64))
    raw = [int(v) for v in bg.random_raw(12)]
    for blk in range(3):
        ctr = start + 1 + blk
        words = [ctr & (2**64 - 1), ctr >> 64, 0, 0]
        assert list(philox.philox4(words, key, bits=64)) == raw[4 * blk:4 * blk + 4]


def test_vectorised_matches_scalar():
    rng = np.random.default_rng(0)
    c = rng.integers(0, 2**32, size=(4, 50), dtype=np.uint64)
    k0, k1 = 0x12345678, 0x9ABCDEF0
    vec = philox.philox4x32_10(c[0], c[1], c[2], c[3], k0, k1)
    for i in range(50):
        assert tuple(int(v[i]) for v in vec) == philox.philox4(c[:, i], (k0, k1), bits=32)


def test_uniform53_grid_and_range():
    assert philox.uniform53(0, 0) == 0.0
    # word 0 supplies the 27 high bits, word 1 the 26 low bits (hand values)
    assert philox.uniform53(0x80000000, 0) == 0.5
    assert philox.uniform53(0, 0x80000000) == 2.0 ** -28
    assert philox.uniform53(0x20, 0x40) == (2.0 ** 26 + 1.0) * 2.0 ** -53
    top = philox.uniform53(0xFFFFFFFF, 0xFFFFFFFF)
    assert top == 1.0 - 2.0**-53
    u = philox.uniforms(0xD3D2, np.arange(4096), 3, 9, 0)
    assert np.all((u >= 0) & (u < 1))
    assert np.all(u * 2.0**53 == np.floor(u * 2.0**53))


def test_uniforms_chi_square():
    u = philox.uniforms(0xD3D0, np.arange(200000), 1, 0, 0)
    counts, _ = np.histogram(u, bins=100, range=(0, 1))
    assert stats.chisquare(counts).pvalue > 1e-3
    # distinct purposes / requests / rounds give independent-looking streams
    v = philox.uniforms(0xD3D0, np.arange(200000), 1, 0, 1)
    assert abs(np.corrcoef(u, v)[0, 1]) < 0.01


def test_uniforms_layout_against_known_answers(golden):
    """uniforms(seed, j, request, round, purpose) is the Philox block at counter (j, request, round,
    purpose) under key (seed low word, seed high word), mapped by uniform53: checked on the
    known-answer vectors, so the counter order and the key split are pinned too."""
    for row in golden("philox4x32_10_kat.txt"):
        words = [int(x, 16) for x in row]
        ctr, key, want = words[:4], words[4:6], words[6:]
        u = philox.uniforms(key[0] | (key[1] << 32), *ctr)
        assert u == ((want[0] >> 5) * 2.0 ** 26 + (want[1] >> 6)) * 2.0 ** -53
