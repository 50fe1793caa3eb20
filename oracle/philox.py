"""Philox counter-based generator (oracle side).

The pages fix no random-number generator for the acceptance test or the residual draw; they only
require that draft tokens be accepted with probability alpha_j and that the replacement be drawn
from the residual distribution ([D3D, 前置知识: 投机解码]; [DScout, 前置知识: 推测解码]). Both
sides of the parity test therefore implement the same counter-based generator, Philox4x32-10,
from its published definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
Random Numbers: As Easy as 1, 2, 3", SC'11, section 3 (the Philox S-box built from two
multiply-hi/lo products per round, a Weyl-sequence key schedule, 10 rounds).

Reading (the pages do not fix the stream layout): key = the 64-bit seed split into (low word, high word); counter
words = (position j, request, round, purpose) with purpose 0 = acceptance test, 1 = residual or
bonus draw; a uniform double takes the top 27 bits of output word 0 and the top 26 bits of word 1:
u = ((x0 >> 5) * 2**26 + (x1 >> 6)) * 2**-53, which lies on the 53-bit grid of [0, 1).

TEST INFRASTRUCTURE: see the package docstring.
"""

import numpy as np

# Round multipliers and Weyl key increments of the 4-word Philox variants (SC'11, section 3.2).
PHILOX_M4x32 = (0xD2511F53, 0xCD9E8D57)
PHILOX_W32 = (0x9E3779B9, 0xBB67AE85)
PHILOX_M4x64 = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
PHILOX_W64 = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)

PURPOSE_ACCEPT = 0
PURPOSE_SAMPLE = 1
PURPOSE_DRAFT = 2


def philox4(counter, key, bits=32, rounds=10):
    """One Philox4xW block on Python integers (exact, any word width W in {32, 64}).

    counter: 4 words, key: 2 words. Each round multiplies words 0 and 2 by the two round
    constants, takes the high and low halves of the double-width products, and mixes the high
    halves with words 1 and 3 and the round key; the key is advanced by the Weyl constants
    between rounds.
    """
    if bits == 32:
        mul, weyl = PHILOX_M4x32, PHILOX_W32
    elif bits == 64:
        mul, weyl = PHILOX_M4x64, PHILOX_W64
    else:
        raise ValueError("Philox4 is defined here for 32- and 64-bit words")
    mask = (1 << bits) - 1
    x0, x1, x2, x3 = (int(c) & mask for c in counter)
    k0, k1 = (int(k) & mask for k in key)
    for _ in range(rounds):
        p0 = mul[0] * x0
        p1 = mul[1] * x2
        x0, x1, x2, x3 = ((p1 >> bits) ^ x1 ^ k0, p1 & mask, (p0 >> bits) ^ x3 ^ k1, p0 & mask)
        k0 = (k0 + weyl[0]) & mask
        k1 = (k1 + weyl[1]) & mask
    return (x0, x1, x2, x3)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10 over NumPy arrays of counters (broadcasting); returns 4 uint32 arrays.

    The 32x32 -> 64-bit products are exact in uint64.
    """
    m32 = np.uint64(0xFFFFFFFF)
    x = [np.asarray(c, dtype=np.uint64) & m32 for c in (c0, c1, c2, c3)]
    x = np.broadcast_arrays(*x)
    x0, x1, x2, x3 = (a.copy() for a in x)
    k0 = np.uint64(int(k0) & 0xFFFFFFFF)
    k1 = np.uint64(int(k1) & 0xFFFFFFFF)
    ma, mb = np.uint64(PHILOX_M4x32[0]), np.uint64(PHILOX_M4x32[1])
    wa, wb = np.uint64(PHILOX_W32[0]), np.uint64(PHILOX_W32[1])
    s32 = np.uint64(32)
    for _ in range(10):
        p0 = ma * x0
        p1 = mb * x2
        x0, x1, x2, x3 = ((p1 >> s32) ^ x1 ^ k0, p1 & m32, (p0 >> s32) ^ x3 ^ k1, p0 & m32)
        k0 = (k0 + wa) & m32
        k1 = (k1 + wb) & m32
    return tuple(a.astype(np.uint32) for a in (x0, x1, x2, x3))


def uniform53(x0, x1):
    """Map two 32-bit words to a double on the 53-bit grid of [0, 1)."""
    hi = np.asarray(x0, dtype=np.uint64) >> np.uint64(5)
    lo = np.asarray(x1, dtype=np.uint64) >> np.uint64(6)
    return (hi.astype(np.float64) * 67108864.0 + lo.astype(np.float64)) * (2.0 ** -53)


def uniforms(seed, position, request, round_, purpose):
    """Uniform(s) for counter (position, request, round, purpose) under the 64-bit key `seed`."""
    seed = int(seed)
    x0, x1, _, _ = philox4x32_10(position, request, round_, purpose,
                                 seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    return uniform53(x0, x1)


def uniform24(word):
    """Map a 32-bit word to the open interval (0, 1) on a 24-bit grid: ((w >> 8) + 1/2) / 2^24 (exact
    in binary64, which needs 25 significant bits here; never 0 or 1)."""
    return ((np.asarray(word, dtype=np.uint64) >> np.uint64(8)).astype(np.float64) + 0.5) * (2.0 ** -24)
