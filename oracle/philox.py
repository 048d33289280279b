"""Philox4x32-10 counter-based generator, uniforms and Gumbel draws (CPU oracle).

Test infrastructure only: imported by tests/, the smoke check and the CPU
baseline of the benchmark, never by the product path.

Philox4x32-10 follows its published definition: J. K. Salmon, M. A. Moraes,
R. O. Dror, D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11,
section 4 (the Philox S-box: two 32x32->64 multiplies per round, ten rounds, a
Weyl key schedule).  Its known-answer vectors (from the Random123 distribution)
live in tests/golden/philox4x32_10_kat.txt.

The pages on speculative speculative decoding do not say how random numbers are
drawn; the layout below is this library's own specification, shared with the
GPU side only as a written definition (no code is shared):

* key     = (seed & 0xffffffff, seed >> 32)
* counter = (idx >> 2, b, j, stream); the draw is output word (idx & 3)
  where b is the sequence, j the position, idx the token id (token streams),
  the block id (block streams) or 0 (the acceptance stream).
* uniform u = ((word >> 9) + 0.5) * 2**-23, an odd multiple of 2**-24 in
  (0, 1) that is exactly representable in binary32 and binary64.
* Gumbel  g = -ln(-ln u).
* a random token in [0, V) from a word: floor(word * V / 2**32), the high
  half of the 64-bit product (every token gets floor or ceil of 2**32 / V
  words).
"""
import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK = 0xFFFFFFFF

# Stream ids (fourth counter word).
DRAFT_TOKEN = 0
DRAFT_BLOCK = 1
ACCEPT = 2
BONUS_TOKEN = 3
BONUS_BLOCK = 4
FALLBACK = 5  # random tokens that stand in for a missed cache entry


def philox4x32_10(ctr, key):
    """Apply ten Philox4x32 rounds.

    ctr: four array-likes of uint32 (broadcastable); key: two ints.
    Returns four uint64 arrays holding the 32-bit output words.
    """
    c = [np.asarray(x, dtype=np.uint64) & np.uint64(_MASK) for x in ctr]
    k0 = int(key[0]) & _MASK
    k1 = int(key[1]) & _MASK
    m0 = np.uint64(M0)
    m1 = np.uint64(M1)
    s32 = np.uint64(32)
    mask = np.uint64(_MASK)
    for _ in range(10):
        p0 = m0 * c[0]  # both factors < 2**32, so the product fits in 64 bits
        p1 = m1 * c[2]
        hi0, lo0 = p0 >> s32, p0 & mask
        hi1, lo1 = p1 >> s32, p1 & mask
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
        k0 = (k0 + W0) & _MASK
        k1 = (k1 + W1) & _MASK
    return c


def draw_words(seed, b, j, stream, idx):
    """32-bit words for draws idx (array) at sequence b, position j, stream."""
    seed = int(seed)
    idx = np.asarray(idx, dtype=np.uint64)
    key = (seed & _MASK, (seed >> 32) & _MASK)
    zero = np.zeros_like(idx)
    out = philox4x32_10((idx >> np.uint64(2), zero + np.uint64(b), zero + np.uint64(j),
                         zero + np.uint64(stream)), key)
    sel = (idx & np.uint64(3)).astype(np.int64)
    words = np.choose(sel, out)
    return words


def uniform_from_word(w):
    """u = ((w >> 9) + 0.5) * 2**-23, in fp64 (exact)."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w >> np.uint64(9)).astype(np.float64) + 0.5) * 2.0 ** -23


def uniforms(seed, b, j, stream, idx):
    return uniform_from_word(draw_words(seed, b, j, stream, idx))


def gumbel_from_uniform(u):
    u = np.asarray(u, dtype=np.float64)
    return -np.log(-np.log(u))


def gumbels(seed, b, j, stream, idx):
    return gumbel_from_uniform(uniforms(seed, b, j, stream, idx))


def token_from_word(w, V):
    """floor(w * V / 2**32): a token in [0, V) from a 32-bit word."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w * np.uint64(V)) >> np.uint64(32)).astype(np.int64)
