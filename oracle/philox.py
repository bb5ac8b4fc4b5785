"""Philox4x32-10 and the uniforms the sampled acceptance rule draws.

Philox4x32 is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC'11), section 3: each round
multiplies words 0 and 2 of the counter by two fixed 32-bit multipliers, XORs
the high halves with the other two words and the round key, and swaps; the
key is bumped by two Weyl constants between rounds.  Ten rounds.

Counter layout used by the verify round (the pages only say the draws are
keyed by seed, lane and position):
    key     = (seed low 32 bits, seed high 32 bits)
    counter = (position, lane, purpose, block)
    purpose ACCEPT (0): word 0 of block 0 is the acceptance uniform of the
                        draft at that position;
    purpose RACE   (1): token v uses word v % 4 of block v // 4.
Uniform: U = ((w >> 9) + 0.5) * 2^-23: 23 random bits, strictly inside (0, 1),
and exactly representable in float32 (with 24 bits, k + 0.5 would need a
25-bit significand for half of the words).
"""
import numpy as np

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)
_MASK = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

ACCEPT = 0
RACE = 1


def philox4x32_10(counter, key):
    """counter: 4 arrays (or ints) of uint32 words; key: 2 arrays/ints.  Returns 4 uint32 arrays."""
    c = [np.asarray(w, dtype=np.uint64) & _MASK for w in counter]
    k0 = np.asarray(key[0], dtype=np.uint64) & _MASK
    k1 = np.asarray(key[1], dtype=np.uint64) & _MASK
    c0, c1, c2, c3 = np.broadcast_arrays(*c)
    c0, c1, c2, c3 = c0.copy(), c1.copy(), c2.copy(), c3.copy()
    for _ in range(10):
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> _S32, p0 & _MASK
        hi1, lo1 = p1 >> _S32, p1 & _MASK
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0) & _MASK, lo1, (hi0 ^ c3 ^ k1) & _MASK, lo0
        k0 = (k0 + _W0) & _MASK
        k1 = (k1 + _W1) & _MASK
    return tuple(w.astype(np.uint32) for w in (c0, c1, c2, c3))


def uniform01(word) -> np.ndarray:
    """Uniform in (0, 1) from a uint32 word: ((w >> 9) + 0.5) * 2^-23 (exact in float32)."""
    w = np.asarray(word, dtype=np.uint32)
    return ((w >> np.uint32(9)).astype(np.float64) + 0.5) * (2.0 ** -23)


def _key(seed: int):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return (seed & 0xFFFFFFFF, seed >> 32)


def accept_uniform(seed: int, pos, lane) -> np.ndarray:
    """Acceptance uniform for the draft at absolute position `pos` of lane `lane`."""
    pos = np.asarray(pos, dtype=np.uint64)
    w = philox4x32_10((pos, np.asarray(lane, np.uint64), np.uint64(ACCEPT), np.uint64(0)), _key(seed))
    return uniform01(w[0])


def race_uniforms(seed: int, pos: int, lane: int, vocab: int) -> np.ndarray:
    """One uniform per token v in [0, vocab) for the race deciding position `pos` of `lane`."""
    nblk = (vocab + 3) // 4
    blk = np.arange(nblk, dtype=np.uint64)
    w = philox4x32_10((np.uint64(pos), np.uint64(lane), np.uint64(RACE), blk), _key(seed))
    words = np.stack(w, axis=1).reshape(-1)[:vocab]
    return uniform01(words)
