"""Counter-based random bits for dropout: Philox4x32-10 and the dropout mask.

Test infrastructure only (see the package docstring).

The 51CTO FlashAttention V1/V2 notes ("FlashAttention V2 相比 V1 有哪些改进",
the figure that sets the V1 and V2 algorithms side by side) show dropout on
the probabilities inside the V1 loop and set it aside.  A fused kernel must
draw the same mask again in the backward pass without storing it, so the
random bits come from a counter-based generator: Philox4x32 with 10 rounds,
as defined by Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
Easy as 1, 2, 3" (SC 2011), section 3.2 (the Philox S-box: two 32x32->64
multiplications per round, the high halves xor-ed with the other two counter
words and the round key, a Weyl sequence for the round keys).  The kernels
carry their own implementation of the same published definition.

Mask layout (the library's definition of which random bits belong to which
score):

* key = (seed mod 2^32, seed div 2^32), seed a 64-bit integer;
* score (i, j) of flat head bh = b*H + h, query row i, key j, uses the call
  with counter (j div 4, i div 4, bh, offset): one call covers a block of
  4 rows x 4 keys;
* in the call's output, word (i mod 4) holds the row and byte (j mod 4) of
  that word (bits 8*(j mod 4) .. 8*(j mod 4) + 7) the key;
* the key is kept iff that byte is below T = round((1 - p) * 256), so
  1 <= T <= 256 and the keep probability is exactly T / 256;
* kept probabilities are scaled by 256 / T, so the dropped-out P has the
  expectation of P.
"""

from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = 0xFFFFFFFF


def philox4x32(counter, key, rounds: int = 10):
    """Philox4x32-``rounds`` of a batch of counters.

    ``counter``: four arrays (or ints) c0..c3 of 32-bit values, broadcast
    together; ``key``: (k0, k1).  Returns the four output words as uint64
    arrays holding 32-bit values.  Each round: (hi0, lo0) = M0 * c0,
    (hi1, lo1) = M1 * c2, then c = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0);
    the key is bumped by the Weyl constants (W0, W1) between rounds.
    """
    c = [np.asarray(x, dtype=np.uint64) & np.uint64(_MASK32) for x in counter]
    c = list(np.broadcast_arrays(*c))
    k0, k1 = int(key[0]) & _MASK32, int(key[1]) & _MASK32
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    for _ in range(rounds):
        p0 = m0 * c[0]  # < 2^64: exact in uint64
        p1 = m1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(_MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(_MASK32)
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
        k0 = (k0 + PHILOX_W0) & _MASK32
        k1 = (k1 + PHILOX_W1) & _MASK32
    return c


def keep_threshold(p: float) -> int:
    """T = round((1 - p) * 256): a byte below T keeps its score (p in [0, 1),
    T >= 1).  Python's round, to nearest with ties to even."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    t = int(round((1.0 - p) * 256.0))
    if t < 1:
        raise ValueError("dropout probability too close to 1 (fewer than 1 in 256 kept)")
    return t


def dropout_bytes(nq: int, nk: int, seed: int, offset: int, bh: int) -> np.ndarray:
    """The random byte of every score (i, j) of flat head ``bh``: uint8 [nq, nk]."""
    i = np.arange(nq, dtype=np.uint64)[:, None]
    j = np.arange(nk, dtype=np.uint64)[None, :]
    words = philox4x32((j >> np.uint64(2), i >> np.uint64(2), bh, offset),
                       (seed & _MASK32, (seed >> 32) & _MASK32))
    w = np.where((i & np.uint64(3)) == 0, words[0],
                 np.where((i & np.uint64(3)) == 1, words[1],
                          np.where((i & np.uint64(3)) == 2, words[2], words[3])))
    return ((w >> ((j & np.uint64(3)) * np.uint64(8))) & np.uint64(0xFF)).astype(np.uint8)


def dropout_multiplier(nq: int, nk: int, p: float, seed: int, offset: int, bh: int) -> np.ndarray:
    """Z [nq, nk] float64: 256 / T where the score is kept, 0 where it is dropped."""
    t = keep_threshold(p)
    keep = dropout_bytes(nq, nk, seed, offset, bh) < t
    return np.where(keep, 256.0 / t, 0.0)


def dropout_multiplier_batched(B: int, H: int, nq: int, nk: int, p: float, seed: int,
                               offset: int) -> np.ndarray:
    """Z [B, H, nq, nk] for every head (flat head index b*H + h)."""
    out = np.empty((B, H, nq, nk))
    for b in range(B):
        for h in range(H):
            out[b, h] = dropout_multiplier(nq, nk, p, seed, offset, b * H + h)
    return out
