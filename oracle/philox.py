"""Philox4x32-10 counter-based generator, for the oracle's dropout decisions.

TEST INFRASTRUCTURE ONLY (see the package header).  Written from the
generator's published definition (Salmon, Moraes, Dror and Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC 2011): a 128-bit counter of four
32-bit words and a 64-bit key of two words; each of the 10 rounds multiplies
counter words 0 and 2 by the constants 0xD2511F53 and 0xCD9E8D57, keeps both
halves of each 64-bit product, and mixes them with the other two words and
the key; the key grows by the Weyl constants 0x9E3779B9 and 0xBB67AE85
between rounds.  Vectorised over arrays of counters with NumPy uint64.
"""
from __future__ import annotations

import numpy as np

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)
_MASK = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Four uint32 output words (as uint64 arrays) for counters (c0..c3) and key (k0, k1)."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK for x in (c0, c1, c2, c3)]
    c = list(np.broadcast_arrays(*c))
    k0 = np.uint64(int(k0) & 0xFFFFFFFF)
    k1 = np.uint64(int(k1) & 0xFFFFFFFF)
    for r in range(10):
        if r > 0:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * c[0]            # < 2^64: exact in uint64
        p1 = _M1 * c[2]
        hi0, lo0 = p0 >> _S32, p0 & _MASK
        hi1, lo1 = p1 >> _S32, p1 & _MASK
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return c


def dropout_keep(b: int, hq: int, Hq: int, rows: np.ndarray, Sk: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Keep decisions [len(rows), Sk] of batch row b, query head hq.

    Element (i, j) draws 16-bit half j % 8 of Philox4x32-10 at counter
    (j // 8, i, b * Hq + hq, low 32 bits of offset) under key (low, high 32 bits
    of seed): half m of the output is the low (m even) or high (m odd) 16 bits
    of word m // 2.  It is kept iff that half is at least threshold(p).
    """
    i = np.asarray(rows, dtype=np.uint64)[:, None]
    j = np.arange(Sk, dtype=np.uint64)[None, :]
    words = philox4x32_10(j >> np.uint64(3), i, np.uint64(b * Hq + hq), np.uint64(offset & 0xFFFFFFFF),
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    m = (j & np.uint64(7)).astype(np.int64)
    w = np.choose(np.broadcast_to(m >> 1, words[0].shape), words)
    half = (w >> (np.uint64(16) * (np.broadcast_to(m, w.shape) & 1).astype(np.uint64))) & np.uint64(0xFFFF)
    return half >= np.uint64(threshold(p))


def threshold(p: float) -> int:
    """The 16-bit threshold of drop probability p (0 <= p < 1): floor(p * 2^16), at most 2^16 - 1."""
    return min(int(np.floor(p * 65536.0)), 0xFFFF)


def drop_probability(p: float) -> float:
    """The probability with which an element is dropped: threshold(p) / 2^16, p rounded down to a
    multiple of 2^-16.  Kept elements are scaled by 1 / (1 - drop_probability(p))."""
    return threshold(p) / 65536.0
