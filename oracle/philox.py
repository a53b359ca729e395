"""Philox4x32-10 counter-based generator, written from its published definition.

Source: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11, section 3.2 (the Philox S-box: two
32x32->64 multiplies per round, Weyl-sequence key schedule), with the
round multipliers 0xD2511F53, 0xCD9E8D57 and key increments 0x9E3779B9,
0xBB67AE85 given there.  Ten rounds.

ORACLE — test infrastructure only.  This is an independent implementation of
the same published generator that the GPU path implements on its own; the two
share no code.

The sampler's use of the generator (counter fields, streams, conversions) is
the reading stated in ``oracle/sampler.py``:
counter = (position i, step t, block b, stream), key = (seed lo32, seed hi32).
"""
from __future__ import annotations

import numpy as np

_MASK = np.uint64(0xFFFFFFFF)
_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)

STREAM_INIT = 0      # initial canvas noise
STREAM_RENOISE = 1   # re-noise of unselected positions
STREAM_SAMPLE = 2    # (u1, u2) for the categorical sample


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  Inputs broadcast; returns four uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK for x in (c0, c1, c2, c3)]
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK
    x0, x1, x2, x3 = np.broadcast_arrays(*c)
    x0, x1, x2, x3 = x0.copy(), x1.copy(), x2.copy(), x3.copy()
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * x0
        p1 = _M1 * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return tuple(v.astype(np.uint32) for v in (x0, x1, x2, x3))


def seed_key(seed: int):
    """64-bit sampler seed -> Philox key (lo32, hi32)."""
    seed &= (1 << 64) - 1
    return seed & 0xFFFFFFFF, seed >> 32


def words(seed: int, positions, step: int, block: int, stream: int):
    """Four words for each canvas position under the sampler's counter layout."""
    k0, k1 = seed_key(seed)
    pos = np.asarray(positions, dtype=np.uint64)
    return philox4x32_10(pos, step, block, stream, k0, k1)


def word_to_token(w, vocab: int) -> np.ndarray:
    """Multiply-shift map of a 32-bit word onto [0, vocab); equals w >> (32-b)
    when vocab = 2^b, i.e. exactly uniform for the power-of-two vocabularies."""
    return ((np.asarray(w, dtype=np.uint64) * np.uint64(vocab)) >> np.uint64(32)).astype(np.int64)


def word_to_unit(w) -> np.ndarray:
    """24-bit uniform in [0, 1): (w >> 8) * 2^-24 (exact in fp32 and fp64)."""
    return (np.asarray(w, dtype=np.uint64) >> np.uint64(8)).astype(np.float64) * 2.0 ** -24
