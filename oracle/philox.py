"""Philox4x32-10 counter-based generator, oracle side.

The pages key the draft noise by (seed, position-1, column) through a counter
hash they name but do not define (PR #65007, Part 1: the noise keys of the
replicated loop; API page, ``_sample_logits``). The hash used here is
Philox4x32 with 10 rounds from Salmon, Moraes, Dror and Shaw, "Parallel
random numbers: as easy as 1, 2, 3" (SC'11): each round multiplies words 0
and 2 by two fixed odd constants, keeps both 32-bit halves of each product,
and mixes the high halves with words 1 and 3 and the round key; the key is
advanced by two Weyl increments between rounds.

Vectorised over NumPy arrays; the 32x32 -> 64 bit products fit uint64 exactly.
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53  # multiplier applied to counter word 0
PHILOX_M1 = 0xCD9E8D57  # multiplier applied to counter word 2
PHILOX_W0 = 0x9E3779B9  # Weyl increment of key word 0 (golden ratio)
PHILOX_W1 = 0xBB67AE85  # Weyl increment of key word 1 (sqrt(3) - 1)
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Return the four 32-bit output words of Philox4x32-10.

    ``c0..c3`` are the counter words and ``k0, k1`` the key words; all are
    broadcast together and may be Python ints or integer arrays. Outputs are
    uint32 arrays of the broadcast shape.
    """
    x0, x1, x2, x3, a, b = np.broadcast_arrays(*(np.asarray(v, dtype=np.uint64) & _MASK
                                                 for v in (c0, c1, c2, c3, k0, k1)))
    x0, x1, x2, x3 = (np.array(v, dtype=np.uint64) for v in (x0, x1, x2, x3))
    ka = np.array(a, dtype=np.uint64)
    kb = np.array(b, dtype=np.uint64)
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    w0, w1 = np.uint64(PHILOX_W0), np.uint64(PHILOX_W1)
    for rnd in range(10):
        if rnd:
            ka = (ka + w0) & _MASK
            kb = (kb + w1) & _MASK
        p0 = m0 * x0  # < 2**64: exact
        p1 = m1 * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        x0, x1, x2, x3 = hi1 ^ x1 ^ ka, lo1, hi0 ^ x3 ^ kb, lo0
    return tuple(v.astype(np.uint32) for v in (x0, x1, x2, x3))
