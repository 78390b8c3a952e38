"""Counter-keyed uniforms and Gumbel noise, oracle side.

What the pages fix (DSparkSpeculator API page, ``_sample_logits``; PR #65007,
Part 1 and its review thread on constants): the noise of a draw is a pure
function of the request's seed, of the position *before* the sampled token
(P-1 for a token at position P) and of the column, and draft noise carries a
salt of 1<<30 so that it never collides with the noise of target sampling.
What they leave open, and the choice made here:

* counter = (column >> 2, low 32 bits of the position key, high 32 bits,
  salt), key = (low 32 bits of the seed, high 32 bits); column c reads output
  word c & 3, so one Philox call serves four adjacent columns;
* uniform u = (2 * (word >> 9) + 1) * 2**-24: an odd multiple of 2**-24,
  strictly inside (0, 1), exact in float32, symmetric around 1/2;
* Gumbel g = -log(-log u);
* verification draws use their own salts (1 for the accept uniforms, 2 for
  the residual / bonus resample) so they are independent of the draft draw,
  which the min(1, p/q) acceptance rule requires.
"""
from __future__ import annotations

import numpy as np

from .philox import philox4x32_10

SALT_DRAFT = 1 << 30
SALT_ACCEPT = 1
SALT_RESAMPLE = 2


def _split64(x):
    x = np.asarray(x).astype(np.int64).view(np.uint64) if np.ndim(x) else np.uint64(int(x) & (2**64 - 1))
    return x & np.uint64(0xFFFFFFFF), x >> np.uint64(32)


def noise_words(seed: int, pos_key: int, salt: int, cols) -> np.ndarray:
    """Philox output word for each column in ``cols`` (uint32 array)."""
    cols = np.asarray(cols, dtype=np.int64)
    s_lo, s_hi = _split64(int(seed))
    p_lo, p_hi = _split64(int(pos_key))
    groups = (cols >> 2).astype(np.uint64)
    w = philox4x32_10(groups, p_lo, p_hi, np.uint64(salt), s_lo, s_hi)
    words = np.stack(w, axis=-1)  # [..., 4]
    return np.take_along_axis(words, (cols & 3)[..., None], axis=-1)[..., 0]


def uniform24(words) -> np.ndarray:
    """Uniform in (0, 1) from the top 23 bits of a word: (2m+1) * 2**-24 (float64, exact)."""
    m = np.asarray(words, dtype=np.uint32) >> np.uint32(9)
    return (2.0 * m.astype(np.float64) + 1.0) * 2.0 ** -24


def gumbel(u) -> np.ndarray:
    """Standard Gumbel variate -log(-log u) in float64.

    -log u is taken as -log1p(u - 1): u - 1 is exact in float64 for these u,
    so the inner logarithm keeps full relative accuracy as u -> 1.
    """
    u = np.asarray(u, dtype=np.float64)
    e = -np.log1p(u - 1.0)
    return -np.log(e)


def gumbel_row(seed: int, pos_key: int, salt: int, V: int) -> np.ndarray:
    """Gumbel noise for columns 0..V-1 of one draw (float64)."""
    return gumbel(uniform24(noise_words(seed, pos_key, salt, np.arange(V))))


def accept_uniform(seed: int, pos_key: int) -> float:
    """The accept-test uniform of one draft position: column 0 of the accept stream."""
    return float(uniform24(noise_words(seed, pos_key, SALT_ACCEPT, np.array([0])))[0])
