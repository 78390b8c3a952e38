"""Shared oracle primitives: the winner rule, bf16 rounding, score margins."""
from __future__ import annotations

import numpy as np


def argmax_rule(x) -> int:
    """Index of the winning column: the first NaN if any, otherwise the first maximum.

    PR #65007, Part 1 (step 4): the ranks pick the winner block as the
    replicated loop does, first NaN block else first maximum. Applied within
    blocks too, the rule composes over any partition of the columns in order,
    so the blockwise winner equals the flat one; NumPy's argmax implements
    exactly this flat rule (NaN propagates as the maximum, ties resolve to the
    lowest index; -0.0 and +0.0 compare equal). An all -inf row gives 0.
    """
    return int(np.argmax(np.asarray(x)))


def bf16_rne(x32) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even; NaN -> quiet NaN.

    The draft-logits cache defaults to bf16 on the pages (PR #65007, the
    unsupported-reason list of the review names a non-bf16 cache).
    """
    b = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    nan = np.isnan(np.asarray(x32, dtype=np.float32))
    r = np.where(nan, (b >> np.uint64(16)) | np.uint64(0x40), r)
    return r.astype(np.uint16)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact; signalling NaNs become quiet NaNs)."""
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(
            np.float64)


def top_two_margin(scores) -> float:
    """Gap between the winning score and the best other score (float64).

    +inf when the winner is NaN (NaN wins by rule, not by value) or when the
    row has a single finite column; 0 for an exact tie.
    """
    s = np.asarray(scores, dtype=np.float64)
    w = int(np.argmax(s))
    if np.isnan(s[w]):
        return float("inf")
    rest = np.delete(s, w)
    rest = rest[~np.isnan(rest)]
    if rest.size == 0:
        return float("inf")
    if not np.isfinite(s[w]):
        return 0.0 if rest.max() == s[w] else float("inf")
    return float(s[w] - rest.max())


def topk_columns(row, k: int) -> np.ndarray:
    """Columns of the k largest entries of a row, in increasing column order.

    DSparkSpeculator API page, ``_sample_sequential_topk``: the candidates are
    the top-k of a step's base logits. The order among equal values is not
    stated there; the reading taken is the winner rule's total order, so a NaN
    ranks above every number, -0.0 equals +0.0, and of equal values the lower
    column ranks higher.
    """
    v = np.asarray(row, dtype=np.float64)
    if not 1 <= k <= v.size:
        raise ValueError("k must be in [1, V]")
    nan = np.isnan(v)
    val = np.where(nan, 0.0, v) + 0.0  # adding +0.0 turns -0.0 into +0.0
    # lexsort's last key is the primary one: NaN first, then value descending, then column
    order = np.lexsort((np.arange(v.size), -val, ~nan))
    return np.sort(order[:k])
