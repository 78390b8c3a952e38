"""Draft LM head, oracle side.

Follows the DSparkSpeculator API page, ``_sample_sequential`` and
``_sample_sequential_topk``: the backbone's hidden state of every (request,
step) row, gathered in (request, step) order, goes through the draft model's
``compute_draft_logits`` to give that row's base draft logits over the draft
vocabulary, before the Markov loop starts.

Readings where the pages are silent: the draft LM head is a plain linear map with
no bias, scale or soft cap (the pages name no logits processor on this path),
logits = hidden @ lm_head^T with hidden [rows, H] and lm_head [V, H] in bf16;
the products of bf16 values are exact in float64 and the sum is kept in
float64, then rounded once to the output type (float32, or bf16 round to
nearest even).
"""
from __future__ import annotations

import numpy as np

from .core import bf16_rne, bf16_to_f64


def draft_logits(hidden_bits, lm_head_bits, out_dtype: str = "f32", cols=None, want_abs: bool = False):
    """Base draft logits [rows, V] (or [rows, len(cols)] for a column subset).

    hidden_bits: [rows, H] uint16 bf16 bit patterns; lm_head_bits: [V, H]
    uint16 bf16 bit patterns; out_dtype "f32" (float32 result) or "bf16"
    (uint16 bit patterns). want_abs also returns sum_h |hidden * lm_head| in
    float64, the scale of the rounding error of any float32 summation order.
    """
    h = bf16_to_f64(hidden_bits)
    w = bf16_to_f64(lm_head_bits if cols is None else np.asarray(lm_head_bits)[np.asarray(cols)])
    z = h @ w.T  # float64 sums of exact products
    z32 = z.astype(np.float32)  # one rounding
    out = bf16_rne(z32) if out_dtype == "bf16" else z32
    if want_abs:
        return out, np.abs(h) @ np.abs(w).T
    return out
