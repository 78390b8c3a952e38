"""Sequential Markov draft loop, oracle side.

Follows the DSparkSpeculator API page: ``_sample_sequential`` (the base draft
logits are ordered (request, step) and the previous token of step 0 is the
request's anchor, the input id at query offset 0), ``_sample_markov_chain``
(for each step: embed the previous token, project the embedding into a
vocabulary-wide Markov bias, add it to that step's base logits, sample, and
feed the sample back as the previous token) and ``_sample_logits`` (the draw
for predicted position P is keyed by P-1, temperature is applied, and the
biased logits are stored into the draft-logits cache at column = step).

Readings where the pages are silent:

* the Markov embedding of token x is row x of a bf16 matrix w1[V, r], with no
  scale or normalisation, and the bias is w2[V, r] @ embedding (PR #65007,
  Part 1, gives w2's shape [draft_vocab, markov_rank] and dtype bf16);
* the bias is kept at full precision and the biased logit z = base + bias is
  rounded once to float32;
* the cache stores z before temperature, rounded to the cache dtype;
* score s = z / T + g for T > 0 and s = z for a greedy (T = 0) request, in
  float32 because the pages' Gumbel noise is float32 by default (PR #65007,
  the fp64 Gumbel option listed under Part 1's unsupported configurations);
* the winner is the first NaN, otherwise the first maximum (``argmax_rule``).

Top-k Markov drafting (the API page's ``_sample_sequential_topk``): the
candidates of each step are chosen once, from the base logits alone
(``topk_columns``); at every step the Markov bias is applied at those columns
only, through the gathered rows of w2, every other entry of the step's row is
-inf, and that row then goes through the same sampler and cache write.
"""
from __future__ import annotations

import numpy as np

from .core import argmax_rule, bf16_rne, bf16_to_f64, top_two_margin, topk_columns
from .noise import SALT_DRAFT, gumbel_row


def _logsumexp(x64: np.ndarray) -> float:
    if np.isnan(x64).any():
        return float("nan")
    m = x64.max()
    if not np.isfinite(m):
        return float(m)
    return float(m + np.log(np.exp(x64 - m).sum()))


def draft_loop(base, base_dtype: str, w1_bits, w2_bits, anchor_tokens, anchor_pos, seeds, temperature,
               cache_dtype: str, K: int | None = None, teacher=None, want_scores: bool = False,
               idx_map=None, row_mapping=None, sample_pos=None, cache_init=None, fp64_gumbel: bool = False,
               topk: int | None = None) -> dict:
    """Run the K-step Markov draft loop for every request.

    base: [B, >=K, V] float32, or uint16 bf16 bit patterns when base_dtype is "bf16";
    w1_bits, w2_bits: [V, r] uint16 bf16 bit patterns;
    anchor_tokens [B], anchor_pos [B] (P0), seeds [B], temperature [B] (0 = greedy).
    teacher: optional [B, K] tokens; when given, step k+1 uses teacher[:, k] as its
    previous token instead of the oracle's own sample (each step then checks
    independently against another implementation's tokens).

    Request-state indexing (the API page's ``_sample_logits`` / ``gumbel_sample``
    call: per-row ``idx_map``, ``sample_pos`` and the cache's ``row_mapping``):
    idx_map [B, K] gives the state slot of row b at step k; temperature and
    seeds are then indexed by slot, the draw is keyed by sample_pos[b, k] - 1
    (the position before the predicted token) instead of anchor_pos[b] + k, and
    the cache row is row_mapping[slot] (the slot itself without a mapping) in
    a cache of cache_init's shape [R, K, V] (cache_init is copied, so rows the
    call does not write keep their values). A negative slot makes that step of
    the row inert (the page's padding slots: no cache write): its token is -1
    and its lse NaN; a later non-inert step of the row then has no valid
    previous token, and uses token 0 (flagged by bad_prev).

    fp64_gumbel (the API page's ``use_fp64_gumbel``): the Gumbel variate and the
    score z / T + g stay in float64 (the same uniforms) and the winner is
    taken over the float64 scores.

    topk (the API page's top-k Markov drafting): the k candidate columns of
    step k of request b are the top-k of base[b, k]; the biased logit there is
    base + (w2[candidate rows] @ embedding), every other column holds -inf,
    and the row is then sampled and cached as in the dense loop.

    Returns tokens [B, K] int32, cache [B, K, V] (float32 or uint16 bf16 bits;
    [R, K, V] with idx_map), lse [B, K] float64 (log-sum-exp of cache / T; NaN
    for greedy rows) and margin [B, K] float64 (top-two gap of the float32
    scores).
    """
    base = np.asarray(base)
    B, _, V = base.shape
    K = base.shape[1] if K is None else int(K)
    w1 = bf16_to_f64(w1_bits)
    w2t = np.ascontiguousarray(bf16_to_f64(w2_bits).T)  # [r, V]
    tokens = np.zeros((B, K), np.int32)
    if idx_map is None:
        cache = np.zeros((B, K, V), np.uint16 if cache_dtype == "bf16" else np.float32)
    else:
        cache = np.array(cache_init, copy=True)
        idx_map = np.asarray(idx_map, np.int64)
    lse = np.full((B, K), np.nan)
    margin = np.zeros((B, K))
    scores_out = np.zeros((B, K, V), np.float64 if fp64_gumbel else np.float32) if want_scores else None
    prev = np.asarray(anchor_tokens, dtype=np.int64).copy()
    bad_prev = False
    if topk is not None:  # candidate selection, once for all steps, from the base logits alone
        cand = [[topk_columns(bf16_to_f64(base[b, k]) if base_dtype == "bf16" else base[b, k], int(topk))
                 for k in range(K)] for b in range(B)]
    if idx_map is None and ((prev < 0).any() or (prev >= V).any()):
        raise ValueError("anchor token out of range")
    for k in range(K):
        live = np.ones(B, bool) if idx_map is None else idx_map[:, k] >= 0
        if ((prev < 0) | (prev >= V))[live].any():
            if idx_map is None:
                raise ValueError("previous token out of range")
            bad_prev = True
        prev = np.where((prev >= 0) & (prev < V), prev, 0)
        emb = w1[prev]  # [B, r]: row gather (markov_embed)
        row = bf16_to_f64(base[:, k]) if base_dtype == "bf16" else base[:, k].astype(np.float64)
        if topk is None:
            bias = emb @ w2t  # [B, V]: markov_bias, exact products, float64 sums
            z32 = (row + bias).astype(np.float32)  # one rounding
        else:
            # bias at the candidates only, through the gathered rows of w2;
            # every other entry of the row is -inf
            z32 = np.full((B, V), -np.inf, np.float32)
            for b in range(B):
                c = cand[b][k]
                z32[b, c] = (row[b, c] + emb[b] @ w2t[:, c]).astype(np.float32)
        if cache_dtype == "bf16":
            cbits = bf16_rne(z32)
            cval = bf16_to_f64(cbits)
        else:
            cbits = z32
            cval = z32.astype(np.float64)
        for b in range(B):
            if idx_map is None:
                slot, crow, key = b, b, int(anchor_pos[b]) + k
            else:
                slot = int(idx_map[b, k])
                if slot < 0:  # inert: no cache write, no sample
                    tokens[b, k] = -1
                    margin[b, k] = np.inf
                    continue
                crow = slot if row_mapping is None else int(row_mapping[slot])
                key = (int(sample_pos[b, k]) - 1) if sample_pos is not None else int(anchor_pos[b]) + k
            cache[crow, k] = cbits[b]
            T = np.float32(temperature[slot])
            if T > 0:
                g64 = gumbel_row(int(seeds[slot]), key, SALT_DRAFT, V)
                if fp64_gumbel:
                    s = z32[b].astype(np.float64) / np.float64(T) + g64
                else:
                    s = (z32[b] / T).astype(np.float32) + g64.astype(np.float32)
                lse[b, k] = _logsumexp(cval[b] / np.float64(T))
            else:
                s = z32[b]
            tokens[b, k] = argmax_rule(s)
            margin[b, k] = top_two_margin(s)
            if want_scores:
                scores_out[b, k] = s
        prev = tokens[:, k].astype(np.int64) if teacher is None else np.asarray(teacher, np.int64)[:, k]
    out = {"tokens": tokens, "cache": cache, "lse": lse, "margin": margin, "bad_prev": bad_prev}
    if want_scores:
        out["scores"] = scores_out
    return out
