"""Rejection-sampling verification with optional exact top-p, oracle side.

Follows PR #65007: the Overview (verification applies temperature, then
top-p, then the rejection sampler over the whole vocabulary), Part 2 (top-p
keeps the smallest prefix, ordered by logit then token id, whose probability
mass reaches p, plus the row maximum; greedy rows skip it) and Tests (the
rejection sampler's outputs are sampled tokens and per-request counts, over
greedy and sampled requests). PR #63554, Notes: at temperature 0 verification
compares with the target argmax and never reads the cached draft logits.

Standard speculative rejection sampling (the method the pages' stock
rejection sampler implements): draft token x at step k is accepted with
probability min(1, p_k(x) / q_k(x)); the first rejected step draws its
replacement from the normalised residual max(0, p_k - q_k); when every draft
is accepted a bonus token is drawn from p_K.

Readings where the pages are silent:

* the accept test is p >= u * q with u the column-0 uniform of the accept
  stream at key P0+k, taken in float32 (the kernel's precision);
* residual and bonus draws are Gumbel-max over log r (log p) + Gumbel noise
  of the resample stream at key P0+j, the same law as inverse-CDF sampling;
  their argmax is taken over float32 scores;
* a residual with zero total mass (p == q, or a draft row holding NaN, which
  makes every q NaN) falls back to sampling from p;
* top_p >= 1 disables top-p for a request;
* a row with no finite logit (every entry -inf: all columns masked) has no
  softmax; its distribution is taken to be the one-hot at column 0, the
  column the winner rule gives such a row (the first of equal maxima). This
  holds for a target row (p, and so its top-p kept set {0}) and for a draft
  cache row (q); the pages' top-p tests name such rows without stating the
  result;
* a draft token of -1 is a placeholder (PR #65007, Tests: rejection sampling
  with -1 placeholder drafts): the request's drafts end there, so the draw
  after the accepted run is taken from p of that row, as when all K drafts
  are accepted;
* request-state indexing: idx_map [B] gives the state slot of request b
  (temperature, seeds and top_p are indexed by slot) and its cache rows are
  row_mapping[slot] (the slot itself without a mapping); a negative slot is a
  padding request: no work, every output token -1 and 0 accepted.
"""
from __future__ import annotations

import numpy as np

from .core import argmax_rule, bf16_to_f64, top_two_margin
from .noise import SALT_RESAMPLE, accept_uniform, gumbel_row


def _softmax(x64: np.ndarray) -> np.ndarray:
    """softmax of a row of finite values, -inf (masked columns) and +inf-free;
    a row with no finite value gives the one-hot at column 0 (see above)."""
    m = np.max(x64)
    if m == -np.inf:
        p = np.zeros(x64.shape, np.float64)
        p[0] = 1.0
        return p
    e = np.exp(x64 - m)
    return e / e.sum()


def top_p_keep(t_row, T: float, p: float):
    """Kept set of exact top-p on one target row (after temperature).

    Returns (mask, near_boundary). Columns are ordered by logit descending,
    then token id ascending; the kept set is the shortest prefix whose float64
    cumulative probability is >= p, and the row maximum is always kept.
    near_boundary is True when the cumulative mass at the cut (or one column
    before it) lies within 1e-6 of p: there a float32 implementation may keep
    a different set (the pages' own test excludes such rows). A row with no
    finite logit keeps {0}: its distribution is the one-hot at column 0.
    """
    t = np.asarray(t_row, dtype=np.float64)
    V = t.size
    mask = np.zeros(V, bool)
    if p >= 1.0:
        mask[:] = True
        return mask, False
    probs = _softmax(t / T)
    order = np.lexsort((np.arange(V), -t))
    cum = np.cumsum(probs[order])
    hit = np.nonzero(cum >= p)[0]
    n = int(hit[0]) + 1 if hit.size else V
    n = max(n, 1)
    mask[order[:n]] = True
    near = abs(cum[n - 1] - p) <= 1e-6 or (n >= 2 and abs(cum[n - 2] - p) <= 1e-6)
    return mask, bool(near)


def verify(target, cache, cache_dtype: str, draft_tokens, temperature, top_p, seeds, anchor_pos,
           idx_map=None, row_mapping=None) -> dict:
    """Verify the drafts of every request.

    target: [B*(K+1), V] float32, row b*(K+1)+j is position P0+1+j of request b;
    cache: [B, K, V] float32 or uint16 bf16 bits (pre-temperature draft logits);
    draft_tokens: [B, K] (-1 = placeholder); temperature, seeds, top_p [B], or
    [slots] with idx_map (0 = greedy; top_p may be None).

    Returns out_tokens [B, K+1] int32 (accepted drafts, then the final token,
    then -1), num_accepted [B], and diagnostics: accept_margin (the smallest
    |p/q - u| over compared steps), sample_margin (top-two gap of the final
    draw's scores), near_top_p (a compared or sampled row has its top-p cut
    within 1e-6 of p), final_row (the row the final token was drawn from).
    """
    draft_tokens = np.asarray(draft_tokens)
    B, K = draft_tokens.shape
    target = np.asarray(target)
    V = target.shape[1]
    out = np.full((B, K + 1), -1, np.int32)
    nacc = np.zeros(B, np.int32)
    acc_margin = np.full(B, np.inf)
    smp_margin = np.full(B, np.inf)
    near_tp = np.zeros(B, bool)
    final_row = np.zeros(B, np.int32)
    for b in range(B):
        slot, crow = b, b
        if idx_map is not None:
            slot = int(idx_map[b])
            if slot < 0:  # padding request
                continue
            crow = slot if row_mapping is None else int(row_mapping[slot])
        T = float(np.float32(temperature[slot]))
        rows = target[b * (K + 1):(b + 1) * (K + 1)]
        d = np.asarray(draft_tokens[b], np.int64)
        if np.any(d < -1) or np.any(d >= V):
            raise ValueError("draft token out of range")
        ph = np.nonzero(d == -1)[0]
        Kb = int(ph[0]) if ph.size else K  # drafts end at the first placeholder
        if T == 0.0:
            # greedy: accept while the draft equals the target argmax
            a = [argmax_rule(rows[j]) for j in range(K + 1)]
            n = 0
            while n < Kb and int(draft_tokens[b, n]) == a[n]:
                n += 1
            out[b, :n] = draft_tokens[b, :n]
            out[b, n] = a[n]
            nacc[b] = n
            final_row[b] = n
            smp_margin[b] = top_two_margin(rows[n])
            continue
        tp = None if top_p is None else float(top_p[slot])
        p_rows = []
        for j in range(K + 1):
            pj = _softmax(rows[j].astype(np.float64) / T)
            if tp is not None and tp < 1.0:
                keep, near = top_p_keep(rows[j], T, tp)
                pj = np.where(keep, pj, 0.0)
                pj = pj / pj.sum()
                p_rows.append((pj, near))
            else:
                p_rows.append((pj, False))
        n = 0
        rejected = False
        for k in range(Kb):
            x = int(draft_tokens[b, k])
            cr = bf16_to_f64(cache[crow, k]) if cache_dtype == "bf16" else np.asarray(cache[crow, k], np.float64)
            qk = _softmax(cr / T) if not np.isnan(cr).any() else np.full(V, np.nan)
            pk, near = p_rows[k]
            near_tp[b] |= near
            u = accept_uniform(int(seeds[slot]), int(anchor_pos[b]) + k)
            p32, q32 = np.float32(pk[x]), np.float32(qk[x])
            ok = bool(p32 >= np.float32(np.float32(u) * q32))  # False when q is NaN
            if np.isnan(qk[x]):
                m = np.inf
            elif qk[x] == 0.0:
                m = np.inf
            else:
                m = abs(pk[x] / qk[x] - u)
            acc_margin[b] = min(acc_margin[b], m)
            if not ok:
                rejected = True
                g = gumbel_row(int(seeds[slot]), int(anchor_pos[b]) + k, SALT_RESAMPLE, V)
                if np.isnan(qk).any():
                    r = np.zeros(V)
                else:
                    r = np.maximum(0.0, pk - qk)
                with np.errstate(divide="ignore"):
                    s = (np.log(r) if r.sum() > 0 else np.log(pk)) + g
                out[b, :n] = draft_tokens[b, :n]
                out[b, n] = argmax_rule(s.astype(np.float32))
                smp_margin[b] = top_two_margin(s)
                final_row[b] = k
                break
            n += 1
        if not rejected:
            pK, near = p_rows[Kb]
            near_tp[b] |= near
            g = gumbel_row(int(seeds[slot]), int(anchor_pos[b]) + Kb, SALT_RESAMPLE, V)
            with np.errstate(divide="ignore"):
                s = np.log(pK) + g
            out[b, :Kb] = draft_tokens[b, :Kb]
            out[b, Kb] = argmax_rule(s.astype(np.float32))
            smp_margin[b] = top_two_margin(s)
            final_row[b] = Kb
        nacc[b] = n
    return {"out_tokens": out, "num_accepted": nacc, "accept_margin": acc_margin, "sample_margin": smp_margin,
            "near_top_p": near_tp, "final_row": final_row}
