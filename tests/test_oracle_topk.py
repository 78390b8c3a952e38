"""Pins of the oracle's top-k Markov drafting (the API page's _sample_sequential_topk).

The candidate selection is checked against torch.topk on rows of distinct
values and, with ties, NaN and signed zeros, against the pairwise order it must
respect; the loop against the dense loop (with k = V, and on base logits whose
non-candidates are masked to -inf, the truncated distribution the page feeds
to the unchanged sampler), against k = 1 (the base argmax whatever the noise)
and against the softmax law of the cached row.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
from scipy import special, stats

import oracle
import workloads


def _ranks_above(a: float, ca: int, b: float, cb: int) -> bool:
    """True when entry (a, column ca) comes before (b, column cb) in the selection order."""
    if math.isnan(a) or math.isnan(b):
        if math.isnan(a) and math.isnan(b):
            return ca < cb
        return math.isnan(a)
    if a != b:  # -0.0 == +0.0 here
        return a > b
    return ca < cb


def test_topk_columns_match_torch_on_distinct_values():
    import torch
    rng = np.random.default_rng(1)
    for V, k in [(5, 1), (37, 5), (1000, 64), (4099, 256), (300, 300)]:
        row = rng.permutation(V).astype(np.float64) * 0.25 - 40.0 + rng.uniform(0, 0.2, V)
        ref = torch.topk(torch.from_numpy(row), k).indices.numpy()
        got = oracle.topk_columns(row, k)
        np.testing.assert_array_equal(got, np.sort(ref))


@pytest.mark.parametrize("seed", range(6))
def test_topk_columns_respect_the_order_with_ties(seed):
    rng = np.random.default_rng([seed, 3])
    vals = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1.5, -2.0, 1.5, 7.0])
    V = int(rng.integers(3, 60))
    row = vals[rng.integers(0, vals.size, V)]
    for k in sorted({1, 2, V // 2 or 1, V - 1 or 1, V}):
        got = oracle.topk_columns(row, k)
        assert got.size == k and np.all(np.diff(got) > 0)
        sel = set(got.tolist())
        for s in sel:
            for u in range(V):
                if u not in sel:
                    assert _ranks_above(row[s], s, row[u], u), (row, k, s, u)


def test_topk_columns_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.topk_columns(np.zeros(4), 5)
    with pytest.raises(ValueError):
        oracle.topk_columns(np.zeros(4), 0)


def _run(wl, **kw):
    return oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos,
                             wl.seeds, wl.temperature, wl.cache_dtype, **kw)


@pytest.mark.parametrize("cache_dtype,base_dtype", [("f32", "f32"), ("bf16", "bf16")])
def test_topk_with_k_equal_to_V_is_the_dense_loop(cache_dtype, base_dtype):
    wl = workloads.make_custom(300, 32, 4, 5, seed=2, cache_dtype=cache_dtype, base_dtype=base_dtype)
    wl.temperature[1] = 0.0
    wl.temperature[3] = 0.7
    dense = _run(wl)
    tk = _run(wl, topk=wl.V)
    for key in ("tokens", "cache", "lse", "margin"):
        np.testing.assert_array_equal(tk[key], dense[key])


@pytest.mark.parametrize("k", [1, 3, 40])
@pytest.mark.parametrize("cache_dtype,base_dtype", [("f32", "f32"), ("bf16", "f32"), ("f32", "bf16")])
def test_topk_is_the_dense_loop_on_the_masked_base(k, cache_dtype, base_dtype):
    wl = workloads.make_custom(257, 32, 5, 6, seed=5, cache_dtype=cache_dtype, base_dtype=base_dtype)
    wl.temperature[0] = 0.0
    wl.temperature[2] = 1.8
    base = np.array(wl.draft_base, copy=True)
    if base_dtype == "f32":  # a NaN and an infinity among the base logits
        base[1, 2, 17] = np.nan
        base[4, 0, 200] = np.inf
    wl.base[:, : wl.K] = base
    tk = _run(wl, topk=k)
    masked = np.array(base, copy=True)
    for b in range(wl.B):
        for s in range(wl.K):
            row = workloads.bf16_bits_to_f32(base[b, s]) if base_dtype == "bf16" else base[b, s]
            keep = np.zeros(wl.V, bool)
            keep[oracle.topk_columns(row, k)] = True
            masked[b, s, ~keep] = 0xFF80 if base_dtype == "bf16" else -np.inf  # -inf
    dense = oracle.draft_loop(masked, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, wl.seeds,
                              wl.temperature, wl.cache_dtype)
    for key in ("tokens", "cache", "lse", "margin"):
        np.testing.assert_array_equal(tk[key], dense[key])
    # and the cache holds -inf exactly outside the candidates
    c = workloads.bf16_bits_to_f32(tk["cache"]) if cache_dtype == "bf16" else tk["cache"]
    assert ((c != -np.inf).sum(axis=2) <= k).all()


def test_topk_of_one_is_the_base_argmax():
    wl = workloads.make_custom(1000, 32, 6, 8, seed=9, temperature=2.0)
    wl.temperature[5] = 0.0
    tk = _run(wl, topk=1)
    for b in range(wl.B):
        for s in range(wl.K):
            assert tk["tokens"][b, s] == oracle.argmax_rule(wl.draft_base[b, s])
            assert (tk["cache"][b, s] != -np.inf).sum() == 1


def test_topk_draw_follows_the_softmax_of_the_cached_row():
    rng = np.random.default_rng(4)
    V, r, B, T, k = 12, 32, 20000, 0.8, 5
    z = rng.standard_normal(V).astype(np.float32)
    base = np.broadcast_to(z, (B, 1, V)).copy()
    w1 = workloads.bf16_bits(rng.standard_normal((V, r)).astype(np.float32) * np.float32(0.3))
    w2 = workloads.bf16_bits(rng.standard_normal((V, r)).astype(np.float32) * np.float32(0.3))
    out = oracle.draft_loop(base, "f32", w1, w2, np.full(B, 3, np.int32), np.arange(B) * 7 + 11,
                            np.full(B, 5, np.int64), np.full(B, T, np.float32), "f32", topk=k)
    row = out["cache"][0, 0].astype(np.float64)
    assert (out["cache"] == out["cache"][0]).all()  # same row everywhere
    cand = np.flatnonzero(np.isfinite(row))
    np.testing.assert_array_equal(cand, oracle.topk_columns(z, k))
    counts = np.bincount(out["tokens"][:, 0], minlength=V)
    assert counts[np.setdiff1d(np.arange(V), cand)].sum() == 0
    p = special.softmax(row[cand] / np.float32(T))
    assert stats.chisquare(counts[cand], p * B).pvalue > 1e-4
