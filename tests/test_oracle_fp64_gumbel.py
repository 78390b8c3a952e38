"""Pins of the oracle's fp64 Gumbel option (the API page's use_fp64_gumbel).

The float64 scores are checked against a 60-digit decimal evaluation of
z / T - ln(-ln u) from the Philox words themselves, the decisions against the
float32 mode wherever float32 rounding cannot matter, and the draw's law
against softmax(z / T).
"""
from __future__ import annotations

import decimal

import numpy as np
import pytest
from scipy import special, stats

import oracle
import workloads
from oracle.noise import SALT_DRAFT, noise_words, uniform24


def _score_decimal(z32: float, T: float, u: float) -> float:
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        g = -((-(decimal.Decimal(u).ln())).ln())
        return float(decimal.Decimal(float(z32)) / decimal.Decimal(float(T)) + g)


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_fp64_scores_match_decimal(T):
    wl = workloads.make_custom(513, 32, 2, 2, seed=4, temperature=T)
    d = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, wl.seeds,
                          wl.temperature, wl.cache_dtype, want_scores=True, fp64_gumbel=True)
    cols = np.array([0, 1, 2, 3, 4, 255, 256, 511, 512])
    for b in range(wl.B):
        for k in range(wl.K):
            words = noise_words(int(wl.seeds[b]), int(wl.anchor_pos[b]) + k, SALT_DRAFT, cols)
            u = uniform24(words)
            z = d["cache"][b, k, cols]  # float32 biased logits
            for j, c in enumerate(cols):
                ref = _score_decimal(z[j], np.float32(T), float(u[j]))
                assert abs(d["scores"][b, k, c] - ref) <= 4e-16 * max(1.0, abs(ref))


def test_fp64_and_fp32_modes_agree_outside_float32_rounding():
    wl = workloads.make_custom(4099, 64, 4, 6, seed=8, temperature=0.8)
    wl.temperature[2] = 0.0  # greedy rows are unaffected
    a = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, wl.seeds,
                          wl.temperature, wl.cache_dtype, want_scores=True)
    t = a["tokens"]  # teacher-force both runs on the same chain
    b = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, wl.seeds,
                          wl.temperature, wl.cache_dtype, want_scores=True, fp64_gumbel=True, teacher=t)
    a = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, wl.seeds,
                          wl.temperature, wl.cache_dtype, want_scores=True, teacher=t)
    # float32 scores are z/T and g each rounded to float32, then added in
    # float32: within a few float32 ulps of the larger term of the float64 sum
    s64, s32 = b["scores"], a["scores"].astype(np.float64)
    zt = a["cache"].astype(np.float64) / wl.temperature[:, None, None].astype(np.float64)
    samp = wl.temperature > 0
    big = np.maximum(np.abs(zt), np.abs(s64 - zt))[samp]
    assert np.all(np.abs(s64 - s32)[samp] <= 3 * np.spacing(big.astype(np.float32)).astype(np.float64))
    clear = a["margin"] > 1e-4
    assert clear.mean() > 0.9
    np.testing.assert_array_equal(a["tokens"][clear], b["tokens"][clear])
    np.testing.assert_array_equal(a["cache"], b["cache"])
    np.testing.assert_array_equal(a["lse"], b["lse"])
    np.testing.assert_array_equal(a["tokens"][2], b["tokens"][2])


def test_fp64_gumbel_max_law():
    rng = np.random.default_rng(9)
    V, r, B, T = 8, 32, 30000, 0.9
    z = np.array([1.0, 0.0, -1.0, 2.0, 0.5, 0.5, -3.0, 1.5], np.float32)
    base = np.broadcast_to(z, (B, 1, V)).copy()
    w1 = np.zeros((V, r), np.uint16)
    w2 = workloads.bf16_bits(rng.standard_normal((V, r)).astype(np.float32))
    out = oracle.draft_loop(base, "f32", w1, w2, np.zeros(B, np.int32), np.arange(B) * 5 + 3, np.full(B, 77),
                            np.full(B, T, np.float32), "f32", fp64_gumbel=True)
    counts = np.bincount(out["tokens"][:, 0], minlength=V)
    p = special.softmax(z.astype(np.float64) / np.float32(T))
    assert stats.chisquare(counts, p * B).pvalue > 1e-4
