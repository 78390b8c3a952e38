"""Pins of the oracle's draft LM head (compute_draft_logits on the API page).

Against dot products summed exactly (math.fsum of exact products, correctly
rounded) on small shapes, against unit hidden vectors (which pick single
lm_head entries: a transposed operand or a dropped column fails), and
the bf16 output as the round-to-nearest-even of the float32 one.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
import workloads


def test_logits_equal_exact_dot_products():
    hidden, lm = workloads.make_lm_head(5, 37, 64, seed=2)
    out = oracle.draft_logits(hidden, lm)
    h = workloads.bf16_bits_to_f32(hidden).astype(np.float64)
    w = workloads.bf16_bits_to_f32(lm).astype(np.float64)
    for m in range(5):
        for v in range(37):
            exact = math.fsum(float(a) * float(b) for a, b in zip(h[m], w[v]))
            assert out[m, v] == np.float32(exact), (m, v)


def test_unit_hidden_vectors_pick_lm_head_entries():
    _, lm = workloads.make_lm_head(1, 50, 96, seed=3)
    H = lm.shape[1]
    hidden = np.zeros((4, H), np.uint16)
    picks = [0, 17, 63, 95]
    for m, hcol in enumerate(picks):
        hidden[m, hcol] = 0x3F80  # 1.0
    out = oracle.draft_logits(hidden, lm)
    for m, hcol in enumerate(picks):
        np.testing.assert_array_equal(out[m], workloads.bf16_bits_to_f32(lm[:, hcol]))


def test_column_subset_and_bf16_output():
    hidden, lm = workloads.make_lm_head(7, 300, 128, seed=4)
    full = oracle.draft_logits(hidden, lm)
    cols = np.array([0, 5, 299, 150, 151])
    np.testing.assert_array_equal(oracle.draft_logits(hidden, lm, cols=cols), full[:, cols])
    b = oracle.draft_logits(hidden, lm, out_dtype="bf16")
    np.testing.assert_array_equal(b, workloads.bf16_bits(full))
    _, a = oracle.draft_logits(hidden, lm, want_abs=True)
    assert (a >= np.abs(full.astype(np.float64)) * (1 - 1e-6)).all()


def test_logit_scale():
    hidden, lm = workloads.make_lm_head(16, 2000, 512, seed=5)
    out = oracle.draft_logits(hidden, lm)
    assert 2.7 < out.std() < 3.3
