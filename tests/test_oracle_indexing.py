"""Pins of the oracle's request-state indexing, padding rows and -1 placeholder drafts.

Each case reduces to a plain (un-indexed) oracle run on a permuted, truncated
or shifted problem, whose own pins live in test_oracle_draft.py and
test_oracle_verify.py: a mistake in the slot, row or position bookkeeping
(a wrong index, a dropped padding guard, an off-by-one in the placeholder cut)
fails one of them.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads

V, R, K, B = 600, 32, 4, 6


def _wl(temperature=1.0, cache_dtype="f32", base_dtype="f32", seed=3):
    wl = workloads.make_custom(V, R, K, B, seed=seed, temperature=temperature, cache_dtype=cache_dtype,
                               base_dtype=base_dtype)
    wl.temperature[1] = 0.0  # one greedy request
    wl.temperature[2] = 0.6
    return wl


def _plain(wl, **kw):
    return oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos,
                             wl.seeds, wl.temperature, wl.cache_dtype, **kw)


def _state(wl, n_slots, perm):
    """Slot arrays holding request b's state at slot perm[b] (other slots: junk)."""
    rng = np.random.default_rng(11)
    temp = rng.uniform(0.3, 2.0, n_slots).astype(np.float32)
    seeds = rng.integers(0, 2**63, n_slots, dtype=np.int64)
    temp[perm] = wl.temperature
    seeds[perm] = wl.seeds
    return temp, seeds


@pytest.mark.parametrize("cache_dtype", ["f32", "bf16"])
def test_indexed_draft_equals_plain_draft_on_permuted_state(cache_dtype):
    wl = _wl(cache_dtype=cache_dtype)
    plain = _plain(wl)
    n_slots, n_rows = 11, 9
    perm = np.array([7, 2, 9, 0, 5, 3])  # request b -> slot
    rowmap = np.array([8, 6, 1, 4, 2, 7, 0, 3, 5, 6, 4])  # slot -> cache row (slots 1, 4, 6, 8, 10 unused)
    temp, seeds = _state(wl, n_slots, perm)
    idx = np.repeat(perm[:, None], K, axis=1)
    spos = wl.anchor_pos[:, None] + 1 + np.arange(K)[None, :]
    init = np.full((n_rows, K, V), 7, np.uint16 if cache_dtype == "bf16" else np.float32)
    d = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, np.zeros(B, np.int64),
                          seeds, temp, wl.cache_dtype, idx_map=idx, row_mapping=rowmap, sample_pos=spos,
                          cache_init=init)
    np.testing.assert_array_equal(d["tokens"], plain["tokens"])
    np.testing.assert_array_equal(d["lse"], plain["lse"])
    written = rowmap[perm]
    for b in range(B):
        np.testing.assert_array_equal(d["cache"][written[b]], plain["cache"][b])
    untouched = np.setdiff1d(np.arange(n_rows), written)
    assert untouched.size == n_rows - B
    assert (d["cache"][untouched] == 7).all()


def test_sample_pos_keys_the_draw_by_the_position_before_the_token():
    wl = _wl()
    shift = 12345
    plain_shifted = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens,
                                      wl.anchor_pos + shift, wl.seeds, wl.temperature, wl.cache_dtype)
    idx = np.repeat(np.arange(B)[:, None], K, axis=1)
    spos = wl.anchor_pos[:, None] + 1 + shift + np.arange(K)[None, :]
    d = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, wl.seeds,
                          wl.temperature, wl.cache_dtype, idx_map=idx, sample_pos=spos,
                          cache_init=np.zeros((B, K, V), np.float32))
    np.testing.assert_array_equal(d["tokens"], plain_shifted["tokens"])
    # and the unshifted keys give different draws for the sampled requests
    plain = _plain(wl)
    assert (plain["tokens"][wl.temperature > 0] != d["tokens"][wl.temperature > 0]).any()


def test_padding_rows_are_inert_and_leave_other_rows_unchanged():
    wl = _wl()
    plain = _plain(wl)
    pad = [1, 4]
    idx = np.repeat(np.arange(B)[:, None], K, axis=1)
    idx[pad] = -1
    init = np.full((B, K, V), -3.5, np.float32)
    d = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, wl.seeds,
                          wl.temperature, wl.cache_dtype, idx_map=idx, cache_init=init)
    live = np.setdiff1d(np.arange(B), pad)
    assert (d["tokens"][pad] == -1).all()
    assert np.isnan(d["lse"][pad]).all()
    assert (d["cache"][pad] == -3.5).all()
    np.testing.assert_array_equal(d["tokens"][live], plain["tokens"][live])
    np.testing.assert_array_equal(d["cache"][live], plain["cache"][live])
    assert not d["bad_prev"]


def test_inert_step_followed_by_live_step_uses_token_zero():
    wl = _wl()
    idx = np.repeat(np.arange(B)[:, None], K, axis=1)
    idx[3, 1] = -1
    init = np.zeros((B, K, V), np.float32)
    d = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, wl.seeds,
                          wl.temperature, wl.cache_dtype, idx_map=idx, cache_init=init)
    assert d["bad_prev"]
    assert d["tokens"][3, 1] == -1
    # step 2 of request 3 is the plain step from previous token 0
    teacher = _plain(wl)["tokens"].copy()
    teacher[3, 1] = 0
    t = _plain(wl, teacher=teacher)
    assert d["tokens"][3, 2] == t["tokens"][3, 2]
    np.testing.assert_array_equal(d["cache"][3, 2], t["cache"][3, 2])


def _verify_plain(wl, cache, drafts, K_=None, rows=None):
    Kx = K if K_ is None else K_
    tgt = wl.target.reshape(B, K + 1, V)[:, : Kx + 1].reshape(B * (Kx + 1), V)
    return oracle.verify(tgt, cache[:, :Kx], wl.cache_dtype, drafts[:, :Kx], wl.temperature, None, wl.seeds,
                         wl.anchor_pos)


@pytest.mark.parametrize("m", [0, 1, 3])
def test_placeholder_drafts_equal_the_truncated_problem(m):
    wl = _wl()
    d = _plain(wl)
    drafts = d["tokens"].copy()
    drafts[:, m:] = -1
    full = oracle.verify(wl.target, d["cache"], wl.cache_dtype, drafts, wl.temperature, None, wl.seeds,
                         wl.anchor_pos)
    short = _verify_plain(wl, d["cache"], d["tokens"], K_=m)
    np.testing.assert_array_equal(full["num_accepted"], short["num_accepted"])
    np.testing.assert_array_equal(full["out_tokens"][:, : m + 1], short["out_tokens"])
    assert (full["out_tokens"][:, m + 1:] == -1).all()


def test_placeholders_per_request():
    wl = _wl()
    d = _plain(wl)
    drafts = d["tokens"].copy()
    cut = [4, 0, 2, 1, 3, 4]
    for b, m in enumerate(cut):
        drafts[b, m:] = -1
    full = oracle.verify(wl.target, d["cache"], wl.cache_dtype, drafts, wl.temperature, None, wl.seeds,
                         wl.anchor_pos)
    for m in set(cut):
        short = _verify_plain(wl, d["cache"], d["tokens"], K_=m)
        for b in [b for b, c in enumerate(cut) if c == m]:
            assert full["num_accepted"][b] == short["num_accepted"][b]
            np.testing.assert_array_equal(full["out_tokens"][b, : m + 1], short["out_tokens"][b])


def test_indexed_verify_equals_plain_verify_with_padding():
    wl = _wl()
    d = _plain(wl)
    plain = oracle.verify(wl.target, d["cache"], wl.cache_dtype, d["tokens"], wl.temperature, None, wl.seeds,
                          wl.anchor_pos)
    n_slots, n_rows = 10, 8
    perm = np.array([6, -1, 1, 9, -1, 0])  # requests 1 and 4 are padding
    rowmap = np.array([5, 2, 0, 0, 0, 0, 7, 0, 0, 3])
    temp, seeds = _state(wl, n_slots, np.where(perm >= 0, perm, 0))
    temp[perm[perm >= 0]] = wl.temperature[perm >= 0]
    seeds[perm[perm >= 0]] = wl.seeds[perm >= 0]
    big = np.full((n_rows, K, V), np.nan, np.float32)
    for b in range(B):
        if perm[b] >= 0:
            big[rowmap[perm[b]]] = d["cache"][b]
    v = oracle.verify(wl.target, big, wl.cache_dtype, d["tokens"], temp, None, seeds, wl.anchor_pos,
                      idx_map=perm, row_mapping=rowmap)
    for b in range(B):
        if perm[b] < 0:
            assert (v["out_tokens"][b] == -1).all() and v["num_accepted"][b] == 0
        else:
            np.testing.assert_array_equal(v["out_tokens"][b], plain["out_tokens"][b])
            assert v["num_accepted"][b] == plain["num_accepted"][b]


def test_out_of_range_drafts_other_than_minus_one_are_rejected():
    wl = _wl()
    d = _plain(wl)
    drafts = d["tokens"].copy()
    drafts[0, 1] = -2
    with pytest.raises(ValueError):
        oracle.verify(wl.target, d["cache"], wl.cache_dtype, drafts, wl.temperature, None, wl.seeds, wl.anchor_pos)
