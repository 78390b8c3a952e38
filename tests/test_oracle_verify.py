"""Pins of the oracle's rejection verification: the rejection-sampling law
(the emitted token follows the target distribution), the acceptance rate, the
special cases, the greedy textbook rule, and exact top-p."""
import numpy as np
import pytest
from scipy import special, stats

from oracle import verify, top_p_keep, draft_loop
from workloads import bf16_bits


def _chi2_ok(counts, probs, min_p=1e-4):
    exp = probs * counts.sum()
    keep = exp > 5
    obs = counts[keep]
    if keep.sum() < 2:  # a single likely outcome: everything must land there
        return obs.sum() == counts.sum()
    e = exp[keep] * obs.sum() / exp[keep].sum()
    return stats.chisquare(obs, e).pvalue > min_p


def _verify_one_step(t0, t1, c0, draft, T, seeds, pos, top_p=None):
    """B requests with K=1: target rows (t0, t1), cache row c0, draft token per request."""
    B = draft.size
    target = np.stack([np.broadcast_to(t0, (B, t0.size)), np.broadcast_to(t1, (B, t1.size))], 1)
    target = target.reshape(B * 2, -1).astype(np.float32)
    cache = np.broadcast_to(c0, (B, 1, c0.size)).astype(np.float32).copy()
    tp = None if top_p is None else np.full(B, top_p, np.float32)
    return verify(target, cache, "f32", draft.reshape(B, 1), np.full(B, T, np.float32), tp, seeds, pos)


PAIRS = {
    "random": (np.array([0.3, -1.0, 2.0, 0.1, -0.5, 1.2, 0.0, -2.0]), np.array([1.0, 0.5, -0.5, 0.2, 2.0, -1.0, 0.3, 0.0])),
    "equal": (np.array([0.3, -1.0, 2.0, 0.1, -0.5, 1.2, 0.0, -2.0]),) * 2,
    "disjoint": (np.array([5.0, 5.0, 5.0, 5.0, -30, -30, -30, -30]), np.array([-30, -30, -30, -30, 5.0, 5.0, 5.0, 5.0])),
    "onehot_p": (np.array([0.0, 0, 0, 0, 0, 0, 40.0, 0]), np.array([1.0, 0.5, -0.5, 0.2, 2.0, -1.0, 0.3, 0.0])),
}


@pytest.mark.parametrize("name", sorted(PAIRS))
def test_rejection_output_follows_target(name):
    t0, c0 = (np.asarray(x, np.float32) for x in PAIRS[name])
    T = 0.9
    B = 20000
    rng = np.random.default_rng(10)
    p = special.softmax(t0.astype(np.float64) / np.float32(T))
    q = special.softmax(c0.astype(np.float64) / np.float32(T))
    draft = rng.choice(8, size=B, p=q)  # draft token drawn from q by an independent generator
    seeds = rng.integers(0, 2**63, B, dtype=np.int64)
    res = _verify_one_step(t0, t0, c0, draft, T, seeds, rng.integers(0, 2**40, B))
    first = res["out_tokens"][:, 0]
    assert _chi2_ok(np.bincount(first, minlength=8), p)
    # acceptance probability = sum_v min(p, q)
    acc = res["num_accepted"].mean()
    want = np.minimum(p, q).sum()
    assert abs(acc - want) <= 5 * np.sqrt(want * (1 - want) / B) + 1e-12


def test_equal_distributions_always_accept():
    t = np.array([0.3, -1.0, 2.0, 0.1], np.float32)
    B = 2000
    rng = np.random.default_rng(11)
    res = _verify_one_step(t, t, t, rng.integers(0, 4, B), 1.0, rng.integers(0, 2**63, B, dtype=np.int64),
                           rng.integers(0, 2**40, B))
    assert np.all(res["num_accepted"] == 1)


def test_zero_target_mass_always_rejects_and_emits_the_target_mode():
    t = np.array([0.0, 0.0, 0.0, 200.0], np.float32)  # p is one-hot at 3 in float64
    c = np.array([1.0, 0.0, 0.5, 0.2], np.float32)
    B = 500
    rng = np.random.default_rng(12)
    res = _verify_one_step(t, t, c, rng.integers(0, 3, B), 1.0, rng.integers(0, 2**63, B, dtype=np.int64),
                           rng.integers(0, 2**40, B))
    assert np.all(res["num_accepted"] == 0)
    assert np.all(res["out_tokens"][:, 0] == 3)
    assert np.all(res["out_tokens"][:, 1] == -1)


def test_one_hot_draft_accepts_with_target_probability():
    # q one-hot at x: accept iff u <= p(x)
    t = np.array([0.0, 1.0, -1.0, 0.5], np.float32)
    c = np.array([0.0, 0.0, 300.0, 0.0], np.float32)
    B = 20000
    rng = np.random.default_rng(13)
    res = _verify_one_step(t, t, c, np.full(B, 2), 1.0, rng.integers(0, 2**63, B, dtype=np.int64),
                           rng.integers(0, 2**40, B))
    p2 = special.softmax(t.astype(np.float64))[2]
    acc = res["num_accepted"].mean()
    assert abs(acc - p2) <= 5 * np.sqrt(p2 * (1 - p2) / B)


def test_bonus_token_follows_last_target_row():
    t0 = np.array([0.3, -1.0, 2.0, 0.1, 0.0, 0.0, 0.0, 0.0], np.float32)
    t1 = np.array([1.5, 0.0, -1.0, 0.5, 0.7, -0.2, 0.9, 0.1], np.float32)
    B = 20000
    rng = np.random.default_rng(14)
    res = _verify_one_step(t0, t1, t0, rng.integers(0, 8, B), 1.2, rng.integers(0, 2**63, B, dtype=np.int64),
                           rng.integers(0, 2**40, B))
    assert np.all(res["num_accepted"] == 1)
    p1 = special.softmax(t1.astype(np.float64) / np.float32(1.2))
    assert _chi2_ok(np.bincount(res["out_tokens"][:, 1], minlength=8), p1)


def test_nan_draft_row_is_rejected_and_resampled_from_target():
    t = np.array([0.3, -1.0, 2.0, 0.1], np.float32)
    c = np.array([0.0, np.nan, 1.0, 0.0], np.float32)
    B = 20000
    rng = np.random.default_rng(15)
    res = _verify_one_step(t, t, c, rng.integers(0, 4, B), 1.0, rng.integers(0, 2**63, B, dtype=np.int64),
                           rng.integers(0, 2**40, B))
    assert np.all(res["num_accepted"] == 0)
    assert _chi2_ok(np.bincount(res["out_tokens"][:, 0], minlength=4), special.softmax(t.astype(np.float64)))


def test_greedy_rows_follow_target_argmax():
    rng = np.random.default_rng(16)
    B, K, V = 50, 4, 40
    target = rng.standard_normal((B * (K + 1), V)).astype(np.float32)
    am = target.reshape(B, K + 1, V).argmax(-1)
    draft = am[:, :K].copy()
    n_ok = rng.integers(0, K + 1, B)  # accept exactly n_ok drafts
    for b in range(B):
        if n_ok[b] < K:
            draft[b, n_ok[b]] = (am[b, n_ok[b]] + 1) % V
            draft[b, n_ok[b] + 1:] = rng.integers(0, V, K - n_ok[b] - 1)
    cache = np.full((B, K, V), np.nan, np.float32)  # never read at T=0
    res = verify(target, cache, "f32", draft, np.zeros(B, np.float32), None, np.zeros(B, np.int64),
                 np.zeros(B, np.int64))
    assert np.array_equal(res["num_accepted"], n_ok)
    for b in range(B):
        n = n_ok[b]
        assert list(res["out_tokens"][b, :n]) == list(am[b, :n])
        assert res["out_tokens"][b, n] == am[b, n]
        assert np.all(res["out_tokens"][b, n + 1:] == -1)


def test_rejection_law_with_top_p():
    # with top-p the emitted token follows the renormalised kept distribution
    t0 = np.array([2.0, 1.5, 1.0, 0.5, 0.0, -0.5, -1.0, -1.5], np.float32)
    c0 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 0.0, 0.0, 0.0], np.float32)
    T, top_p = 1.0, 0.8
    keep, near = top_p_keep(t0, T, top_p)
    assert not near
    p = special.softmax(t0.astype(np.float64)) * keep
    p /= p.sum()
    B = 20000
    rng = np.random.default_rng(17)
    q = special.softmax(c0.astype(np.float64))
    res = _verify_one_step(t0, t0, c0, rng.choice(8, size=B, p=q), T, rng.integers(0, 2**63, B, dtype=np.int64),
                           rng.integers(0, 2**40, B), top_p=top_p)
    counts = np.bincount(res["out_tokens"][:, 0], minlength=8)
    assert np.all(counts[~keep] == 0)
    assert _chi2_ok(counts, p)


def _lm_like_row(rng, V):
    x = rng.standard_normal(V) * 2 + 8 * (rng.random(V) < 0.01)
    return bf16_bits(x.astype(np.float32)).astype(np.uint32) << 16


def _row_families(rng, V):
    yield "lm_bf16", (_lm_like_row(rng, V)).view(np.float32)
    yield "quarter_ties", (np.round(rng.standard_normal(V) * 8) / 4).astype(np.float32)
    x = (rng.standard_normal(V) * 2).astype(np.float32)
    x[rng.random(V) < 0.3] = -np.inf
    yield "neg_inf_30pct", x
    x = (rng.standard_normal(V) * 0.5).astype(np.float32)
    x[rng.integers(0, V)] = 12.0
    yield "peaked", x
    yield "flat", np.zeros(V, np.float32)


@pytest.mark.parametrize("p", [0.01, 0.5, 0.9, 0.95, 0.99, 0.9999, 1 - 1e-7])
def test_top_p_matches_threshold_formulation(p):
    # Independent formulation: column v is kept iff the mass of all columns
    # ahead of it in the (logit desc, id asc) order is < p; the row max is kept.
    rng = np.random.default_rng(int(p * 1e6))
    V = 600
    ids = np.arange(V)
    for name, t in _row_families(rng, V):
        for T in (1.0, 0.7):
            keep, near = top_p_keep(t, T, p)
            if near:
                continue
            probs = special.softmax(t.astype(np.float64) / T)
            ahead = (t[None, :] > t[:, None]) | ((t[None, :] == t[:, None]) & (ids[None, :] < ids[:, None]))
            mass_ahead = (ahead * probs[None, :]).sum(1)
            want = mass_ahead < p
            want[np.argmax(t)] = True
            assert np.array_equal(keep, want), (name, T, p)
            # minimality: the kept mass reaches p, and not without its smallest member
            assert probs[keep].sum() >= p - 1e-12 or keep.all()


def test_top_p_one_disables_and_zero_keeps_max():
    t = np.array([0.1, 3.0, 3.0, -1.0], np.float32)
    assert top_p_keep(t, 1.0, 1.0)[0].all()
    k0, _ = top_p_keep(t, 1.0, 0.0)
    assert k0.tolist() == [False, True, False, False]


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_whole_pipeline_first_token_follows_target(T):
    # Markov draft (tiny vocabulary) + verification: the first emitted token
    # follows the target's first distribution, and a second emitted token
    # (present when the first draft was accepted) follows the second one.
    rng = np.random.default_rng(18)
    V, r, B, K = 6, 32, 30000, 2
    w1, w2 = bf16_bits(rng.standard_normal((V, r)).astype(np.float32) * 0.3), bf16_bits(
        rng.standard_normal((V, r)).astype(np.float32) * 0.3)
    base_row = rng.standard_normal((K + 1, V)).astype(np.float32)
    base = np.broadcast_to(base_row, (B, K + 1, V)).copy()
    tgt_rows = (base_row + rng.standard_normal((K + 1, V)).astype(np.float32) * 0.7).astype(np.float32)
    target = np.broadcast_to(tgt_rows, (B, K + 1, V)).reshape(B * (K + 1), V).copy()
    seeds = rng.integers(0, 2**63, B, dtype=np.int64)
    pos = rng.integers(1, 2**30, B)
    temps = np.full(B, T, np.float32)
    d = draft_loop(base[:, :K], "f32", w1, w2, np.full(B, 1), pos, seeds, temps, "f32")
    v = verify(target, d["cache"], "f32", d["tokens"], temps, None, seeds, pos)
    p0 = special.softmax(tgt_rows[0].astype(np.float64) / np.float32(T))
    p1 = special.softmax(tgt_rows[1].astype(np.float64) / np.float32(T))
    assert _chi2_ok(np.bincount(v["out_tokens"][:, 0], minlength=V), p0)
    sel = v["num_accepted"] >= 1
    assert sel.sum() > 2000
    assert _chi2_ok(np.bincount(v["out_tokens"][sel, 1], minlength=V), p1)


# Rows with no finite logit (every column masked, -inf): the winner rule gives
# such a row column 0, and its distribution is read as the one-hot there.

def test_no_finite_target_row_keeps_column_zero_under_top_p():
    z = np.full(37, -np.inf, np.float32)
    for p in (0.01, 0.5, 0.95, 1 - 1e-7):
        keep, _ = top_p_keep(z, np.float32(0.8), np.float32(p))
        assert keep[0] and keep.sum() == 1


def test_no_finite_target_rows_emit_column_zero():
    # every target row masked: p is the one-hot at 0. A draft of 0 is always
    # accepted (p(0) = 1 >= u q(0)), any other draft with q > 0 always rejected,
    # and the final token (residual or bonus) is 0 in both cases.
    z = np.full(8, -np.inf, np.float32)
    c0 = np.array([0.3, -1.0, 2.0, 0.1, -0.5, 1.2, 0.0, -2.0], np.float32)
    rng = np.random.default_rng(3)
    B = 200
    seeds = rng.integers(0, 2**63, B, dtype=np.int64)
    pos = rng.integers(0, 2**40, B)
    draft = rng.integers(0, 8, B)
    res = _verify_one_step(z, z, c0, draft, 1.0, seeds, pos)
    n = res["num_accepted"]
    assert np.array_equal(n, (draft == 0).astype(np.int32))
    out = res["out_tokens"]
    for b in range(B):
        assert out[b, n[b]] == 0
        assert not np.isnan(res["accept_margin"][b])


def test_no_finite_draft_row_accepts_with_target_probability():
    # a masked cache row makes q the one-hot at 0 (draft token 0): accept iff
    # p(0) >= u, i.e. with probability p(0); a rejection resamples from
    # max(0, p - q), which is p without column 0
    t0 = np.array([0.5, 1.0, -0.5, 0.2, 1.5, -1.0, 0.0, 0.3], np.float32)
    z = np.full(8, -np.inf, np.float32)
    T = 1.0
    B = 20000
    rng = np.random.default_rng(4)
    seeds = rng.integers(0, 2**63, B, dtype=np.int64)
    res = _verify_one_step(t0, t0, z, np.zeros(B, np.int64), T, seeds, rng.integers(0, 2**40, B))
    p = special.softmax(t0.astype(np.float64) / T)
    acc = res["num_accepted"].mean()
    assert abs(acc - p[0]) <= 5 * np.sqrt(p[0] * (1 - p[0]) / B)
    first = res["out_tokens"][:, 0]
    # overall the first emitted token still follows p
    assert _chi2_ok(np.bincount(first, minlength=8), p)
    rej = res["num_accepted"] == 0
    assert np.all(first[rej] != 0)


def test_no_finite_rows_on_both_sides():
    # p and q both the one-hot at 0: the draft 0 is accepted; a bonus from the
    # masked last row is 0 again
    z = np.full(8, -np.inf, np.float32)
    res = _verify_one_step(z, z, z, np.zeros(5, np.int64), 0.7, np.arange(5), np.arange(5) * 11)
    assert np.all(res["num_accepted"] == 1)
    assert np.all(res["out_tokens"] == 0)
