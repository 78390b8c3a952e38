"""Pins of the oracle's Markov draft loop: projection special cases, the
Gumbel-max sampling law, the Markov chain law and the position keying."""
import numpy as np
import pytest
from scipy import special, stats

from oracle import draft_loop, bf16_to_f64
from workloads import bf16_bits, bf16_bits_to_f32


def _bits(x):
    return bf16_bits(np.asarray(x, np.float32))


def _run(base, w1, w2, anchors, pos, seeds, temps, cache_dtype="f32", base_dtype="f32", **kw):
    return draft_loop(base, base_dtype, w1, w2, np.asarray(anchors), np.asarray(pos), np.asarray(seeds),
                      np.asarray(temps, np.float32), cache_dtype, **kw)


def test_zero_embedding_leaves_base_in_cache():
    rng = np.random.default_rng(0)
    V, r, B, K = 300, 32, 3, 1
    w1 = _bits(rng.standard_normal((V, r)))
    w1[[5, 17, 200]] = 0  # anchors embed to the zero vector
    w2 = _bits(rng.standard_normal((V, r)))
    base = rng.standard_normal((B, K, V)).astype(np.float32)
    out = _run(base, w1, w2, [5, 17, 200], [1, 2, 3], [1, 2, 3], [1.0, 0.0, 0.7])
    assert np.array_equal(out["cache"][:, 0], base[:, 0])
    assert out["tokens"][1, 0] == np.argmax(base[1, 0])  # greedy: plain argmax


def test_one_hot_embedding_selects_a_w2_column():
    rng = np.random.default_rng(1)
    V, r = 257, 64
    w1 = np.zeros((V, r), np.uint16)
    j = 37
    w1[11, j] = _bits([1.0])[0]
    w2 = _bits(rng.standard_normal((V, r)))
    base = rng.standard_normal((1, 1, V)).astype(np.float32)
    out = _run(base, w1, w2, [11], [9], [4], [1.0])
    want = (base[0, 0].astype(np.float64) + bf16_bits_to_f32(w2[:, j])).astype(np.float32)
    assert np.array_equal(out["cache"][0, 0], want)


def test_bias_is_full_precision_projection():
    # bias = w2 @ w1[prev] in float64 (library matmul on the exactly widened
    # bf16 values), then z rounded once to float32
    rng = np.random.default_rng(2)
    V, r = 500, 96
    w1, w2 = _bits(rng.standard_normal((V, r)) * 0.1), _bits(rng.standard_normal((V, r)) * 0.1)
    base = rng.standard_normal((1, 1, V)).astype(np.float32)
    out = _run(base, w1, w2, [3], [0], [0], [1.0])
    bias = bf16_to_f64(w2) @ bf16_to_f64(w1[3])
    assert np.array_equal(out["cache"][0, 0], (base[0, 0].astype(np.float64) + bias).astype(np.float32))


def test_bf16_cache_is_rounded_biased_logit():
    import torch
    rng = np.random.default_rng(3)
    V, r = 400, 32
    w1, w2 = _bits(rng.standard_normal((V, r))), _bits(rng.standard_normal((V, r)))
    base_bits = _bits(rng.standard_normal((2, 1, V)) * 4)
    out_f = _run(bf16_bits_to_f32(base_bits), w1, w2, [1, 2], [0, 0], [0, 1], [1.0, 1.0], cache_dtype="f32")
    out_b = _run(base_bits, w1, w2, [1, 2], [0, 0], [0, 1], [1.0, 1.0], cache_dtype="bf16", base_dtype="bf16")
    want = torch.from_numpy(out_f["cache"]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out_b["cache"], want)
    assert np.array_equal(out_b["tokens"], out_f["tokens"])  # same z, same scores


def test_lse_matches_scipy():
    rng = np.random.default_rng(4)
    V, r = 1000, 32
    w1, w2 = _bits(rng.standard_normal((V, r)) * 0.2), _bits(rng.standard_normal((V, r)) * 0.2)
    base = (rng.standard_normal((2, 2, V)) * 3).astype(np.float32)
    out = _run(base, w1, w2, [1, 2], [5, 6], [0, 1], [0.7, 0.0])
    want = special.logsumexp(out["cache"][0].astype(np.float64) / np.float64(np.float32(0.7)), axis=-1)
    assert np.allclose(out["lse"][0], want, rtol=1e-13)
    assert np.all(np.isnan(out["lse"][1]))  # greedy rows carry no draft distribution


def _chi2_ok(counts, probs, min_p=1e-4):
    exp = probs * counts.sum()
    keep = exp > 5
    obs = counts[keep]
    if keep.sum() < 2:  # a single likely outcome: everything must land there
        return obs.sum() == counts.sum()
    e = exp[keep] * obs.sum() / exp[keep].sum()
    return stats.chisquare(obs, e).pvalue > min_p


@pytest.mark.parametrize("T", [1.0, 0.6, 1.7])
def test_gumbel_max_law(T):
    # With w2 = 0 the score is base/T + g, so a draw must follow softmax(base/T).
    rng = np.random.default_rng(5)
    V, r, B = 8, 32, 30000
    z = np.array([1.0, 0.0, -1.0, 2.0, 0.5, 0.5, -3.0, 1.5], np.float32)
    base = np.broadcast_to(z, (B, 1, V)).copy()
    w1 = np.zeros((V, r), np.uint16)
    w2 = _bits(rng.standard_normal((V, r)))
    out = _run(base, w1, w2, np.zeros(B, int), np.arange(B) * 3 + 11, np.full(B, 99), np.full(B, T))
    counts = np.bincount(out["tokens"][:, 0], minlength=V)
    assert _chi2_ok(counts, special.softmax(z.astype(np.float64) / np.float32(T)))


def test_markov_chain_joint_law():
    # P(x0, x1) = softmax((b0 + W2 w1[a]) / T)[x0] * softmax((b1 + W2 w1[x0]) / T)[x1]
    rng = np.random.default_rng(6)
    V, r, B, T = 4, 32, 24000, 0.8
    w1 = _bits(rng.standard_normal((V, r)) * 0.7)
    w2 = _bits(rng.standard_normal((V, r)) * 0.7)
    b0 = np.array([0.2, -0.4, 0.9, 0.0], np.float32)
    b1 = np.array([-0.3, 0.6, 0.1, 0.4], np.float32)
    base = np.broadcast_to(np.stack([b0, b1])[None], (B, 2, V)).copy()
    seeds = rng.integers(0, 2**63, B, dtype=np.int64)
    out = _run(base, w1, w2, np.full(B, 2), np.full(B, 1000), seeds, np.full(B, T))
    W1, W2 = bf16_to_f64(w1), bf16_to_f64(w2)

    def step_probs(brow, prev):
        z = (brow.astype(np.float64) + W2 @ W1[prev]).astype(np.float32)
        return special.softmax(z.astype(np.float64) / np.float32(T))

    p0 = step_probs(b0, 2)
    joint = np.array([[p0[i] * step_probs(b1, i)[j] for j in range(V)] for i in range(V)]).ravel()
    counts = np.bincount(out["tokens"][:, 0] * V + out["tokens"][:, 1], minlength=V * V)
    assert _chi2_ok(counts, joint)
    # the step-1 law really depends on the previous token: the conditional
    # rows differ by far more than sampling noise
    cond = np.array([step_probs(b1, i) for i in range(V)])
    assert np.abs(cond[:, None] - cond[None]).max() > 0.2


def test_steps_are_keyed_by_position_before_the_token():
    # Draft step k predicts position P0+1+k and is keyed P0+k: with no bias
    # and equal base rows, step k at anchor position P equals step 0 at P+k.
    rng = np.random.default_rng(7)
    V, r, B, K = 512, 32, 6, 4
    w1 = np.zeros((V, r), np.uint16)
    w2 = _bits(rng.standard_normal((V, r)))
    row = rng.standard_normal(V).astype(np.float32)
    base = np.broadcast_to(row, (B, K, V)).copy()
    seeds = rng.integers(0, 2**63, B, dtype=np.int64)
    pos = rng.integers(10, 1000, B)
    full = _run(base, w1, w2, np.zeros(B, int), pos, seeds, np.ones(B))["tokens"]
    for k in range(K):
        one = _run(base[:, :1], w1, w2, np.zeros(B, int), pos + k, seeds, np.ones(B))["tokens"][:, 0]
        assert np.array_equal(full[:, k], one)
    # and steps use different draws: identical rows still give varied tokens
    assert len(set(full.ravel().tolist())) > B


def test_nan_column_wins_and_first_nan_is_taken():
    rng = np.random.default_rng(8)
    V, r = 2000, 32
    w1, w2 = _bits(rng.standard_normal((V, r))), _bits(rng.standard_normal((V, r)))
    base = rng.standard_normal((2, 1, V)).astype(np.float32)
    base[:, 0, [1500, 700]] = np.nan
    out = _run(base, w1, w2, [0, 1], [3, 3], [1, 2], [1.0, 0.0])
    assert out["tokens"][:, 0].tolist() == [700, 700]
    assert np.isnan(out["lse"][0, 0])


def test_teacher_forcing_replaces_previous_token():
    rng = np.random.default_rng(9)
    V, r, B, K = 300, 32, 2, 3
    w1, w2 = _bits(rng.standard_normal((V, r))), _bits(rng.standard_normal((V, r)))
    base = rng.standard_normal((B, K, V)).astype(np.float32)
    args = (base, w1, w2, [3, 4], [10, 20], [5, 6], [1.0, 1.0])
    free = _run(*args)
    teach = np.array([[7, 8, 9], [1, 2, 3]])
    forced = _run(*args, teacher=teach)
    assert np.array_equal(forced["tokens"][:, 0], free["tokens"][:, 0])  # step 0 only sees the anchor
    alt = _run(base[:, 1:2], w1, w2, teach[:, 0], [11, 21], [5, 6], [1.0, 1.0])
    assert np.array_equal(forced["cache"][:, 1], alt["cache"][:, 0])
    assert np.array_equal(forced["tokens"][:, 1], alt["tokens"][:, 0])
