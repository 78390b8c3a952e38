"""Pins of the winner rule, bf16 rounding and the margin helper."""
import numpy as np
import pytest
import torch

from oracle import argmax_rule, bf16_rne, bf16_to_f64, top_two_margin

nan, inf = float("nan"), float("inf")


@pytest.mark.parametrize("row,want", [
    ([1.0, nan, 5.0, nan], 1),  # first NaN wins over any value
    ([1.0, 5.0, 2.0, 5.0], 1),  # first maximum on ties
    ([-inf, -inf, -inf], 0),  # all -inf
    ([-0.0, 0.0, -1.0], 0),  # signed zeros compare equal
    ([0.0, -0.0], 0),
    ([3.0, inf, 1e38, inf], 1),  # +inf beats finite values
    ([inf, 2.0, nan], 2),  # NaN beats +inf
])
def test_argmax_rule_cases(row, want):
    assert argmax_rule(np.array(row, np.float32)) == want
    assert argmax_rule(np.array(row, np.float64)) == want


def _blockwise_winner(x, block):
    """The pages' rule between blocks: per-block winner, then the first NaN
    block, otherwise the first block holding the maximum."""
    best_v, best_i = None, None
    for s in range(0, x.size, block):
        blk = x[s:s + block]
        nan_pos = np.nonzero(np.isnan(blk))[0]
        if nan_pos.size:
            i, v = s + int(nan_pos[0]), np.nan
        else:
            m = blk.max()
            i, v = s + int(np.nonzero(blk == m)[0][0]), m
        if best_i is None:
            best_v, best_i = v, i
        elif np.isnan(best_v):
            continue
        elif np.isnan(v) or v > best_v:
            best_v, best_i = v, i
    return best_i


@pytest.mark.parametrize("block", [7, 64, 1024])
def test_blockwise_composition_equals_flat_rule(block):
    rng = np.random.default_rng(block)
    for trial in range(200):
        V = int(rng.integers(1, 5000))
        x = rng.standard_normal(V).astype(np.float32)
        kind = trial % 5
        if kind == 1:  # ties across blocks at the maximum
            cols = rng.choice(V, size=min(V, 3), replace=False)
            x[cols] = x.max() + 1
        elif kind == 2:  # NaN somewhere
            x[rng.choice(V, size=min(V, 2), replace=False)] = np.nan
        elif kind == 3:  # +inf ties and -inf
            x[rng.choice(V, size=min(V, 2), replace=False)] = np.inf
            x[rng.choice(V, size=min(V, 5), replace=False)] = -np.inf
        elif kind == 4:  # quantised values: many ties
            x = np.round(x * 2) / 2
        assert argmax_rule(x) == _blockwise_winner(x, block)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 10,
        rng.standard_normal(1000).astype(np.float32) * 1e-39,  # subnormals
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.3895314e38, -3.4028235e38, 1.1754944e-38], np.float32),
    ])
    # exact midpoints between bf16 neighbours, both even and odd lower halves
    mids = (np.arange(1, 4000, dtype=np.uint32) << np.uint32(15)) | np.uint32(0x3F800000)
    x = np.concatenate([x, mids.view(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16_rne(x)
    assert np.array_equal(got, want)
    nanbits = bf16_rne(np.array([np.nan, -np.nan], np.float32))
    assert np.all(np.isnan(bf16_to_f64(nanbits)))


def test_bf16_widening_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (f == ref) | (np.isnan(f) & np.isnan(ref))
    assert same.all()


def test_top_two_margin():
    assert top_two_margin([1.0, 3.0, 2.5]) == pytest.approx(0.5)
    assert top_two_margin([1.0, 3.0, 3.0]) == 0.0
    assert top_two_margin([1.0, nan, 3.0]) == inf
    assert top_two_margin([2.0]) == inf
