"""The seeded input generators: reproducible, prefix-consistent, and carrying
the planted features the edge workload is meant to exercise."""
import numpy as np
import pytest

from workloads import make_workload, make_custom, WORKLOADS, bf16_bits_to_f32


def test_reproducible_and_prefix_consistent():
    a = make_workload("boosted_v32000", B=3)
    b = make_workload("boosted_v32000", B=8)
    for f in ("base", "anchor_tokens", "anchor_pos", "seeds", "temperature"):
        assert np.array_equal(getattr(a, f), getattr(b, f)[:3]), f
    assert np.array_equal(a.target, b.target[: 3 * (a.K + 1)])
    c = make_workload("boosted_v32000", B=3)
    assert np.array_equal(a.base, c.base) and np.array_equal(a.w2, c.w2)


@pytest.mark.parametrize("wname", ["tiny_v4096", "boosted_v32000"])
def test_shapes_and_distributions(wname):
    wl = make_workload(wname)
    spec = WORKLOADS[wname]
    assert wl.base.shape == (wl.B, wl.K + 1, wl.V)
    assert wl.target.shape == (wl.B * (wl.K + 1), wl.V)
    assert wl.w1.shape == wl.w2.shape == (wl.V, wl.r)
    w = bf16_bits_to_f32(wl.w2)
    assert abs(w.std() - spec.w_std) < 0.05 * spec.w_std
    resid = wl.target.reshape(wl.B, wl.K + 1, wl.V) - wl.base
    assert abs(resid.std() - spec.target_std) < 0.05 * spec.target_std
    assert np.all((wl.anchor_tokens >= 0) & (wl.anchor_tokens < wl.V))


def test_boosted_workload_boost_and_temperatures():
    wl = make_workload("boosted_v32000")
    assert np.all((wl.temperature >= 0.6) & (wl.temperature <= 1.2))
    # 5% of the columns of each request sit ~6 above the rest, in all K+1 rows
    m = wl.base[0].mean(0)  # boosted columns average ~6 over the request's K+1 rows
    assert 0.04 < (m > 3).mean() < 0.07


def test_odd_vocab_workload_planted_features():
    wl = make_workload("odd_vocab_v50017", B=16)
    assert wl.V == 50017 and wl.r == 192
    assert (wl.temperature == 0).sum() == 4
    assert 3 in wl.tie_requests
    assert any(b == 6 for b, _, _ in wl.nan_rows)
    w2 = bf16_bits_to_f32(wl.w2)
    for c in wl.tie_cols:
        assert np.all(w2[c] == 0)
    blocks = {c // 1024 for c in wl.tie_cols}
    assert len(blocks) == 4  # four distinct blocks, one of them holding a pair
    b = wl.tie_requests[0]
    for j in range(wl.K + 1):
        row = wl.base[b, j]
        vals = row[list(wl.tie_cols)]
        assert np.all(vals == vals[0]) and vals[0] == np.nanmax(row)
    for b, k, cols in wl.nan_rows:
        assert np.all(np.isnan(wl.base[b, k, list(cols)]))
        assert not np.isnan(wl.target).any()


def test_custom_bf16_base():
    wl = make_custom(100, 32, 2, 3, base_dtype="bf16", cache_dtype="bf16")
    assert wl.base.dtype == np.uint16
    t = wl.target.reshape(3, 3, 100) - bf16_bits_to_f32(wl.base)
    assert abs(t.std() - 0.5) < 0.1
