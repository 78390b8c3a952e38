"""GPU parity of the fp64 Gumbel option (mds_markov_draft_loop_ex, MDS_DRAFT_FP64_GUMBEL).

Draft tokens against the oracle's float64 scores under teacher forcing
(mismatch excused only at a float64 top-two gap <= 1e-3), planted ties and NaN
columns decided exactly, cache and log-sum-exp as in the float32 mode.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from parity import CACHE_TOL, TOK_MARGIN, cache_to_numpy, dev_tensors

pytestmark = pytest.mark.gpu


def _run(wl, fp64=True):
    import torch
    import markov_draft_sampling_amd as mds
    d = dev_tensors(wl)
    spos = torch.from_numpy(wl.anchor_pos[:, None] + 1 + np.arange(wl.K)[None, :]).cuda()
    ws = mds.new_workspace(mds.draft_workspace_bytes(wl.B, wl.K, wl.V, wl.r), torch.device("cuda"))
    mds.markov_draft_loop_ex(d["base"], d["w1"], d["w2"], d["anchor_tokens"], None, spos, d["temperature"], d["seeds"],
                             d["cache"], d["draft_tokens"], draft_lse=d["draft_lse"], fp64_gumbel=fp64, workspace=ws)
    torch.cuda.synchronize()
    assert mds.workspace_status(ws) == 0
    return d


def _check(wl, d, rows):
    rows = np.asarray(rows)
    toks = d["draft_tokens"].cpu().numpy()
    ref = oracle.draft_loop(wl.draft_base[rows], wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens[rows],
                            wl.anchor_pos[rows], wl.seeds[rows], wl.temperature[rows], wl.cache_dtype,
                            teacher=toks[rows], fp64_gumbel=True)
    mism = ref["tokens"] != toks[rows]
    bad = mism & (ref["margin"] > TOK_MARGIN)
    assert not bad.any(), (np.argwhere(bad)[:5], toks[rows][bad][:5], ref["tokens"][bad][:5])
    gc = cache_to_numpy(d["cache"], wl.cache_dtype)[rows]
    if wl.cache_dtype == "bf16":
        g = workloads.bf16_bits_to_f32(gc).astype(np.float64)
        o = workloads.bf16_bits_to_f32(ref["cache"]).astype(np.float64)
        tol = np.maximum(CACHE_TOL, np.abs(o) * 2.0 ** -7 * 1.01)
    else:
        g, o = gc.astype(np.float64), ref["cache"].astype(np.float64)
        tol = CACHE_TOL
    ok = (np.abs(g - o) <= tol) | (np.isnan(g) & np.isnan(o))
    assert ok.all()
    lse = d["draft_lse"].cpu().numpy()[rows]
    samp = np.broadcast_to((wl.temperature[rows] > 0)[:, None], lse.shape)
    err = np.abs(lse - ref["lse"])[samp]
    both_nan = (np.isnan(lse) & np.isnan(ref["lse"]))[samp]
    assert ((err <= 1e-4 + 1e-5 * np.abs(ref["lse"][samp])) | both_nan).all()
    return toks, ref


@pytest.mark.parametrize("wname", ["tiny_v4096", "boosted_v32000", "odd_vocab_v50017"])
def test_fp64_gumbel_matches_oracle(wname):
    wl = workloads.make_workload(wname, B=None if wname == "tiny_v4096" else 8)
    d = _run(wl)
    toks, ref = _check(wl, d, np.arange(wl.B))
    # planted ties and NaN columns are decided by rule, exactly
    for b, k, cols in wl.nan_rows:
        if b < wl.B and k < wl.K:
            assert toks[b, k] == ref["tokens"][b, k]
    for b in wl.tie_requests:
        if b < wl.B:
            np.testing.assert_array_equal(toks[b], ref["tokens"][b])


def test_fp64_gumbel_headline_rows():
    wl = workloads.make_workload("headline_v200064", B=32)
    d = _run(wl)
    _check(wl, d, [0, 11, 31])


def test_fp64_and_fp32_runs_agree_on_clear_steps():
    wl = workloads.make_workload("boosted_v32000", B=8)
    d64 = _run(wl, fp64=True)
    t64 = d64["draft_tokens"].cpu().numpy()
    d32 = _run(wl, fp64=False)
    t32 = d32["draft_tokens"].cpu().numpy()
    ref = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, wl.seeds,
                            wl.temperature, wl.cache_dtype, teacher=t32)
    first = np.argmax(np.concatenate([t64 != t32, np.ones((wl.B, 1), bool)], axis=1), axis=1)
    for b in range(wl.B):  # until the chains part, a step differs only where float32 rounding decides
        for k in range(min(first[b] + 1, wl.K)):
            if t64[b, k] != t32[b, k]:
                assert ref["margin"][b, k] <= 1e-4


def test_fp64_gumbel_needs_rank_up_to_256():
    import torch
    import markov_draft_sampling_amd as mds
    wl = workloads.make_custom(1000, 288, 2, 2, seed=1)
    d = dev_tensors(wl)
    spos = torch.from_numpy(wl.anchor_pos[:, None] + 1 + np.arange(wl.K)[None, :]).cuda()
    with pytest.raises(mds.MdsError):
        mds.markov_draft_loop_ex(d["base"], d["w1"], d["w2"], d["anchor_tokens"], None, spos, d["temperature"],
                                 d["seeds"], d["cache"], d["draft_tokens"], fp64_gumbel=True)


@pytest.mark.parametrize("T", [1.0, 0.7])
@pytest.mark.parametrize("V", [50016, 50017])
def test_fp64_near_ties_decided_exactly(V, T):
    # Planted columns whose float64 scores z / T + g all lie within 2e-7 of 1
    # (zero w2 rows: z is the base logit; the base holds fp32((s - g) T) for
    # a random target s with the oracle's own float64 noise g): apart for the
    # float64 keys (2^-28 relative; the top two at least 1e-8), in no reliable
    # order for float32 scores, whose rounding is of the same size. Per row
    # sixteen of them sit in one lane (columns c0 .. c0 + 3 of one tile and of
    # the wave's next three tiles, c0 + 64 j ..), four more in other lanes and
    # waves. The draft tokens must equal the oracle's exact float64 winners,
    # with no excuse. V = 50016: aligned rows, the fast loop with its float32
    # filter; V = 50017: unaligned rows, the general loop (float64 throughout).
    print(f"fp64 near ties: V={V} T={T}", flush=True)
    wl = workloads.make_custom(V, 64, 3, 4, seed=21, temperature=T)
    B, K, V = wl.B, wl.K, wl.V
    rng = np.random.default_rng(5)
    wl.base[:] = -50.0
    planted = {}
    lane_misses = 0
    T32 = np.float32(T)
    for b in range(B):
        for k in range(K):
            c0 = 2048 + 1664 * (b * K + k)  # a multiple of 64: lane-aligned
            cols = np.concatenate([(c0 + 64 * np.arange(4)[:, None] + np.arange(4)).ravel(),
                                   c0 + np.array([4, 9, 16, 77])])
            g = oracle.gumbel(oracle.uniform24(oracle.noise_words(int(wl.seeds[b]), int(wl.anchor_pos[b]) + k,
                                                                  oracle.SALT_DRAFT, cols)))
            for _ in range(1000):  # redraw until the float64 top two are clearly apart for the 2^-28 keys
                z = ((1.0 + rng.random(len(cols)) * 2e-7 - g) * T).astype(np.float32)
                s64 = z.astype(np.float64) / np.float64(T32) + g
                top = np.sort(s64)
                if top[-1] - top[-2] >= 1e-8:
                    break
            else:
                raise AssertionError("no planted row with a clear float64 winner")
            wl.base[b, k, cols] = z
            planted[(b, k)] = cols
            # the construction's power: float32 scores (numpy's rounding) that
            # leave the float64 winner out of its lane's top two
            s32 = z / T32 + g.astype(np.float32)
            win = int(np.argmax(s64))
            lane_misses += win < 16 and win not in np.argsort(-s32[:16], kind="stable")[:2]
    assert lane_misses >= 2
    allc = np.unique(np.concatenate(list(planted.values())))
    wl.w2[allc] = 0  # bias 0 at the planted columns, whatever the previous token
    d64 = _run(wl)
    toks = d64["draft_tokens"].cpu().numpy()
    ref = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, wl.seeds,
                            wl.temperature, wl.cache_dtype, teacher=toks, fp64_gumbel=True)
    np.testing.assert_array_equal(toks, ref["tokens"])
    for (b, k), cols in planted.items():
        assert toks[b, k] in cols
    # every row is a near-tie at float32 resolution (the general parity rule
    # would excuse any of them), yet each was decided exactly
    assert (ref["margin"] < 1e-5).all(), ref["margin"]


def test_fp64_float32_overflow_decided_exactly():
    # T = 1e-37: planted logits 100 .. 107.5 give float32 scores past the
    # float32 range (+inf, all equal) and float64 scores ~1e39 that are far
    # apart; the rest of the row scores -10. Sixteen planted columns per row
    # sit in one lane, the largest logit last, so a filter that ranked the
    # float32 scores would keep only the first two. V = 50016: the fast loop.
    print("fp64 float32 overflow: V=50016 T=1e-37", flush=True)
    wl = workloads.make_custom(50016, 64, 2, 4, seed=29, temperature=1e-37)
    B, K = wl.B, wl.K
    wl.base[:] = -1e-36
    wl.w2[:] = 0  # no Markov bias: z is the base logit
    planted = {}
    for b in range(B):
        for k in range(K):
            c0 = 2048 + 1664 * (b * K + k)
            cols = (c0 + 64 * np.arange(4)[:, None] + np.arange(4)).ravel()
            wl.base[b, k, cols] = (100.0 + 0.5 * np.arange(16)).astype(np.float32)
            planted[(b, k)] = cols
    d = _run(wl)
    toks = d["draft_tokens"].cpu().numpy()
    with np.errstate(all="ignore"):
        ref = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos,
                                wl.seeds, wl.temperature, wl.cache_dtype, teacher=toks, fp64_gumbel=True)
    np.testing.assert_array_equal(toks, ref["tokens"])
    for (b, k), cols in planted.items():
        assert toks[b, k] == cols[-1]
