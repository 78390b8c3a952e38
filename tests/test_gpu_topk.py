"""GPU parity of top-k Markov drafting (mds_markov_draft_loop_topk).

Against the oracle's top-k loop under teacher forcing, with the rules of
tests/parity.py: draft tokens exact unless the top-two score gap is <= 1e-3;
the cache element by element (the -inf columns, i.e. the candidate sets,
exactly); the log-sum-exp to 1e-4 + 1e-5 |lse|. Then verification on the
top-k cache against the oracle's verification.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from parity import Report, cache_to_numpy, compare_draft, compare_verify, dev_tensors

pytestmark = pytest.mark.gpu


def _spos(wl):
    import torch
    return torch.from_numpy(wl.anchor_pos[:, None] + 1 + np.arange(wl.K)[None, :]).cuda()


def _run(wl, topk, fp64=False, pad_to=None, verify=False):
    import torch
    import markov_draft_sampling_amd as mds
    d = dev_tensors(wl, pad_to=pad_to)
    ws = mds.new_workspace(mds.draft_topk_workspace_bytes(wl.B, wl.K, wl.V, wl.r, topk), torch.device("cuda"))
    mds.markov_draft_loop_topk(d["base"], d["w1"], d["w2"], d["anchor_tokens"], None, _spos(wl), d["temperature"],
                               d["seeds"], d["cache"], d["draft_tokens"], topk, draft_lse=d["draft_lse"],
                               fp64_gumbel=fp64, workspace=ws)
    if verify:
        mds.rejection_verify(d["target"], d["cache"], d["draft_tokens"], d["temperature"], d["seeds"],
                             d["anchor_pos"], d["out_tokens"], d["num_accepted"], draft_lse=d["draft_lse"],
                             top_p=d["top_p"])
    torch.cuda.synchronize()
    d["status"] = mds.workspace_status(ws)
    return d


def _check(wl, d, topk, rows=None, fp64=False, verify=False):
    rows = np.arange(wl.B) if rows is None else np.asarray(rows)
    toks = d["draft_tokens"].cpu().numpy()
    cache = cache_to_numpy(d["cache"], wl.cache_dtype)
    lse = d["draft_lse"].cpu().numpy()
    rep = Report()
    ref = compare_draft(wl, rows, toks, cache, lse, rep, topk=topk, fp64_gumbel=fp64)
    if verify:
        compare_verify(wl, rows, toks, cache, d["out_tokens"].cpu().numpy(), d["num_accepted"].cpu().numpy(), rep)
    assert rep.ok(), rep.notes[:5]
    # the candidate sets, exactly: finite (or NaN) entries of each cache row
    c = workloads.bf16_bits_to_f32(cache[rows]) if wl.cache_dtype == "bf16" else cache[rows]
    o = workloads.bf16_bits_to_f32(ref["cache"]) if wl.cache_dtype == "bf16" else ref["cache"]
    np.testing.assert_array_equal(c == -np.inf, o == -np.inf)
    assert d["status"] == 0
    return toks, ref


@pytest.mark.parametrize("wname,topk", [("tiny_v4096", 1), ("tiny_v4096", 7), ("tiny_v4096", 256),
                                         ("boosted_v32000", 64), ("odd_vocab_v50017", 33), ("zipf_top_p_v151936", 64)])
def test_topk_matches_oracle(wname, topk):
    wl = workloads.make_workload(wname, B=None if wname == "tiny_v4096" else 6)
    d = _run(wl, topk, verify=True)
    _check(wl, d, topk, verify=True)


@pytest.mark.parametrize("V,topk", [(8193, 5), (20001, 128), (600, 256), (70001, 117)])
def test_topk_ragged_vocabularies(V, topk):
    wl = workloads.make_custom(V, 64, 3, 4, seed=V, temperature=0.9)
    wl.temperature[2] = 0.0
    d = _run(wl, topk)
    _check(wl, d, topk)


def test_topk_strided_rows_and_bf16():
    wl = workloads.make_custom(5001, 96, 4, 5, seed=8, base_dtype="bf16", cache_dtype="bf16", temperature=1.3)
    d = _run(wl, 40, pad_to=64)
    _check(wl, d, 40)


def test_topk_ties_nan_and_inf_rows():
    wl = workloads.make_custom(9000, 32, 4, 6, seed=3, temperature=1.0)
    base = wl.base
    base[:] = np.round(base)  # many equal values: the lower column ranks first
    base[1, 0, [5, 700, 8500]] = np.nan  # NaN candidates, the first one wins
    base[2, 1, :] = -np.inf  # a row of -inf: every column ties, token 0
    base[3, 2, 4000] = np.inf
    base[4, :, :] = 0.0  # all equal: candidates are columns 0..k-1
    wl.temperature[5] = 0.0
    d = _run(wl, 16)
    toks, ref = _check(wl, d, 16)
    assert toks[1, 0] == 5 and toks[2, 1] == 0
    cache = cache_to_numpy(d["cache"], "f32")
    assert np.isfinite(cache[4, 0, :16]).all() and (cache[4, 0, 16:] == -np.inf).all()


@pytest.mark.parametrize("topk", [16, 64, 256])
def test_topk_chunk_survivor_paths(topk):
    # Per 8192-column chunk, the survivors of the thread-maximum bound: few
    # (random chunks, ~70 for k = 64), many (chunk 0 of row (0, 0): 63
    # threads whose 32 values all lie above the bound, 2017 survivors),
    # equal values over 64 threads, a chunk decreasing with the column, and
    # the ragged tail chunk.
    V = 3 * 8192 + 100
    wl = workloads.make_custom(V, 64, 2, 3, seed=topk)
    cols = np.arange(8192)
    thread = (cols % 1024) // 4
    base = wl.base
    base[0, 0, :8192] = np.where(thread < 64, 1000.0 - thread, -1000.0)
    base[1, 1, 2 * 8192:3 * 8192] = np.linspace(50.0, -50.0, 8192, dtype=np.float32)
    base[2, 0, :8192] = np.where(thread < 64, 7.0, -7.0)  # equal values: the lower column ranks first
    d = _run(wl, topk)
    _check(wl, d, topk)


def test_topk_fp64_gumbel():
    wl = workloads.make_workload("boosted_v32000", B=6)
    d = _run(wl, 50, fp64=True)
    _check(wl, d, 50, fp64=True)


def test_topk_indexed_with_padding():
    import torch
    import markov_draft_sampling_amd as mds
    wl = workloads.make_custom(12000, 64, 4, 8, seed=21)
    rng = np.random.default_rng(5)
    n_slots, n_rows = 14, 10
    perm = rng.permutation(n_slots)[: wl.B].astype(np.int32)
    perm[6] = -1
    rowmap = rng.integers(0, n_rows, n_slots).astype(np.int32)
    live = perm[perm >= 0]
    rowmap[live] = rng.permutation(n_rows)[: live.size]
    temp = rng.uniform(0.5, 1.5, n_slots).astype(np.float32)
    temp[perm[1]] = 0.0
    seeds = rng.integers(0, 2**63, n_slots, dtype=np.int64)
    idx = np.repeat(perm[:, None], wl.K, axis=1).astype(np.int32)
    idx[3, 1] = -1
    spos = (wl.anchor_pos[:, None] + 1 + np.arange(wl.K)[None, :] + 77).astype(np.int64)
    d = dev_tensors(wl)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    cache = torch.full((n_rows, wl.K, wl.V), 5.5, dtype=torch.float32, device="cuda")
    ws = mds.new_workspace(mds.draft_topk_workspace_bytes(wl.B, wl.K, wl.V, wl.r, 24), torch.device("cuda"))
    mds.markov_draft_loop_topk(d["base"], d["w1"], d["w2"], d["anchor_tokens"], t(idx), t(spos), t(temp), t(seeds),
                               cache, d["draft_tokens"], 24, row_mapping=t(rowmap), draft_lse=d["draft_lse"],
                               workspace=ws)
    torch.cuda.synchronize()
    toks = d["draft_tokens"].cpu().numpy()
    ref = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, seeds, temp,
                            "f32", teacher=toks, idx_map=idx, row_mapping=rowmap, sample_pos=spos,
                            cache_init=np.full((n_rows, wl.K, wl.V), 5.5, np.float32), topk=24)
    mism = (ref["tokens"] != toks) & (ref["margin"] > 1e-3)
    assert not mism.any()
    assert (toks[6] == -1).all() and toks[3, 1] == -1
    assert ref["bad_prev"] and (mds.workspace_status(ws) & mds.STATUS_BAD_ANCHOR)
    g = cache.cpu().numpy().astype(np.float64)
    o = ref["cache"].astype(np.float64)
    with np.errstate(invalid="ignore"):
        assert ((np.abs(g - o) <= 2e-3) | (g == o)).all()
    lse = d["draft_lse"].cpu().numpy()
    live_steps = ref["tokens"] >= 0
    samp = live_steps & (temp[np.maximum(idx, 0)] > 0)
    assert (np.abs(lse[samp] - ref["lse"][samp]) <= 1e-4 + 1e-5 * np.abs(ref["lse"][samp])).all()
    assert np.isnan(lse[~live_steps]).all()


@pytest.mark.parametrize("K", [1, 5])
def test_topk_inert_steps_anywhere(K):
    # inert steps first, last, two in a row and alternating (the chain issues
    # a step's loads before it knows the step is live, and a live step after
    # an inert one has no previous token: token 0, flagged); K = 1 as well
    import torch
    import markov_draft_sampling_amd as mds
    print(f"top-k inert steps: K={K}", flush=True)
    wl = workloads.make_custom(9000, 64, K, 6, seed=33)
    B = wl.B
    idx = np.repeat(np.arange(B, dtype=np.int32)[:, None], K, axis=1)
    if K == 1:
        idx[1, 0] = idx[4, 0] = -1
    else:
        idx[0, 0] = -1               # inert first step
        idx[1, K - 1] = -1           # inert last step
        idx[2, 1] = idx[2, 2] = -1   # two in a row
        idx[3, 1::2] = -1            # alternating
        idx[5, :] = -1               # a padding request
    temp = wl.temperature.copy()
    temp[4] = 0.0  # a greedy request
    spos = (wl.anchor_pos[:, None] + 1 + np.arange(K)[None, :]).astype(np.int64)
    d = dev_tensors(wl)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    cache = torch.full((B, K, wl.V), 2.5, dtype=torch.float32, device="cuda")
    ws = mds.new_workspace(mds.draft_topk_workspace_bytes(B, K, wl.V, wl.r, 20), torch.device("cuda"))
    mds.markov_draft_loop_topk(d["base"], d["w1"], d["w2"], d["anchor_tokens"], t(idx), t(spos), t(temp),
                               d["seeds"], cache, d["draft_tokens"], 20, draft_lse=d["draft_lse"], workspace=ws)
    torch.cuda.synchronize()
    toks = d["draft_tokens"].cpu().numpy()
    ref = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, wl.seeds,
                            temp, "f32", teacher=toks, idx_map=idx, sample_pos=spos,
                            cache_init=np.full((B, K, wl.V), 2.5, np.float32), topk=20)
    mism = (ref["tokens"] != toks) & (ref["margin"] > 1e-3)
    assert not mism.any(), np.argwhere(mism)[:5]
    assert ((toks == -1) == (idx < 0)).all()
    flagged = bool(mds.workspace_status(ws) & mds.STATUS_BAD_ANCHOR)
    assert flagged == bool(ref["bad_prev"])
    if K > 1:
        assert flagged
    g = cache.cpu().numpy().astype(np.float64)
    o = ref["cache"].astype(np.float64)
    with np.errstate(invalid="ignore"):
        assert ((np.abs(g - o) <= 2e-3) | (g == o)).all()
    lse = d["draft_lse"].cpu().numpy()
    live_steps = idx >= 0
    samp = live_steps & (temp[:, None] > 0)
    assert (np.abs(lse[samp] - ref["lse"][samp]) <= 1e-4 + 1e-5 * np.abs(ref["lse"][samp])).all()
    assert np.isnan(lse[~live_steps]).all()


def test_topk_headline_rows():
    wl = workloads.make_workload("headline_v200064", B=32)
    d = _run(wl, 64, verify=True)
    _check(wl, d, 64, rows=[0, 13, 31], verify=True)


def test_topk_argument_errors():
    import torch
    import markov_draft_sampling_amd as mds
    wl = workloads.make_custom(300, 32, 2, 2, seed=1)
    d = dev_tensors(wl)
    for k in (0, 257, 301):
        with pytest.raises(mds.MdsError):
            mds.markov_draft_loop_topk(d["base"], d["w1"], d["w2"], d["anchor_tokens"], None, _spos(wl),
                                       d["temperature"], d["seeds"], d["cache"], d["draft_tokens"], k)
    torch.cuda.synchronize()
