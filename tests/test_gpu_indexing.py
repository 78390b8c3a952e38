"""GPU parity of request-state indexing, padding rows and -1 placeholder drafts.

The indexed draft loop and verification (mds_markov_draft_loop_ex,
mds_rejection_verify_indexed) against the oracle's indexed runs, and the plain
verification with placeholder drafts; same parity rules as tests/parity.py.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from parity import ACC_MARGIN, CACHE_TOL, TOK_MARGIN, cache_to_numpy, dev_tensors, run_gpu

pytestmark = pytest.mark.gpu

SENT_F32 = 123.25
SENT_BF16 = 0x42F6  # 123.0


def _setup(V=8200, r=64, K=4, B=12, cache_dtype="f32", top_p=None, seed=5):
    wl = workloads.make_custom(V, r, K, B, seed=seed, cache_dtype=cache_dtype)
    rng = np.random.default_rng([seed, 99])
    n_slots, n_rows = 20, 16
    perm = rng.permutation(n_slots)[:B].astype(np.int32)  # request b -> slot
    perm[[i for i in (3, 10) if i < B]] = -1  # padding requests
    rowmap = rng.permutation(n_rows).astype(np.int32)
    rowmap = np.concatenate([rowmap, rowmap[:n_slots - n_rows]]).astype(np.int32)
    # slots of live requests map to distinct rows
    live = perm[perm >= 0]
    rowmap[live] = rng.permutation(n_rows)[: live.size]
    temp = rng.uniform(0.5, 1.5, n_slots).astype(np.float32)
    temp[perm[1]] = 0.0  # greedy
    temp[perm[2]] = 0.6
    seeds = rng.integers(0, 2**63, n_slots, dtype=np.int64)
    tp = None
    if top_p is not None:
        tp = np.ones(n_slots, np.float32)
        tp[perm[[0, 4, 6]]] = top_p
    idx = np.repeat(perm[:, None], K, axis=1).astype(np.int32)
    idx[5, 2] = -1  # an inert step: the next step of request 5 has no previous token
    spos = (wl.anchor_pos[:, None] + 1 + np.arange(K)[None, :] + rng.integers(0, 1000, B)[:, None]).astype(np.int64)
    return wl, dict(n_slots=n_slots, n_rows=n_rows, perm=perm, rowmap=rowmap, temp=temp, seeds=seeds, top_p=tp,
                    idx=idx, spos=spos)


def _run_draft(wl, ix):
    import torch
    import markov_draft_sampling_amd as mds
    d = dev_tensors(wl)
    cdt = torch.bfloat16 if wl.cache_dtype == "bf16" else torch.float32
    if wl.cache_dtype == "bf16":
        cache = torch.full((ix["n_rows"], wl.K, wl.V), SENT_BF16, dtype=torch.int16, device="cuda").view(cdt)
    else:
        cache = torch.full((ix["n_rows"], wl.K, wl.V), SENT_F32, dtype=cdt, device="cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    ws = mds.new_workspace(mds.draft_workspace_bytes(wl.B, wl.K, wl.V, wl.r), torch.device("cuda"))
    mds.markov_draft_loop_ex(d["base"], d["w1"], d["w2"], d["anchor_tokens"], t(ix["idx"]), t(ix["spos"]),
                                  t(ix["temp"]), t(ix["seeds"]), cache, d["draft_tokens"], row_mapping=t(ix["rowmap"]),
                                  draft_lse=d["draft_lse"], workspace=ws)
    torch.cuda.synchronize()
    return d, cache, mds.workspace_status(ws)


def _oracle_draft(wl, ix, teacher):
    init = np.full((ix["n_rows"], wl.K, wl.V), SENT_BF16 if wl.cache_dtype == "bf16" else SENT_F32,
                   np.uint16 if wl.cache_dtype == "bf16" else np.float32)
    return oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos,
                             ix["seeds"], ix["temp"], wl.cache_dtype, teacher=teacher, idx_map=ix["idx"],
                             row_mapping=ix["rowmap"], sample_pos=ix["spos"], cache_init=init)


@pytest.mark.parametrize("cache_dtype", ["f32", "bf16"])
def test_indexed_draft_matches_oracle(cache_dtype):
    wl, ix = _setup(cache_dtype=cache_dtype)
    d, cache, status = _run_draft(wl, ix)
    toks = d["draft_tokens"].cpu().numpy()
    lse = d["draft_lse"].cpu().numpy()
    gc = cache_to_numpy(cache, wl.cache_dtype)
    ref = _oracle_draft(wl, ix, toks)
    # tokens: exact, excused only at a top-two score gap <= 1e-3
    mism = ref["tokens"] != toks
    assert not (mism & (ref["margin"] > TOK_MARGIN)).any(), (toks, ref["tokens"])
    assert (toks[[3, 10]] == -1).all() and toks[5, 2] == -1
    # the step after the inert one had no previous token: flagged, token 0 used
    assert ref["bad_prev"] and (status & 1)
    # cache: written rows within tolerance, rows no live request maps to untouched
    if wl.cache_dtype == "bf16":
        g = workloads.bf16_bits_to_f32(gc).astype(np.float64)
        o = workloads.bf16_bits_to_f32(ref["cache"]).astype(np.float64)
        tol = np.maximum(CACHE_TOL, np.abs(o) * 2.0 ** -7 * 1.01)
    else:
        g, o = gc.astype(np.float64), ref["cache"].astype(np.float64)
        tol = CACHE_TOL
    assert (np.abs(g - o) <= tol).all()
    untouched = np.setdiff1d(np.arange(ix["n_rows"]), ix["rowmap"][ix["perm"][ix["perm"] >= 0]])
    sent = SENT_BF16 if wl.cache_dtype == "bf16" else SENT_F32
    assert (gc[untouched] == sent).all()
    # the inert step of request 5 left its cache column alone
    assert (gc[ix["rowmap"][ix["perm"][5]], 2] == sent).all()
    # lse: sampled live rows close, inert rows NaN
    live = ref["tokens"] >= 0
    samp = live & (ix["temp"][np.maximum(ix["idx"], 0)] > 0)
    err = np.abs(lse[samp] - ref["lse"][samp])
    assert (err <= 1e-4 + 1e-5 * np.abs(ref["lse"][samp])).all()
    assert np.isnan(lse[~live]).all()


@pytest.mark.parametrize("top_p", [None, 0.9])
def test_indexed_verify_matches_oracle(top_p):
    import torch
    import markov_draft_sampling_amd as mds
    wl, ix = _setup(top_p=top_p)
    d, cache, _ = _run_draft(wl, ix)
    toks = d["draft_tokens"].cpu().numpy()
    gc = cache_to_numpy(cache, wl.cache_dtype)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    out = torch.full((wl.B, wl.K + 1), -9, dtype=torch.int32, device="cuda")
    nacc = torch.full((wl.B,), -9, dtype=torch.int32, device="cuda")
    mds.rejection_verify_indexed(d["target"], cache, d["draft_tokens"], t(ix["perm"]), t(ix["temp"]), t(ix["seeds"]),
                                 d["anchor_pos"], out, nacc, row_mapping=t(ix["rowmap"]),
                                 top_p=None if top_p is None else t(ix["top_p"]))
    torch.cuda.synchronize()
    ref = oracle.verify(wl.target, gc, wl.cache_dtype, toks, ix["temp"], ix["top_p"], ix["seeds"], wl.anchor_pos,
                        idx_map=ix["perm"], row_mapping=ix["rowmap"])
    go, gn = out.cpu().numpy(), nacc.cpu().numpy()
    same = (gn == ref["num_accepted"]) & (go == ref["out_tokens"]).all(axis=1)
    exc = (ref["accept_margin"] <= ACC_MARGIN) | (ref["sample_margin"] <= TOK_MARGIN) | ref["near_top_p"]
    assert (same | exc).all(), (go, ref["out_tokens"], gn, ref["num_accepted"])
    assert (go[[3, 10]] == -1).all() and (gn[[3, 10]] == 0).all()
    # request 5's drafts end at its inert step (a -1 placeholder at step 2)
    assert gn[5] <= 2 and (go[5, gn[5] + 1:] == -1).all()


@pytest.mark.parametrize("wname", ["boosted_v32000", "odd_vocab_v50017"])
def test_plain_verify_with_placeholder_drafts(wname):
    import torch
    import markov_draft_sampling_amd as mds
    wl = workloads.make_workload(wname, B=8)
    d = run_gpu(wl, verify=False)
    toks = d["draft_tokens"].cpu().numpy()
    cut = np.array([wl.K, 0, 1, 2, wl.K - 1, 3, 0, 2])[: wl.B]
    for b, m in enumerate(cut):
        toks[b, m:] = -1
    dt = torch.from_numpy(toks).cuda()
    mds.rejection_verify(d["target"], d["cache"], dt, d["temperature"], d["seeds"], d["anchor_pos"],
                         d["out_tokens"], d["num_accepted"], draft_lse=d["draft_lse"])
    torch.cuda.synchronize()
    gc = cache_to_numpy(d["cache"], wl.cache_dtype)
    ref = oracle.verify(wl.target, gc, wl.cache_dtype, toks, wl.temperature, wl.top_p, wl.seeds, wl.anchor_pos)
    go, gn = d["out_tokens"].cpu().numpy(), d["num_accepted"].cpu().numpy()
    same = (gn == ref["num_accepted"]) & (go == ref["out_tokens"]).all(axis=1)
    exc = (ref["accept_margin"] <= ACC_MARGIN) | (ref["sample_margin"] <= TOK_MARGIN) | ref["near_top_p"]
    assert (same | exc).all(), (go, ref["out_tokens"])
    assert (gn <= cut).all()


def test_out_of_range_slot_is_inert_and_flagged():
    import torch
    import markov_draft_sampling_amd as mds
    wl, ix = _setup(B=6)
    ix["idx"][4, :] = ix["n_slots"] + 3  # slot past the state arrays
    d, cache, status = _run_draft(wl, ix)
    assert status & mds.STATUS_BAD_INDEX
    toks = d["draft_tokens"].cpu().numpy()
    assert (toks[4] == -1).all()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    perm = ix["perm"].copy()
    perm[2] = ix["n_slots"] + 1
    out = torch.full((wl.B, wl.K + 1), -9, dtype=torch.int32, device="cuda")
    nacc = torch.full((wl.B,), -9, dtype=torch.int32, device="cuda")
    ws = mds.new_workspace(mds.verify_workspace_bytes(wl.B, wl.K, wl.V, False, False), torch.device("cuda"))
    mds.rejection_verify_indexed(d["target"], cache, d["draft_tokens"], t(perm), t(ix["temp"]), t(ix["seeds"]),
                                 d["anchor_pos"], out, nacc, row_mapping=t(ix["rowmap"]), workspace=ws)
    torch.cuda.synchronize()
    assert mds.workspace_status(ws) & mds.STATUS_BAD_INDEX
    assert (out.cpu().numpy()[2] == -1).all() and int(nacc[2]) == 0
