"""Back-to-back draft calls of different shapes on one workspace (the
workspace layout depends on B and K, so one call's partials can land where
the next call keeps its winner keys): each call matches
the oracle, and repeating a call repeats its tokens exactly."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from parity import Report, cache_to_numpy, compare_draft, dev_tensors

pytestmark = pytest.mark.gpu


def _draft(wl, ws):
    import torch
    import markov_draft_sampling_amd as mds
    d = dev_tensors(wl)
    mds.markov_draft_loop(d["base"], d["w1"], d["w2"], d["anchor_tokens"], d["anchor_pos"], d["temperature"],
                          d["seeds"], d["cache"], d["draft_tokens"], d["draft_lse"], workspace=ws)
    torch.cuda.synchronize()
    assert mds.workspace_status(ws) == 0
    return d["draft_tokens"].cpu().numpy(), cache_to_numpy(d["cache"], wl.cache_dtype), d["draft_lse"].cpu().numpy()


def test_calls_on_one_workspace():
    import torch
    import markov_draft_sampling_amd as mds
    wa = workloads.make_workload("boosted_v32000", B=8)
    wb = workloads.make_custom(9001, 128, 3, 3, seed=12, temperature=0.8)
    ws = mds.new_workspace(max(mds.draft_workspace_bytes(wa.B, wa.K, wa.V, wa.r),
                               mds.draft_workspace_bytes(wb.B, wb.K, wb.V, wb.r)), torch.device("cuda"))
    first = None
    for wl in (wa, wb, wa):
        toks, cache, lse = _draft(wl, ws)
        rep = Report()
        compare_draft(wl, np.arange(wl.B), toks, cache, lse, rep)
        assert rep.ok(), rep.notes[:3]
        if wl is wa:
            if first is None:
                first = toks
            else:
                np.testing.assert_array_equal(toks, first)


def test_dense_and_topk_calls_share_a_workspace():
    """A top-k drafting call between two dense calls on one workspace: the
    dense calls keep their winner keys in a region the library leaves at zero
    and the top-k call leaves untouched, so each dense call still matches the
    oracle and the top-k call matches one on a fresh workspace."""
    import torch
    import markov_draft_sampling_amd as mds
    wl = workloads.make_workload("boosted_v32000", B=8)
    topk = 16
    dev = torch.device("cuda")
    size = max(mds.draft_workspace_bytes(wl.B, wl.K, wl.V, wl.r),
               mds.draft_topk_workspace_bytes(wl.B, wl.K, wl.V, wl.r, topk))
    ws = mds.new_workspace(size, dev)

    def topk_call(workspace):
        d = dev_tensors(wl)
        spos = (d["anchor_pos"][:, None] + 1 + torch.arange(wl.K, device=dev)[None, :]).contiguous()
        mds.markov_draft_loop_topk(d["base"], d["w1"], d["w2"], d["anchor_tokens"], None, spos, d["temperature"],
                                   d["seeds"], d["cache"], d["draft_tokens"], topk, draft_lse=d["draft_lse"],
                                   workspace=workspace)
        torch.cuda.synchronize()
        assert mds.workspace_status(workspace) == 0
        return d["draft_tokens"].cpu().numpy(), cache_to_numpy(d["cache"], wl.cache_dtype)

    monkey_env = pytest.MonkeyPatch()
    monkey_env.setenv("MDS_DRAFT_PATH", "stream")
    try:
        first = _draft(wl, ws)
        t_shared, c_shared = topk_call(ws)
        again = _draft(wl, ws)
    finally:
        monkey_env.undo()
    for toks, cache, lse in (first, again):
        rep = Report()
        compare_draft(wl, np.arange(wl.B), toks, cache, lse, rep)
        assert rep.ok(), rep.notes[:3]
    np.testing.assert_array_equal(first[0], again[0])
    t_fresh, c_fresh = topk_call(mds.new_workspace(size, dev))
    np.testing.assert_array_equal(t_shared, t_fresh)
    np.testing.assert_array_equal(c_shared, c_fresh)
