"""HIP graph capture of whole draft + verify steps through the C-ABI.

The library enqueues kernels only (no memsets, no allocation, no
synchronisation), so a step can be captured into a graph. Each case runs the
step eagerly on a side stream, captures it, then replays the graph three
times with eager work (output fills, synchronisations) between the replays;
every replay must reproduce the eager outputs bit for bit. Cases: the step as
the benchmark times it (indexed entry point with tiled w2, verification with
draft log-normalisers, V=200064 B=32), the bf16 top-p workload (the counting
statistics pass, the top-p pass and the decision kernel), the draft LM head
fused with the loop, and top-k drafting.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from parity import dev_tensors

pytestmark = pytest.mark.gpu


def _replay_matches(step, outs):
    import torch
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    s.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(3):
        for o in outs:
            if o.dtype in (torch.int32, torch.int64):
                o.fill_(-1)
            else:
                o.fill_(float(rep) - 7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), (rep, o.shape)


def _verify(mds, d, workspace, top_p=None):
    mds.rejection_verify(d["target"], d["cache"], d["draft_tokens"], d["temperature"], d["seeds"], d["anchor_pos"],
                         d["out_tokens"], d["num_accepted"], draft_lse=d["draft_lse"], top_p=top_p,
                         workspace=workspace)


def test_graph_replay_of_the_benchmarked_step():
    import torch
    import markov_draft_sampling_amd as mds
    print("graph: headline V=200064 B=32, tiled w2", flush=True)
    wl = workloads.make_workload("headline_v200064", B=32)
    d = dev_tensors(wl)
    B, K, V, r = wl.B, wl.K, wl.V, wl.r
    w2t = mds.tile_markov_w2(d["w2"])
    spos = (d["anchor_pos"][:, None] + 1 + torch.arange(K, device="cuda")[None, :]).contiguous()
    ws_d = mds.new_workspace(mds.draft_workspace_bytes(B, K, V, r))
    ws_v = mds.new_workspace(mds.verify_workspace_bytes(B, K, V, False, True))

    def step():
        mds.markov_draft_loop_ex(d["base"], d["w1"], w2t, d["anchor_tokens"], None, spos, d["temperature"],
                                 d["seeds"], d["cache"], d["draft_tokens"], draft_lse=d["draft_lse"],
                                 workspace=ws_d, w2_tiled=True)
        _verify(mds, d, ws_v)

    _replay_matches(step, [d["draft_tokens"], d["draft_lse"], d["cache"], d["out_tokens"], d["num_accepted"]])
    assert mds.workspace_status(ws_d) == 0 and mds.workspace_status(ws_v) == 0


def test_graph_replay_top_p_workload():
    import markov_draft_sampling_amd as mds
    print("graph: bf16 top-p V=151936 B=8", flush=True)
    wl = workloads.make_workload("zipf_top_p_v151936", B=8)
    d = dev_tensors(wl)
    B, K, V, r = wl.B, wl.K, wl.V, wl.r
    ws_d = mds.new_workspace(mds.draft_workspace_bytes(B, K, V, r))
    ws_v = mds.new_workspace(mds.verify_workspace_bytes(B, K, V, True, True))

    def step():
        mds.markov_draft_loop(d["base"], d["w1"], d["w2"], d["anchor_tokens"], d["anchor_pos"], d["temperature"],
                              d["seeds"], d["cache"], d["draft_tokens"], d["draft_lse"], workspace=ws_d)
        _verify(mds, d, ws_v, top_p=d["top_p"])

    _replay_matches(step, [d["draft_tokens"], d["draft_lse"], d["cache"], d["out_tokens"], d["num_accepted"]])


def test_graph_replay_lm_head_fused_loop():
    import torch
    import markov_draft_sampling_amd as mds
    print("graph: LM head + loop, V=33001 H=512 B=8", flush=True)
    B, K, V, H, r = 8, 4, 33001, 512, 256
    wl = workloads.make_custom(V, r, K, B, seed=3)
    hidden, lm = workloads.make_lm_head(B * K, V, H, seed=3)
    d = dev_tensors(wl)
    bits = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    h, w = bits(hidden), bits(lm)
    ws_d = mds.new_workspace(mds.draft_workspace_bytes(B, K, V, r))
    ws_v = mds.new_workspace(mds.verify_workspace_bytes(B, K, V, False, True))
    base = d["base"]

    def step():
        mds.markov_draft_loop_from_hidden(h, w, base, d["w1"], d["w2"], d["anchor_tokens"], d["anchor_pos"],
                                          d["temperature"], d["seeds"], d["cache"], d["draft_tokens"],
                                          d["draft_lse"], workspace=ws_d)
        _verify(mds, d, ws_v)

    _replay_matches(step, [d["draft_tokens"], d["draft_lse"], d["cache"], d["out_tokens"], d["num_accepted"]])


def test_graph_replay_topk_drafting():
    import torch
    import markov_draft_sampling_amd as mds
    print("graph: top-k k=16, V=20000 B=6", flush=True)
    wl = workloads.make_custom(20000, 128, 3, 6, seed=8)
    d = dev_tensors(wl)
    B, K, V, r = wl.B, wl.K, wl.V, wl.r
    spos = (d["anchor_pos"][:, None] + 1 + torch.arange(K, device="cuda")[None, :]).contiguous()
    ws_d = mds.new_workspace(mds.draft_topk_workspace_bytes(B, K, V, r, 16))
    ws_v = mds.new_workspace(mds.verify_workspace_bytes(B, K, V, False, True))

    def step():
        mds.markov_draft_loop_topk(d["base"], d["w1"], d["w2"], d["anchor_tokens"], None, spos, d["temperature"],
                                   d["seeds"], d["cache"], d["draft_tokens"], 16, draft_lse=d["draft_lse"],
                                   workspace=ws_d)
        _verify(mds, d, ws_v)

    _replay_matches(step, [d["draft_tokens"], d["draft_lse"], d["cache"], d["out_tokens"], d["num_accepted"]])
