"""The allocation-free draft entry point (mds_markov_draft_loop_noalloc, whose
scratch is a fixed array inside the library) against mds_markov_draft_loop
with a caller workspace: identical tokens, cache and draft log-sum-exp on two
calls in a row, the second one smaller, then a third call back at the first
size; its size limit and its caller-owned status word."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from parity import dev_tensors

pytestmark = pytest.mark.gpu


def _plain(wl):
    import torch
    import markov_draft_sampling_amd as mds
    d = dev_tensors(wl)
    mds.markov_draft_loop(d["base"], d["w1"], d["w2"], d["anchor_tokens"], d["anchor_pos"], d["temperature"],
                          d["seeds"], d["cache"], d["draft_tokens"], d["draft_lse"])
    torch.cuda.synchronize()
    return d


def _noalloc(wl):
    import torch
    import markov_draft_sampling_amd as mds
    d = dev_tensors(wl)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    mds.markov_draft_loop_noalloc(d["base"], d["w1"], d["w2"], d["anchor_tokens"], d["anchor_pos"],
                                  d["temperature"], d["seeds"], d["cache"], d["draft_tokens"], d["draft_lse"], status)
    torch.cuda.synchronize()
    return d, int(status.item())


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def _same(a, b, label):
    # bit patterns: the planted NaN columns must match too
    import torch
    assert torch.equal(a["draft_tokens"], b["draft_tokens"]), label
    assert torch.equal(_bits(a["cache"]), _bits(b["cache"])), label
    assert torch.equal(_bits(a["draft_lse"]), _bits(b["draft_lse"])), label


def test_noalloc_matches_the_workspace_call_on_consecutive_calls():
    big = workloads.make_workload("boosted_v32000")             # B=8, K=5, V=32000, r=128
    small = workloads.make_custom(4099, 64, 3, 2, seed=21, temperature=0.8)
    for wl, label in ((big, "first call"), (small, "second, smaller call"), (big, "third call")):
        want = _plain(wl)
        got, status = _noalloc(wl)
        assert status == 0, label
        _same(want, got, label)
        print(f"noalloc {label}: {wl.name} tokens {got['draft_tokens'].cpu().numpy().tolist()[:2]}", flush=True)


def test_noalloc_large_batch_and_odd_vocab():
    # K*B = 896, the largest the headline batches use, on the odd vocabulary
    wl = workloads.make_workload("odd_vocab_v50017", B=128)
    want = _plain(wl)
    got, status = _noalloc(wl)
    assert status == 0
    _same(want, got, "odd vocabulary B=128")


def test_noalloc_size_limit_and_status_word():
    import torch
    import markov_draft_sampling_amd as mds
    wl = workloads.make_custom(1000, 32, 8, 129, seed=3)  # K*B = 1032 > 1024: refused before any launch
    d = dev_tensors(wl)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(mds.MdsError, match="unsupported"):
        mds.markov_draft_loop_noalloc(d["base"], d["w1"], d["w2"], d["anchor_tokens"], d["anchor_pos"],
                                      d["temperature"], d["seeds"], d["cache"], d["draft_tokens"], d["draft_lse"],
                                      status)
    wl = workloads.make_custom(2000, 64, 2, 3, seed=4)
    d = dev_tensors(wl)
    d["anchor_tokens"][1] = 5000  # out of range: token 0 is used and the status bit set
    mds.markov_draft_loop_noalloc(d["base"], d["w1"], d["w2"], d["anchor_tokens"], d["anchor_pos"],
                                  d["temperature"], d["seeds"], d["cache"], d["draft_tokens"], d["draft_lse"], status)
    torch.cuda.synchronize()
    assert int(status.item()) & mds.STATUS_BAD_ANCHOR
    wl.anchor_tokens[1] = 0
    want = _plain(wl)
    _same(want, d, "bad anchor")
