"""Parity at the full workload sizes, in the launch configuration bench.py
times (V=200064, r=256, K=7 at B=1/32/128; the bf16 top-p workload at
V=151936, B=32). The oracle checks sampled requests one by one under
teacher forcing; every request's verification is checked on the GPU's own
drafts and cache."""
import numpy as np
import pytest

import workloads
from parity import Report, compare_draft, compare_verify, run_gpu, cache_to_numpy

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["auto", "stream"])
def draft_path(request, monkeypatch):
    monkeypatch.setenv("MDS_DRAFT_PATH", request.param)
    return request.param


def _check(wl, rows, label):
    d = run_gpu(wl)
    toks = d["draft_tokens"].cpu().numpy()
    out = d["out_tokens"].cpu().numpy()
    nacc = d["num_accepted"].cpu().numpy()
    lse = d["draft_lse"].cpu().numpy()
    cache = cache_to_numpy(d["cache"], wl.cache_dtype)
    rep = Report()
    compare_draft(wl, rows, toks, cache, lse, rep)
    compare_verify(wl, rows, toks, cache, out, nacc, rep)
    # properties that hold for every request
    assert np.all((toks >= 0) & (toks < wl.V))
    for b in range(wl.B):
        n = nacc[b]
        assert 0 <= n <= wl.K
        assert np.array_equal(out[b, :n], toks[b, :n])
        assert 0 <= out[b, n] < wl.V and np.all(out[b, n + 1:] == -1)
    print(f"{label}: tokens excused {rep.tokens_excused}/{rep.tokens_total} bad {rep.tokens_bad}; cache max err "
          f"{rep.cache_max_err:.2e} excused {rep.cache_excused} bad {rep.cache_bad}; lse max err {rep.lse_max_err:.1e};"
          f" requests excused {rep.req_excused}/{rep.req_total} bad {rep.req_bad}", flush=True)
    assert rep.ok(), rep.notes[:5]


@pytest.mark.parametrize("B,rows", [(32, [0, 7, 19, 31]), (1, [0]), (128, [0, 64, 127])])
def test_headline_workload(draft_path, B, rows):
    wl = workloads.make_workload("headline_v200064", B=B)
    _check(wl, rows, f"V=200064 B={B} {draft_path}")


def test_bf16_top_p_workload(draft_path):
    wl = workloads.make_workload("zipf_top_p_v151936")
    _check(wl, [0, 13, 31], f"bf16 top-p V=151936 B=32 {draft_path}")


def test_resident_kernel_engages_on_the_headline_workload(monkeypatch):
    import torch
    import markov_draft_sampling_amd as mds
    from parity import dev_tensors
    monkeypatch.setenv("MDS_DRAFT_PATH", "auto")
    wl = workloads.make_workload("headline_v200064", B=8)
    d = dev_tensors(wl)
    ws = mds.new_workspace(mds.draft_workspace_bytes(wl.B, wl.K, wl.V, wl.r))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = mds.markov_draft_loop_timed(d["base"], d["w1"], d["w2"], d["anchor_tokens"], d["anchor_pos"],
                                    d["temperature"], d["seeds"], d["cache"], d["draft_tokens"], d["draft_lse"], ws,
                                    e0, e1)
    torch.cuda.synchronize()
    assert n == 1
    assert mds.workspace_status(ws) == 0
