"""HIP path vs the CPU oracle on the same seeded inputs: draft tokens (under
teacher forcing), the draft-logits cache, the draft log-sum-exp, and the
verification outputs, with the margin rules of tests/parity.py."""
import numpy as np
import pytest

import workloads
from parity import Report, compare_draft, compare_verify, full_parity, run_gpu, cache_to_numpy, dev_tensors

pytestmark = pytest.mark.gpu


def _assert(rep: Report, label: str):
    print(f"PARITY {label}: tokens {rep.tokens_total} (excused {rep.tokens_excused}, bad {rep.tokens_bad}); "
          f"cache max err {rep.cache_max_err:.2e} (excused {rep.cache_excused}, bad {rep.cache_bad}); "
          f"lse max err {rep.lse_max_err:.2e} bad {rep.lse_bad}; requests {rep.req_total} "
          f"(excused {rep.req_excused}, bad {rep.req_bad})", flush=True)
    assert rep.ok(), rep.notes[:5]


def test_tiny_workload():
    wl = workloads.make_workload("tiny_v4096")
    _assert(full_parity(wl), "tiny")


def test_tiny_config_matches_golden():
    import json, os
    wl = workloads.make_workload("tiny_v4096")
    d = run_gpu(wl)
    want = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_v4096_oracle.json")))
    assert d["draft_tokens"].cpu().tolist() == want["draft_tokens"]
    assert d["out_tokens"].cpu().tolist() == want["out_tokens"]


def test_boosted_workload():
    wl = workloads.make_workload("boosted_v32000")
    _assert(full_parity(wl), "V=32000 r=128 K=5 B=8")


@pytest.mark.parametrize("B", workloads.ODD_VOCAB_BATCHES)
def test_odd_vocab_workload(B):
    wl = workloads.make_workload("odd_vocab_v50017", B=B)
    _assert(full_parity(wl), f"edge V=50017 B={B}")


def test_edge_config_planted_ties_and_nan_are_exact():
    # exact ties and NaN columns are decided by the rule alone (no margin):
    # the first NaN column wins its step; in greedy requests with planted ties
    # the first tie column wins every other step and every target row
    wl = workloads.make_workload("odd_vocab_v50017", B=16)
    d = run_gpu(wl)
    toks = d["draft_tokens"].cpu().numpy()
    out = d["out_tokens"].cpu().numpy()
    nacc = d["num_accepted"].cpu().numpy()
    nan_steps = {(b, k): cols for b, k, cols in wl.nan_rows}
    for (b, k), cols in nan_steps.items():
        assert toks[b, k] == cols[0], (b, k, toks[b, k], cols)
    first_tie = min(wl.tie_cols)
    assert wl.tie_requests
    for b in wl.tie_requests:
        for k in range(wl.K):
            if (b, k) not in nan_steps:
                assert toks[b, k] == first_tie, (b, k, toks[b, k])
        n = nacc[b]
        assert np.all(out[b, : n + 1] == first_tie) and np.all(out[b, n + 1:] == -1)


@pytest.mark.parametrize("V,r,K,B,bd,cd", [
    (1000, 64, 2, 3, "f32", "f32"),      # V below one slab of tiles
    (4099, 32, 3, 17, "f32", "f32"),     # ragged last tile, two batch tiles, r = 32 (runtime rank path)
    (8207, 96, 2, 5, "bf16", "bf16"),    # ragged, runtime rank, bf16 in and out
    (16384, 128, 4, 32, "bf16", "f32"),
    (20011, 256, 3, 2, "f32", "bf16"),
    (12345, 512, 2, 3, "f32", "f32"),    # largest rank
    (4099, 64, 7, 600, "f32", "f32"),    # K*B = 4200 > 4096: winner keys outside the zero-kept region
    (3001, 320, 5, 830, "f32", "bf16"),  # the same with the rank > 256 step kernel
])
def test_custom_shapes(V, r, K, B, bd, cd):
    wl = workloads.make_custom(V, r, K, B, base_dtype=bd, cache_dtype=cd, w_std=0.05)
    _assert(full_parity(wl), f"custom V={V} r={r} K={K} B={B} {bd}->{cd}")


def test_padded_rows_take_vector_path_on_odd_vocab():
    wl = workloads.make_workload("odd_vocab_v50017", B=8)
    _assert(full_parity(wl, pad_to=64), "edge V=50017 rows padded to 64")


def test_verify_recomputes_draft_lse_when_not_given():
    wl = workloads.make_workload("boosted_v32000")
    _assert(full_parity(wl, with_lse=False), "V=32000 without draft lse")


def test_greedy_requests_do_not_read_the_cache():
    import markov_draft_sampling_amd as mds
    import torch
    wl = workloads.make_custom(3000, 64, 3, 6, temperature=0.0)
    d = run_gpu(wl, verify=False)
    d["cache"].fill_(float("nan"))  # poison: greedy verification must not read it
    mds.rejection_verify(d["target"], d["cache"], d["draft_tokens"], d["temperature"], d["seeds"], d["anchor_pos"],
                         d["out_tokens"], d["num_accepted"], draft_lse=d["draft_lse"])
    torch.cuda.synchronize()
    rep = Report()
    compare_verify(wl, np.arange(wl.B), d["draft_tokens"].cpu().numpy(), cache_to_numpy(d["cache"], "f32"),
                   d["out_tokens"].cpu().numpy(), d["num_accepted"].cpu().numpy(), rep)
    _assert(rep, "greedy with poisoned cache")


def test_bad_anchor_sets_sticky_status():
    import markov_draft_sampling_amd as mds
    import torch
    wl = workloads.make_custom(2000, 64, 2, 3)
    d = dev_tensors(wl)
    d["anchor_tokens"][1] = 5000  # out of range
    ws = mds.new_workspace(mds.draft_workspace_bytes(3, 2, 2000, 64))
    mds.markov_draft_loop(d["base"], d["w1"], d["w2"], d["anchor_tokens"], d["anchor_pos"], d["temperature"],
                          d["seeds"], d["cache"], d["draft_tokens"], d["draft_lse"], workspace=ws)
    torch.cuda.synchronize()
    assert mds.workspace_status(ws) & mds.STATUS_BAD_ANCHOR
    wl.anchor_tokens[1] = 0  # the kernel substituted token 0
    rep = Report()
    compare_draft(wl, np.arange(3), d["draft_tokens"].cpu().numpy(), cache_to_numpy(d["cache"], "f32"),
                  d["draft_lse"].cpu().numpy(), rep)
    _assert(rep, "bad anchor")


def test_non_default_stream_and_graph_replay():
    import markov_draft_sampling_amd as mds
    import torch
    wl = workloads.make_workload("boosted_v32000", B=4)
    d = dev_tensors(wl)
    ws_d = mds.new_workspace(mds.draft_workspace_bytes(4, wl.K, wl.V, wl.r))
    ws_v = mds.new_workspace(mds.verify_workspace_bytes(4, wl.K, wl.V, False, True))

    def step():
        mds.markov_draft_loop(d["base"], d["w1"], d["w2"], d["anchor_tokens"], d["anchor_pos"], d["temperature"],
                              d["seeds"], d["cache"], d["draft_tokens"], d["draft_lse"], workspace=ws_d)
        mds.rejection_verify(d["target"], d["cache"], d["draft_tokens"], d["temperature"], d["seeds"],
                             d["anchor_pos"], d["out_tokens"], d["num_accepted"], draft_lse=d["draft_lse"],
                             workspace=ws_v)

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    s.synchronize()
    eager = (d["draft_tokens"].clone(), d["out_tokens"].clone(), d["cache"].clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for _ in range(3):
        d["draft_tokens"].fill_(-1)
        d["out_tokens"].fill_(-1)
        d["cache"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d["draft_tokens"], eager[0])
        assert torch.equal(d["out_tokens"], eager[1])
        assert torch.equal(d["cache"], eager[2])
