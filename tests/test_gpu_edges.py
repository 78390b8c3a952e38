"""Edge shapes and degenerate inputs through the whole path (draft loop and
verification) against the oracle, with the margin rules of tests/parity.py:
one draft step and the largest K, vocabularies smaller than one tile, a batch
of greedy requests only, a very low temperature, and the top-k and LM-head
entry points at their smallest sizes."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from parity import Report, cache_to_numpy, compare_draft, full_parity

pytestmark = pytest.mark.gpu


def _ok(rep: Report):
    assert rep.ok(), rep.notes[:5]


@pytest.mark.parametrize("V,r,K,B", [
    (3000, 64, 1, 3),     # a single draft step
    (2000, 32, 32, 2),    # the largest K
    (2, 32, 3, 4),        # the smallest vocabulary
    (15, 64, 4, 3),       # less than one 16-column tile
    (17, 32, 2, 40),      # one full tile and one column, two batch tiles
])
def test_edge_shapes(V, r, K, B):
    wl = workloads.make_custom(V, r, K, B, seed=V + K, temperature=0.9)
    _ok(full_parity(wl))


def test_greedy_batch():
    wl = workloads.make_custom(5000, 64, 3, 6, seed=4, temperature=0.0)
    _ok(full_parity(wl))


def test_low_temperature():
    # z / T spans thousands: exp underflows everywhere but at the maximum
    wl = workloads.make_custom(4000, 64, 3, 4, seed=5, temperature=0.002)
    _ok(full_parity(wl))


def test_topk_smallest_vocabulary():
    import torch
    import markov_draft_sampling_amd as mds
    from parity import dev_tensors
    wl = workloads.make_custom(2, 32, 3, 3, seed=9, temperature=1.1)
    for k in (1, 2):
        d = dev_tensors(wl)
        spos = torch.from_numpy(wl.anchor_pos[:, None] + 1 + np.arange(wl.K)[None, :]).cuda()
        mds.markov_draft_loop_topk(d["base"], d["w1"], d["w2"], d["anchor_tokens"], None, spos, d["temperature"],
                                   d["seeds"], d["cache"], d["draft_tokens"], k, draft_lse=d["draft_lse"])
        torch.cuda.synchronize()
        rep = Report()
        compare_draft(wl, np.arange(wl.B), d["draft_tokens"].cpu().numpy(), cache_to_numpy(d["cache"], "f32"),
                      d["draft_lse"].cpu().numpy(), rep, topk=k)
        _ok(rep)


def test_lm_head_single_row():
    import torch
    import markov_draft_sampling_amd as mds
    hidden, lm = workloads.make_lm_head(1, 37, 256, seed=3)
    h = torch.from_numpy(hidden.view(np.int16)).view(torch.bfloat16).cuda()
    w = torch.from_numpy(lm.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.full((1, 1, 37), 3.0, dtype=torch.float32, device="cuda")
    mds.draft_lm_head(h, w, out, 1)
    torch.cuda.synchronize()
    ref, absd = oracle.draft_logits(hidden, lm, want_abs=True)
    err = np.abs(out.cpu().numpy().reshape(1, 37).astype(np.float64) - ref)
    assert (err <= 256 * 2.0 ** -24 * absd + 2.0 ** -24 * np.abs(ref)).all()


@pytest.mark.parametrize("top_p", [None, 0.9])
def test_rows_without_a_finite_logit(top_p):
    # masked rows (every column -inf): a draft base row gives token 0 and a
    # draft distribution q that is the one-hot at 0; a target row gives p
    # (and its top-p kept set) the one-hot at 0; checked against the oracle
    V, K, B = 3000, 3, 6
    wl = workloads.make_custom(V, 64, K, B, seed=5, temperature=0.9, top_p=top_p)
    wl.base[1, 0, :] = -np.inf
    wl.base[2, 1, :] = -np.inf
    wl.base[5, :, :] = -np.inf
    tgt = wl.target.reshape(B, K + 1, V)
    tgt[3, 0, :] = -np.inf
    tgt[4, :, :] = -np.inf
    tgt[2, 1, :] = -np.inf
    tgt[5, :, :] = -np.inf
    rep = full_parity(wl)
    _ok(rep)
    from parity import run_gpu
    d = run_gpu(wl)
    toks = d["draft_tokens"].cpu().numpy()
    out = d["out_tokens"].cpu().numpy()
    nacc = d["num_accepted"].cpu().numpy()
    assert toks[1, 0] == 0 and toks[2, 1] == 0 and np.all(toks[5] == 0)
    # request 5: p and q both one-hot at 0 and every draft 0, so all accepted
    # and the bonus from the masked last row is 0
    assert nacc[5] == K and np.all(out[5] == 0)
    # request 4: every target row masked, so the emitted token is always 0
    assert out[4, nacc[4]] == 0
