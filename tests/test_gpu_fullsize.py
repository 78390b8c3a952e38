"""Parity at the full workload sizes, in the launch configuration bench.py
times: the headline workload (V=200064, r=256, K=7, fp32) at B = 1, 8, 32
and 128, and the bf16 top-p workload (V=151936, r=256, K=7, B=32). Every
request is compared with the oracle: its draft tokens under teacher forcing,
its whole draft-logits cache, its draft log-sum-exp, and its verification on
the GPU's own drafts and cache. The oracle runs over chunks of requests to
bound host memory; each case prints its excused and unexcused counts."""
import numpy as np
import pytest

import workloads
from parity import Report, compare_draft, compare_verify, run_gpu, cache_to_numpy

pytestmark = pytest.mark.gpu

CHUNK = 8  # requests per oracle call


def _check(wl, label):
    d = run_gpu(wl)
    toks = d["draft_tokens"].cpu().numpy()
    out = d["out_tokens"].cpu().numpy()
    nacc = d["num_accepted"].cpu().numpy()
    lse = d["draft_lse"].cpu().numpy()
    cache = cache_to_numpy(d["cache"], wl.cache_dtype)
    del d
    rep = Report()
    for b0 in range(0, wl.B, CHUNK):
        rows = np.arange(b0, min(wl.B, b0 + CHUNK))
        compare_draft(wl, rows, toks, cache, lse, rep)
        compare_verify(wl, rows, toks, cache, out, nacc, rep)
    assert rep.req_total == wl.B and rep.tokens_total == wl.B * wl.K
    assert rep.cache_total == wl.B * wl.K * wl.V
    # properties that hold for every request
    assert np.all((toks >= 0) & (toks < wl.V))
    for b in range(wl.B):
        n = nacc[b]
        assert 0 <= n <= wl.K
        assert np.array_equal(out[b, :n], toks[b, :n])
        assert 0 <= out[b, n] < wl.V and np.all(out[b, n + 1:] == -1)
    print(f"PARITY {label}: tokens {rep.tokens_total} excused {rep.tokens_excused} bad {rep.tokens_bad}; "
          f"cache {rep.cache_total} max err {rep.cache_max_err:.2e} excused {rep.cache_excused} bad {rep.cache_bad}; "
          f"lse max err {rep.lse_max_err:.1e} bad {rep.lse_bad}; requests {rep.req_total} excused "
          f"{rep.req_excused} bad {rep.req_bad}", flush=True)
    assert rep.ok(), rep.notes[:5]


@pytest.mark.parametrize("B", workloads.HEADLINE_BATCHES)
def test_headline_workload(B):
    wl = workloads.make_workload("headline_v200064", B=B)
    _check(wl, f"headline V=200064 B={B}")


def test_bf16_top_p_workload():
    wl = workloads.make_workload("zipf_top_p_v151936")
    _check(wl, "bf16 top-p V=151936 B=32")
