"""The draft LM head and the Markov loop in one call (mds_markov_draft_loop_from_hidden).

Its outputs must equal those of the two calls it stands for, mds_draft_lm_head
then mds_markov_draft_loop on the same inputs (both checked against the
oracle elsewhere): draft tokens, the draft-logits cache and the base rows of
steps 1..K-1 bit for bit; draft_lse within float32 summation-order rounding
(the fused step 0 merges q partials over a different column partition).
Shapes cover the fused path (B <= 32, B*K <= 256, rank <= 256: full rounds of
256-row tiles plus a 64-row tail, a vocabulary below one round, padding
requests, greedy rows, bf16 base and cache, rank 128) and the two-launch
fallback (B > 32, B*K > 256).
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


def _run(B, K, V, H, r, *, seed, base_dtype="f32", cache_dtype="f32", greedy_every=0):
    import torch
    import markov_draft_sampling_amd as mds
    wl = workloads.make_custom(V, r, K, B, seed=seed)
    hidden, lm = workloads.make_lm_head(B * K, V, H, seed=seed)
    print(f"fused LM head + loop: B={B} K={K} V={V} H={H} r={r} base={base_dtype} cache={cache_dtype}", flush=True)
    bits = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    h, w, w1, w2 = bits(hidden), bits(lm), bits(wl.w1), bits(wl.w2)
    temp = wl.temperature.copy()
    temp[1::3] = 0.7
    if greedy_every:
        temp[::greedy_every] = 0.0
    args = (t(wl.anchor_tokens), t(wl.anchor_pos), t(temp), t(wl.seeds))
    bdt = torch.bfloat16 if base_dtype == "bf16" else torch.float32
    cdt = torch.bfloat16 if cache_dtype == "bf16" else torch.float32
    out = {}
    for name in ("two_calls", "fused"):
        base = torch.full((B, K + 1, V), 7.25, dtype=bdt, device="cuda")
        cache = torch.full((B, K, V), -3.5, dtype=cdt, device="cuda")
        toks = torch.full((B, K), -9, dtype=torch.int32, device="cuda")
        lse = torch.full((B, K), -9.0, dtype=torch.float32, device="cuda")
        if name == "two_calls":
            mds.draft_lm_head(h, w, base, K)
            mds.markov_draft_loop(base, w1, w2, *args, cache, toks, lse)
        else:
            mds.markov_draft_loop_from_hidden(h, w, base, w1, w2, *args, cache, toks, lse)
        torch.cuda.synchronize()
        as_bits = lambda x: x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32).cpu().numpy()  # noqa: E731
        out[name] = (as_bits(base[:, 1:K]), as_bits(cache), toks.cpu().numpy(), lse.cpu().numpy())
    (b0, c0, k0, l0), (b1, c1, k1, l1) = out["two_calls"], out["fused"]
    assert np.array_equal(k0, k1), np.argwhere(k0 != k1)[:5]
    assert np.array_equal(c0, c1), np.argwhere(c0 != c1)[:5]
    assert np.array_equal(b0, b1)
    assert ((l0 == l1) | (np.isnan(l0) & np.isnan(l1)) | (np.abs(l0 - l1) <= 2e-6 * np.abs(l0))).all(), (l0, l1)
    assert (k0 >= 0).all() and (k0 < V).all()


@pytest.mark.parametrize("B,K,V,H,r", [
    (32, 7, 200064, 256, 256),   # the headline shape: 768 tiles of 256 rows plus a 64-row tail
    (5, 3, 4099, 256, 256),      # below one round: 64-row tiles only; padding requests 5..31
    (16, 4, 70001, 512, 128),    # rank 128, ragged vocabulary
    (1, 1, 1000, 256, 256),      # one row
])
def test_fused_loop_equals_the_two_calls(B, K, V, H, r):
    _run(B, K, V, H, r, seed=B * 131 + V)


def test_fused_loop_bf16_base_and_cache_with_greedy_rows():
    _run(32, 7, 33001, 256, 256, seed=5, base_dtype="bf16", cache_dtype="bf16", greedy_every=4)


@pytest.mark.parametrize("B,K", [(40, 3), (32, 9)])
def test_unfused_fallback_equals_the_two_calls(B, K):
    _run(B, K, 5000, 256, 256, seed=B + K)


def test_fused_loop_headline_hidden_size():
    _run(32, 7, 200064, 4096, 256, seed=11)
