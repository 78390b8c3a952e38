"""GPU parity of the draft LM head (mds_draft_lm_head).

Element by element against the oracle (exact products, float64 sums, one
rounding) within the float32 summation bound: any order of H float32
additions is within H * 2^-24 * sum|hidden * lm_head| of the exact sum, plus
the rounding of the output (2^-24 relative for float32, 2^-8 for bf16).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu


def _dev(hidden, lm):
    import torch
    h = torch.from_numpy(hidden.view(np.int16)).view(torch.bfloat16).cuda()
    w = torch.from_numpy(lm.view(np.int16)).view(torch.bfloat16).cuda()
    return h, w


def _check(hidden, lm, got, out_dtype="f32", cols=None):
    ref, absd = oracle.draft_logits(hidden, lm, cols=cols, want_abs=True)
    H = hidden.shape[1]
    ref = ref.astype(np.float64)
    tol = H * 2.0 ** -24 * absd + 2.0 ** -24 * np.abs(ref)
    if out_dtype == "bf16":
        got = workloads.bf16_bits_to_f32(got)
        tol = tol + 2.0 ** -8 * np.abs(ref)
    err = np.abs(got.astype(np.float64) - ref)
    assert (err <= tol).all(), (np.argwhere(err > tol)[:5], float(err.max()))
    return float(err.max())


def _run(B, K, V, H, seed, out_dtype="f32", pad=0, extra_steps=0):
    import torch
    import markov_draft_sampling_amd as mds
    hidden, lm = workloads.make_lm_head(B * K, V, H, seed=seed)
    h, w = _dev(hidden, lm)
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    sentinel = 7.25
    out = torch.full((B, K + extra_steps, V + pad), sentinel, dtype=dt, device="cuda")[..., :V]
    mds.draft_lm_head(h, w, out, K)
    torch.cuda.synchronize()
    o = out.contiguous().cpu()
    if out_dtype == "bf16":
        arr = o.view(torch.int16).numpy().view(np.uint16)
    else:
        arr = o.numpy()
    # rows past K are not written
    if extra_steps:
        rest = arr[:, K:]
        assert (rest == (0x40E8 if out_dtype == "bf16" else np.float32(sentinel))).all()
    return hidden, lm, arr[:, :K].reshape(B * K, V)


@pytest.mark.parametrize("B,K,V,H", [(1, 7, 4096, 256), (8, 7, 32000, 512), (32, 7, 12345, 256), (3, 5, 130, 256),
                                     (2, 3, 999, 1024), (5, 3, 700, 768),
                                     # past one round of 128-row tiles on 256 CUs: 64-row tail tiles, ragged
                                     (2, 3, 33001, 256)])
def test_lm_head_matches_oracle(B, K, V, H):
    hidden, lm, got = _run(B, K, V, H, seed=B * 31 + V)
    _check(hidden, lm, got)


def test_lm_head_two_row_tiles_bf16_strided():
    hidden, lm, got = _run(40, 7, 5000, 512, seed=3, out_dtype="bf16", pad=24, extra_steps=1)
    _check(hidden, lm, got, out_dtype="bf16")


def test_lm_head_headline_sampled_columns():
    B, K, V, H = 32, 7, 200064, 4096
    hidden, lm, got = _run(B, K, V, H, seed=4)
    rng = np.random.default_rng(0)
    cols = np.concatenate([rng.choice(V - 64, 1024, replace=False), np.arange(V - 64, V)])
    _check(hidden, lm, got[:, cols], cols=cols)


def test_lm_head_feeds_the_draft_loop():
    import torch
    import markov_draft_sampling_amd as mds
    wl = workloads.make_custom(4096, 64, 3, 4, seed=6)
    hidden, lm = workloads.make_lm_head(wl.B * wl.K, wl.V, 256, seed=6)
    h, w = _dev(hidden, lm)
    base = torch.zeros((wl.B, wl.K + 1, wl.V), dtype=torch.float32, device="cuda")
    mds.draft_lm_head(h, w, base, wl.K)
    w1 = torch.from_numpy(wl.w1.view(np.int16)).view(torch.bfloat16).cuda()
    w2 = torch.from_numpy(wl.w2.view(np.int16)).view(torch.bfloat16).cuda()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    cache = torch.empty((wl.B, wl.K, wl.V), dtype=torch.float32, device="cuda")
    toks = torch.empty((wl.B, wl.K), dtype=torch.int32, device="cuda")
    mds.markov_draft_loop(base, w1, w2, t(wl.anchor_tokens), t(wl.anchor_pos), t(wl.temperature), t(wl.seeds), cache,
                          toks)
    torch.cuda.synchronize()
    gbase = base.cpu().numpy()
    _check(hidden, lm, gbase[:, : wl.K].reshape(-1, wl.V))
    g = toks.cpu().numpy()
    ref = oracle.draft_loop(gbase, "f32", wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, wl.seeds, wl.temperature,
                            "f32", K=wl.K, teacher=g)
    assert not ((ref["tokens"] != g) & (ref["margin"] > 1e-3)).any()


def test_lm_head_rejects_unsupported_hidden_size():
    import torch
    import markov_draft_sampling_amd as mds
    hidden, lm = workloads.make_lm_head(4, 100, 96, seed=1)
    h, w = _dev(hidden, lm)
    out = torch.empty((2, 2, 100), dtype=torch.float32, device="cuda")
    with pytest.raises(mds.MdsError):
        mds.draft_lm_head(h, w, out, 2)
