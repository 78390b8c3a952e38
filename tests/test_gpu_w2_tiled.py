"""markov_w2 in the tiled order (mds_tile_markov_w2, MDS_DRAFT_W2_TILED).

The tiling kernel's output must follow the layout's index formula, written
out here with numpy independently of the kernel. The draft loop run on the
tiled matrix must give, bit for bit, the tokens, cache and draft_lse of the
same call on the row-major matrix (which the other parity tests check against
the oracle); one small case is also compared with the oracle directly.
Shapes: the headline (every tile full: the fixed-count fast loop), B = 1 and
8 (padding rows in the batch tile), B = 128 (four batch tiles: the general
loop), ragged vocabularies (the padded last tile), ranks 96 and 128 (fewer
rank slices), bf16 base and cache, greedy and T != 1 rows, the fp64 Gumbel
option and request-state indexing.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from parity import Report, compare_draft, cache_to_numpy

pytestmark = pytest.mark.gpu


def _bf16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("V,r", [(200064, 256), (33001, 256), (1000, 96), (17, 512)])
def test_tiled_order_follows_the_index_formula(V, r):
    import torch
    import markov_draft_sampling_amd as mds
    print(f"tile w2: V={V} r={r}", flush=True)
    rng = np.random.default_rng([V, r])
    w2 = rng.integers(0, 1 << 16, (V, r), dtype=np.uint16)  # bit patterns: the tiling only moves them
    w2d = _bf16(w2)
    got = mds.tile_markov_w2(w2d)
    T = -(-V // 16)
    assert tuple(got.shape) == (T, 16 * r)
    # into a given buffer holding other values: every element, padding included, is written
    buf = torch.full((T, 16 * r), 7.0, dtype=torch.bfloat16, device="cuda")
    assert mds.tile_markov_w2(w2d, out=buf) is buf
    torch.cuda.synchronize()
    # element (v, j) at t*16r + s*512 + (m + 16 g)*8 + e with v = 16 t + m, j = 32 s + 8 g + e
    padded = np.zeros((T * 16, r), np.uint16)
    padded[:V] = w2
    want = padded.reshape(T, 16, r // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(T, 16 * r)
    for t in (got, buf):
        assert np.array_equal(t.view(torch.int16).cpu().numpy().view(np.uint16), want)


def _run_both(wl, temp=None, fp64=False, indexed=False):
    """The _ex call on row-major and on tiled w2; returns both outputs as bit arrays."""
    import torch
    import markov_draft_sampling_amd as mds
    B, K, V = wl.B, wl.K, wl.V
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    base = _bf16(wl.base) if wl.base_dtype == "bf16" else t(wl.base)
    w1, w2 = _bf16(wl.w1), _bf16(wl.w2)
    w2t = mds.tile_markov_w2(w2)
    temp = wl.temperature if temp is None else temp
    seeds = wl.seeds
    spos = (wl.anchor_pos[:, None] + 1 + np.arange(K)[None, :]).astype(np.int64)
    idx = rowmap = None
    n_slots = n_rows = B
    if indexed:
        rng = np.random.default_rng([B, K, V])
        n_slots, n_rows = 2 * B, B
        perm = rng.permutation(n_slots)[:B].astype(np.int32)
        perm[1] = -1  # a padding request
        idx = np.repeat(perm[:, None], K, axis=1).astype(np.int32)
        idx[0, K // 2] = -1  # an inert step
        rowmap = np.zeros(n_slots, np.int32)
        rowmap[perm[perm >= 0]] = rng.permutation(n_rows)[: (perm >= 0).sum()]
        t_s = np.ones(n_slots, np.float32)
        t_s[perm[perm >= 0]] = temp[perm >= 0]
        s_s = rng.integers(0, 2**63, n_slots, dtype=np.int64)
        s_s[perm[perm >= 0]] = seeds[perm >= 0]
        temp, seeds = t_s, s_s
    cdt = torch.bfloat16 if wl.cache_dtype == "bf16" else torch.float32
    out = []
    for tiled in (False, True):
        cache = torch.full((n_rows, K, V), -3.5, dtype=cdt, device="cuda")
        toks = torch.full((B, K), -9, dtype=torch.int32, device="cuda")
        lse = torch.full((B, K), -9.0, dtype=torch.float32, device="cuda")
        ws = mds.new_workspace(mds.draft_workspace_bytes(B, K, V, wl.r), torch.device("cuda"))
        mds.markov_draft_loop_ex(base, w1, w2t if tiled else w2, t(wl.anchor_tokens), None if idx is None else t(idx),
                                 t(spos), t(temp), t(seeds), cache, toks, row_mapping=None if rowmap is None
                                 else t(rowmap), draft_lse=lse, fp64_gumbel=fp64, workspace=ws, w2_tiled=tiled)
        torch.cuda.synchronize()
        out.append((toks.cpu().numpy(), cache_to_numpy(cache, wl.cache_dtype), lse.cpu().numpy().view(np.uint32),
                    mds.workspace_status(ws)))
    return out


def _assert_same(out):
    (k0, c0, l0, s0), (k1, c1, l1, s1) = out
    assert np.array_equal(k0, k1), np.argwhere(k0 != k1)[:5]
    assert np.array_equal(c0.view(np.uint8), c1.view(np.uint8)), np.argwhere(c0 != c1)[:5]
    assert np.array_equal(l0, l1)
    assert s0 == s1
    return k0


@pytest.mark.parametrize("B", [32, 8, 1])
def test_tiled_equals_row_major_headline(B):
    wl = workloads.make_workload("headline_v200064", B=B)
    print(f"tiled vs row-major: headline B={B}", flush=True)
    k = _assert_same(_run_both(wl))
    assert ((k >= 0) & (k < wl.V)).all()


@pytest.mark.parametrize("V,r,K,B,dt", [
    (50017, 256, 3, 128, "f32"),   # four batch tiles, ragged vocabulary
    (33001, 256, 7, 32, "f32"),    # fast loop plus the padded last tile
    (70001, 128, 4, 16, "f32"),    # rank 128
    (5000, 96, 3, 5, "bf16"),      # rank 96, bf16 base and cache, padding rows
])
def test_tiled_equals_row_major(V, r, K, B, dt):
    print(f"tiled vs row-major: V={V} r={r} K={K} B={B} {dt}", flush=True)
    wl = workloads.make_custom(V, r, K, B, seed=V + B, base_dtype=dt, cache_dtype=dt)
    temp = wl.temperature.copy()
    temp[1::3] = 0.7
    temp[::4] = 0.0  # greedy rows
    _assert_same(_run_both(wl, temp=temp))


def test_tiled_equals_row_major_fp64_gumbel():
    print("tiled vs row-major: headline B=32, fp64 Gumbel", flush=True)
    _assert_same(_run_both(workloads.make_workload("headline_v200064", B=32), fp64=True))


def test_tiled_equals_row_major_indexed():
    print("tiled vs row-major: indexed V=8200 B=12", flush=True)
    wl = workloads.make_custom(8200, 64, 4, 12, seed=5)
    k = _assert_same(_run_both(wl, indexed=True))
    assert (k[1] == -1).all() and k[0, 2] == -1


def test_tiled_matches_the_oracle():
    print("tiled vs oracle: V=4099 r=256 K=3 B=5", flush=True)
    wl = workloads.make_custom(4099, 256, 3, 5, seed=9)
    (_, _, _, _), (k1, c1, l1, _) = _run_both(wl)
    rep = Report()
    compare_draft(wl, np.arange(wl.B), k1, c1, l1.view(np.float32), rep)
    assert rep.ok(), rep
    assert rep.tokens_total == wl.B * wl.K


def test_tiled_headline_matches_the_oracle():
    # the draft call exactly as the benchmark times it (indexed entry point,
    # tiled w2, per-step sample positions) against the oracle on every request
    print("tiled vs oracle: headline V=200064 r=256 K=7 B=32", flush=True)
    wl = workloads.make_workload("headline_v200064", B=32)
    (_, _, _, _), (k1, c1, l1, st) = _run_both(wl)
    rep = Report()
    compare_draft(wl, np.arange(wl.B), k1, c1, l1.view(np.float32), rep)
    assert rep.ok(), rep.notes[:5]
    assert rep.tokens_total == wl.B * wl.K and st == 0
