"""Test helpers: run the HIP path on a workload and compare it with the oracle.

Parity rules:
* draft token (b, k): must equal the oracle's, unless the oracle's top-two
  float32 scores at that step differ by at most 1e-3 (excused);
* accept count / emitted tokens of a request: must equal the oracle's, unless
  some compared step's |p/q - u| <= 1e-5, the final draw's top-two score gap
  <= 1e-3, or a compared row's top-p cut lies within 1e-6 of p (excused);
* cache: |gpu - oracle| <= 2e-3 per element; a bf16 element whose float32
  value lies within 8 float32 ulps of a bf16 rounding midpoint may differ by
  one bf16 ulp (excused);
* draft log-sum-exp: |gpu - oracle| <= 1e-4 + 1e-5 |oracle|.
Every excused and unexcused mismatch is counted.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
from workloads import Workload, bf16_bits_to_f32

TOK_MARGIN = 1e-3
ACC_MARGIN = 1e-5
CACHE_TOL = 2e-3


def torch_mod():
    import torch
    return torch


def dev_tensors(wl: Workload, device="cuda", pad_to: int | None = None):
    """Device copies of a workload's inputs plus output buffers.

    pad_to: round the row length of base/cache/target up to a multiple of this
    (strided rows) to exercise the vector path on odd V.
    """
    torch = torch_mod()
    B, K, V = wl.B, wl.K, wl.V
    Vp = V if not pad_to else (V + pad_to - 1) // pad_to * pad_to

    def padded(arr, dtype):
        shape = arr.shape[:-1] + (Vp,)
        t = torch.zeros(shape, dtype=dtype, device=device)
        src = torch.from_numpy(np.ascontiguousarray(arr))
        if dtype == torch.bfloat16:
            src = src.view(torch.int16).view(torch.bfloat16)
        t[..., :V] = src.to(device)
        return t[..., :V]

    base = padded(wl.base.view(np.int16) if wl.base_dtype == "bf16" else wl.base,
                  torch.bfloat16 if wl.base_dtype == "bf16" else torch.float32)
    target = padded(wl.target, torch.float32)
    cdt = torch.bfloat16 if wl.cache_dtype == "bf16" else torch.float32
    cache = torch.full((B, K, Vp), float("nan"), dtype=cdt, device=device)[..., :V]
    w1 = torch.from_numpy(wl.w1.view(np.int16)).view(torch.bfloat16).to(device)
    w2 = torch.from_numpy(wl.w2.view(np.int16)).view(torch.bfloat16).to(device)
    d = dict(
        base=base, w1=w1, w2=w2, target=target, cache=cache,
        anchor_tokens=torch.from_numpy(wl.anchor_tokens).to(device),
        anchor_pos=torch.from_numpy(wl.anchor_pos).to(device),
        temperature=torch.from_numpy(wl.temperature).to(device),
        seeds=torch.from_numpy(wl.seeds).to(device),
        top_p=None if wl.top_p is None else torch.from_numpy(wl.top_p).to(device),
        draft_tokens=torch.full((B, K), -7, dtype=torch.int32, device=device),
        draft_lse=torch.full((B, K), float("nan"), dtype=torch.float32, device=device),
        out_tokens=torch.full((B, K + 1), -9, dtype=torch.int32, device=device),
        num_accepted=torch.full((B,), -9, dtype=torch.int32, device=device),
    )
    return d


def run_gpu(wl: Workload, d=None, with_lse=True, verify=True, pad_to=None):
    import markov_draft_sampling_amd as mds
    torch = torch_mod()
    d = d or dev_tensors(wl, pad_to=pad_to)
    mds.markov_draft_loop(d["base"], d["w1"], d["w2"], d["anchor_tokens"], d["anchor_pos"], d["temperature"],
                          d["seeds"], d["cache"], d["draft_tokens"], d["draft_lse"])
    if verify:
        mds.rejection_verify(d["target"], d["cache"], d["draft_tokens"], d["temperature"], d["seeds"], d["anchor_pos"],
                             d["out_tokens"], d["num_accepted"], draft_lse=d["draft_lse"] if with_lse else None,
                             top_p=d["top_p"])
    torch.cuda.synchronize()
    return d


def cache_to_numpy(cache, cache_dtype):
    torch = torch_mod()
    c = cache.contiguous().cpu()
    if cache_dtype == "bf16":
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()


@dataclasses.dataclass
class Report:
    tokens_total: int = 0
    tokens_excused: int = 0
    tokens_bad: int = 0
    cache_total: int = 0
    cache_excused: int = 0
    cache_bad: int = 0
    cache_max_err: float = 0.0
    lse_bad: int = 0
    lse_max_err: float = 0.0
    req_total: int = 0
    req_excused: int = 0
    req_bad: int = 0
    notes: list = dataclasses.field(default_factory=list)

    def ok(self):
        return self.tokens_bad == 0 and self.cache_bad == 0 and self.lse_bad == 0 and self.req_bad == 0


def _midpoint_near(z32: np.ndarray) -> np.ndarray:
    low = z32.view(np.uint32) & np.uint32(0xFFFF)
    return np.abs(low.astype(np.int64) - 0x8000) <= 8


def compare_draft(wl: Workload, rows, gpu_tokens, gpu_cache, gpu_lse, rep: Report, **oracle_kw):
    """Teacher-forced oracle on requests `rows`; compares tokens, cache and lse.

    oracle_kw: options of the draft loop (topk, fp64_gumbel) passed to the oracle.
    """
    with np.errstate(invalid="ignore"):  # inf - inf where both sides hold the same infinity
        return _compare_draft(wl, rows, gpu_tokens, gpu_cache, gpu_lse, rep, **oracle_kw)


def _compare_draft(wl: Workload, rows, gpu_tokens, gpu_cache, gpu_lse, rep: Report, **oracle_kw):
    rows = np.asarray(rows)
    base = wl.draft_base[rows]
    teacher = gpu_tokens[rows]
    args = (base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens[rows], wl.anchor_pos[rows], wl.seeds[rows],
            wl.temperature[rows])
    ref = oracle.draft_loop(*args, wl.cache_dtype, teacher=teacher, **oracle_kw)
    # tokens
    mism = ref["tokens"] != teacher
    exc = mism & (ref["margin"] <= TOK_MARGIN)
    rep.tokens_total += mism.size
    rep.tokens_excused += int(exc.sum())
    rep.tokens_bad += int((mism & ~exc).sum())
    if (mism & ~exc).any():
        i = np.argwhere(mism & ~exc)[0]
        rep.notes.append(f"token mismatch at request {rows[i[0]]} step {i[1]}: gpu {teacher[tuple(i)]} "
                         f"oracle {ref['tokens'][tuple(i)]} margin {ref['margin'][tuple(i)]}")
    # cache
    gc = gpu_cache[rows]
    if wl.cache_dtype == "bf16":
        g = bf16_bits_to_f32(gc).astype(np.float64)
        o = bf16_bits_to_f32(ref["cache"]).astype(np.float64)
        z32 = oracle.draft_loop(*args, "f32", teacher=teacher, **oracle_kw)["cache"]
        near = _midpoint_near(z32)
        ulp = np.abs(o) * 2.0 ** -7
        err = np.abs(g - o)
        both_nan = np.isnan(g) & np.isnan(o)
        bad = ~both_nan & ~(err <= CACHE_TOL) & (g != o)
        excused = bad & near & (err <= ulp * 1.01)
        bad &= ~excused
        rep.cache_excused += int(excused.sum())
    else:
        g = gc.astype(np.float64)
        o = ref["cache"].astype(np.float64)
        err = np.abs(g - o)
        both_nan = np.isnan(g) & np.isnan(o)
        bad = ~both_nan & ~(err <= CACHE_TOL) & (g != o)
    rep.cache_total += bad.size
    rep.cache_bad += int(bad.sum())
    fin = np.isfinite(err)
    if fin.any():
        rep.cache_max_err = max(rep.cache_max_err, float(err[fin].max()))
    if bad.any():
        i = np.argwhere(bad)[0]
        rep.notes.append(f"cache mismatch at {tuple(int(x) for x in i)}: gpu {g[tuple(i)]} oracle {o[tuple(i)]}")
    # lse (sampled requests only)
    if gpu_lse is not None:
        samp = wl.temperature[rows] > 0
        gl = gpu_lse[rows][samp].astype(np.float64)
        ol = ref["lse"][samp]
        err = np.abs(gl - ol)
        both_nan = np.isnan(gl) & np.isnan(ol)
        badl = ~both_nan & ~(err <= 1e-4 + 1e-5 * np.abs(ol)) & (gl != ol)
        rep.lse_bad += int(badl.sum())
        if (~both_nan).any():
            e = err[~both_nan]
            if np.isfinite(e).any():
                rep.lse_max_err = max(rep.lse_max_err, float(e[np.isfinite(e)].max()))
        if badl.any():
            rep.notes.append(f"lse mismatch: gpu {gl[badl][:3]} oracle {ol[badl][:3]}")
    return ref


def compare_verify(wl: Workload, rows, gpu_tokens, gpu_cache, gpu_out, gpu_nacc, rep: Report):
    """Oracle verification of requests `rows` on the GPU's drafts and cache."""
    rows = np.asarray(rows)
    K = wl.K
    tgt = wl.target.reshape(wl.B, K + 1, wl.V)[rows].reshape(len(rows) * (K + 1), wl.V)
    ref = oracle.verify(tgt, gpu_cache[rows], wl.cache_dtype, gpu_tokens[rows], wl.temperature[rows],
                        None if wl.top_p is None else wl.top_p[rows], wl.seeds[rows], wl.anchor_pos[rows])
    same = (ref["num_accepted"] == gpu_nacc[rows]) & np.all(ref["out_tokens"] == gpu_out[rows], axis=1)
    exc = (~same) & ((ref["accept_margin"] <= ACC_MARGIN) | (ref["sample_margin"] <= TOK_MARGIN) |
                     ref["near_top_p"])
    rep.req_total += len(rows)
    rep.req_excused += int(exc.sum())
    bad = ~same & ~exc
    rep.req_bad += int(bad.sum())
    if bad.any():
        i = int(np.argwhere(bad)[0][0])
        rep.notes.append(f"verify mismatch request {rows[i]}: gpu {gpu_out[rows][i]} n={gpu_nacc[rows][i]} "
                         f"oracle {ref['out_tokens'][i]} n={ref['num_accepted'][i]} "
                         f"acc_margin {ref['accept_margin'][i]} smp_margin {ref['sample_margin'][i]}")
    return ref


def full_parity(wl: Workload, rows=None, with_lse=True, pad_to=None) -> Report:
    d = run_gpu(wl, with_lse=with_lse, pad_to=pad_to)
    rows = np.arange(wl.B) if rows is None else np.asarray(rows)
    toks = d["draft_tokens"].cpu().numpy()
    cache = cache_to_numpy(d["cache"], wl.cache_dtype)
    lse = d["draft_lse"].cpu().numpy()
    out = d["out_tokens"].cpu().numpy()
    nacc = d["num_accepted"].cpu().numpy()
    rep = Report()
    compare_draft(wl, rows, toks, cache, lse, rep)
    compare_verify(wl, rows, toks, cache, out, nacc, rep)
    return rep
