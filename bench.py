"""Benchmark of one draft + verify step on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--batch 32]

A step is one pass of the whole hot path over one batch: the K-step Markov
draft loop (fused projection + sampling + cache write per step) followed by
rejection verification, on synthetic inputs of the headline workload:
V=200064, r=256 (w2 = 102 MB bf16), K=7, B=32, fp32 base logits, target and
draft-logits cache. Inputs are resident in HBM before timing starts. The
Markov step kernels read w2 in its tiled order (mds_tile_markov_w2, made once
from the row-major matrix before the first step, as weights are prepared at
load time; --w2-layout row-major reads the [V, r] matrix itself).

Timing: W untimed steps, then S timed steps. Before each timed step a 512 MiB
buffer is read so the Infinity Cache (MALL) and L2 hold none of the inputs
(the target model's forward pass evicts them in serving); reading rather than
writing leaves no dirty lines whose write-back would compete with the step.
Each step is timed
with HIP events on the stream the kernels run on, and the flush is outside
the events. The same steps run back to back without flushes are reported as
`warm`. For the roofline entry the steps run once more, the library
recording events around the launches of the dominant kernel (the fused
Markov-step kernel, or the variant's); those records sit between kernels, so
this pass is not the timed one.

Prints one JSON line. One GPU only: --gpus N with N > 1 exits with an error.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "draft+verify tokens/s at V=200k,K=7,B=32; HBM GB/s % of MI355X peak"


def algorithmic_bytes(B, K, V, r, s_base=4, s_cache=4, s_tgt=4, top_p=False):
    """Bytes the method must move per step (each w2 byte once per Markov step).

    Verification reads every target row once for its statistics and one
    target and one cache row per request for the final draw; with top-p the
    kept set needs one more pass over the target rows (its threshold is not
    known until the statistics are)."""
    draft_step = V * r * 2 + B * V * (s_base + s_cache)
    draft = K * draft_step
    verify = B * (K + 1) * V * s_tgt + B * V * (s_tgt + s_cache)
    if top_p:
        verify += B * (K + 1) * V * s_tgt
    return draft_step, draft, verify


def topk_bytes(B, K, V, r, topk, s_base=4, s_cache=4):
    """Top-k drafting: bytes of the selection launch (base logits read once,
    the -inf cache rows written, the chunk candidates written) and of the
    whole draft call (plus the merge and the K-step chain over gathered rows)."""
    NC = -(-V // 8192)
    select = B * K * V * (s_base + s_cache) + B * K * NC * topk * 8
    merge = B * K * NC * topk * 8 + B * K * topk * 4
    chain = B * K * (topk * (r * 2 + s_base + s_cache + 4) + r * 2)
    return select, select + merge + chain


def lm_head_bytes(M, V, H, s_out=4):
    """Draft LM head: lm_head and hidden read once, the base logits written."""
    return V * H * 2 + M * H * 2 + M * V * s_out


def fused_draft_bytes(B, K, V, r, H, s_base=4, s_cache=4):
    """The draft call from hidden states: the LM head (lm_head, hidden, base rows
    of steps 1..K-1 written), step 0 in its work-groups (w2, cache row 0), then
    steps 1..K-1 (w2, base row, cache row each)."""
    return (V * H * 2 + B * K * H * 2 + B * (K - 1) * V * s_base + (V * r * 2 + B * V * s_cache)
            + (K - 1) * (V * r * 2 + B * V * (s_base + s_cache)))


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "markov_draft_sampling_amd", "csrc")


def recorded_traffic(profile: str, sources) -> float | None:
    """HBM bytes per launch from a committed counter summary, or None when the
    kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(PROFILES, profile)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "kernel_source_sha256"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256(b"".join(open(os.path.join(CSRC, n), "rb").read() for n in sources)).hexdigest()
    if fields.get("kernel_source_sha256") != h or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


def cpu_baseline(wl, n_req: int, repeats: int = 2, lm=None, **draft_kw):
    """The oracle, as it stands, on the first n_req requests of the workload
    (draft_kw: the draft loop's options, topk or fp64_gumbel; lm: (hidden,
    lm_head) bf16 bits, whose LM head then gives the base logits)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        ctx = None
    rows = np.arange(n_req)
    K = wl.K
    tgt = wl.target.reshape(wl.B, K + 1, wl.V)[rows].reshape(n_req * (K + 1), wl.V)
    t0 = time.perf_counter()
    for _ in range(repeats):
        base = wl.draft_base[rows]
        if lm is not None:
            base = oracle.draft_logits(lm[0][: n_req * K], lm[1]).reshape(n_req, K, wl.V)
        d = oracle.draft_loop(base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens[rows],
                              wl.anchor_pos[rows], wl.seeds[rows], wl.temperature[rows], wl.cache_dtype, **draft_kw)
        oracle.verify(tgt, d["cache"], wl.cache_dtype, d["tokens"], wl.temperature[rows],
                      None if wl.top_p is None else wl.top_p[rows], wl.seeds[rows], wl.anchor_pos[rows])
    dt = (time.perf_counter() - t0) / repeats
    if ctx is not None:
        ctx.unregister() if hasattr(ctx, "unregister") else None
    return {"value": n_req * K / dt, "unit": "tokens/s", "cores": 1, "host_cpu_count": os.cpu_count(),
            "blas_threads": 1, "kind": "oracle",
            "sample": f"{n_req} of the {wl.B} requests ({'LM head, ' if lm is not None else ''}all {K} draft steps "
                      f"+ verification), run {repeats} times, "
                      f"float64 NumPy, BLAS limited to 1 thread; {dt:.1f} s per run"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=None, help="requests (default: the workload's own batch)")
    ap.add_argument("--workload", default="headline_v200064",
                    choices=("headline_v200064", "zipf_top_p_v151936", "boosted_v32000", "odd_vocab_v50017",
                             "tiny_v4096"),
                    help="seeded synthetic workload (the headline one by default; zipf_top_p_v151936 has bf16 base "
                         "logits and cache and top-p 0.95 on the target)")
    ap.add_argument("--cpu-sample", type=int, default=32, help="requests the CPU oracle baseline runs on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true", help="do not flush caches between timed steps")
    ap.add_argument("--variant", choices=("plain", "indexed", "fp64", "topk", "lmhead", "lmhead_fused"), default="plain",
                    help="plain: batch-indexed draft + verify; indexed: the same work through request-state slots, "
                         "a row mapping and per-step sample positions; fp64: the float64 Gumbel option; topk: "
                         "top-k Markov drafting (--topk candidates per row); lmhead: the draft LM head "
                         "(hidden [B*K, --hidden] x lm_head [V, --hidden]) computes the base logits, then plain; "
                         "lmhead_fused: the same as one call, step 0 inside the LM head's work-groups")
    ap.add_argument("--w2-layout", choices=("tiled", "row-major"), default="tiled",
                    help="w2 as read by the dense Markov step kernels of the plain, indexed and fp64 variants: "
                         "tiled once before the timed steps, or the row-major [V, r] matrix (the LM head and top-k "
                         "variants read it row-major)")
    ap.add_argument("--hidden", type=int, default=4096, help="hidden size of --variant lmhead")
    ap.add_argument("--topk", type=int, default=64, help="candidates per row of --variant topk")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB elementwise copy (reference dispatch for counter scaling)")
    a = ap.parse_args()
    if a.gpus != 1:
        print("bench.py runs on one GPU only: the path is measured on a single MI355X "
              "(the library has no multi-GPU code)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import markov_draft_sampling_amd as mds
    import workloads

    assert torch.cuda.is_available(), "no GPU"
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    wl = workloads.make_workload(a.workload, B=a.batch)
    B, K, V, r = wl.B, wl.K, wl.V, wl.r
    if a.variant != "plain" and (a.workload != "headline_v200064" or wl.base_dtype != "f32"):
        print("the variants run on the headline workload only", file=sys.stderr)
        sys.exit(2)
    print(f"# workload {a.workload} V={V} r={r} K={K} B={B} generated in {time.perf_counter() - t_gen:.1f}s",
          file=sys.stderr, flush=True)

    bf16_of = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    # [B, K+1, V]; the draft reads rows 0..K-1
    base = bf16_of(wl.base) if wl.base_dtype == "bf16" else torch.from_numpy(wl.base).to(dev)
    target = torch.from_numpy(wl.target).to(dev)
    top_p = None if wl.top_p is None else torch.from_numpy(wl.top_p).to(dev)
    w1 = torch.from_numpy(wl.w1.view(np.int16)).view(torch.bfloat16).to(dev)
    w2 = torch.from_numpy(wl.w2.view(np.int16)).view(torch.bfloat16).to(dev)
    anchor = torch.from_numpy(wl.anchor_tokens).to(dev)
    apos = torch.from_numpy(wl.anchor_pos).to(dev)
    temp = torch.from_numpy(wl.temperature).to(dev)
    seeds = torch.from_numpy(wl.seeds).to(dev)
    cache = torch.empty((B, K, V), dtype=torch.bfloat16 if wl.cache_dtype == "bf16" else torch.float32, device=dev)
    toks = torch.empty((B, K), dtype=torch.int32, device=dev)
    lse = torch.empty((B, K), dtype=torch.float32, device=dev)
    out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    nacc = torch.empty((B,), dtype=torch.int32, device=dev)
    ws_d = mds.new_workspace(mds.draft_topk_workspace_bytes(B, K, V, r, a.topk) if a.variant == "topk" else
                             mds.draft_workspace_bytes(B, K, V, r), dev)
    ws_v = mds.new_workspace(mds.verify_workspace_bytes(B, K, V, top_p is not None, True), dev)
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)  # 512 MiB, read to evict caches
    stream = torch.cuda.current_stream(dev)
    if a.variant in ("lmhead", "lmhead_fused"):
        t_gen = time.perf_counter()
        hid_np, lm_np = workloads.make_lm_head(B * K, V, a.hidden, seed=1)
        hidden = torch.from_numpy(hid_np.view(np.int16)).view(torch.bfloat16).to(dev)
        lm_head = torch.from_numpy(lm_np.view(np.int16)).view(torch.bfloat16).to(dev)
        print(f"# LM head inputs H={a.hidden} generated in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr,
              flush=True)
    spos = (apos[:, None] + 1 + torch.arange(K, device=dev)[None, :]).contiguous()
    tiled = a.w2_layout == "tiled" and a.variant in ("plain", "indexed", "fp64")
    w2_step, tile_ms = w2, None
    if tiled:  # once, as at weight-load time (timed on a second call into the same buffer)
        w2_step = mds.tile_markov_w2(w2)
        t_a, t_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_a.record(stream)
        mds.tile_markov_w2(w2, out=w2_step)
        t_b.record(stream)
        torch.cuda.synchronize()
        tile_ms = t_a.elapsed_time(t_b)
    if a.variant == "indexed":
        # request b lives in slot perm[b] of 2B slots; slot s owns cache row rowmap[s]
        rng = np.random.default_rng(17)
        n_slots = 2 * B
        perm = rng.permutation(n_slots)[:B].astype(np.int32)
        rowmap = rng.integers(0, B, n_slots).astype(np.int32)
        rowmap[perm] = rng.permutation(B)
        s_temp = np.full(n_slots, 0.5, np.float32)
        s_seed = rng.integers(0, 2**63, n_slots, dtype=np.int64)
        s_temp[perm], s_seed[perm] = wl.temperature, wl.seeds
        idx_b = torch.from_numpy(perm).to(dev)
        idx_bk = idx_b[:, None].expand(B, K).contiguous()
        rmap = torch.from_numpy(rowmap).to(dev)
        s_temp, s_seed = torch.from_numpy(s_temp).to(dev), torch.from_numpy(s_seed).to(dev)

    def step(events=None):
        if a.variant == "lmhead_fused":
            mds.markov_draft_loop_from_hidden(hidden, lm_head, base, w1, w2, anchor, apos, temp, seeds, cache, toks,
                                              lse, workspace=ws_d, events=events)
            if events is not None:
                launches.append(1)
            mds.rejection_verify(target, cache, toks, temp, seeds, apos, out, nacc, draft_lse=lse,
                                 top_p=top_p, workspace=ws_v)
            return
        if a.variant == "lmhead":
            mds.draft_lm_head(hidden, lm_head, base, K, events=events)
            if events is not None:
                launches.append(1)
            mds.markov_draft_loop(base, w1, w2, anchor, apos, temp, seeds, cache, toks, lse, workspace=ws_d)
            mds.rejection_verify(target, cache, toks, temp, seeds, apos, out, nacc, draft_lse=lse,
                                 top_p=top_p, workspace=ws_v)
            return
        if a.variant == "plain" and not tiled:
            if events is None:
                mds.markov_draft_loop(base, w1, w2, anchor, apos, temp, seeds, cache, toks, lse, workspace=ws_d)
            else:
                launches.append(mds.markov_draft_loop_timed(base, w1, w2, anchor, apos, temp, seeds, cache, toks, lse,
                                                            ws_d, events[0], events[1]))
            mds.rejection_verify(target, cache, toks, temp, seeds, apos, out, nacc, draft_lse=lse,
                                 top_p=top_p, workspace=ws_v)
            return
        if a.variant == "topk":
            mds.markov_draft_loop_topk(base, w1, w2, anchor, None, spos, temp, seeds, cache, toks, a.topk,
                                       draft_lse=lse, workspace=ws_d, events=events)
            if events is not None:
                launches.append(1)
            mds.rejection_verify(target, cache, toks, temp, seeds, apos, out, nacc, draft_lse=lse,
                                 top_p=top_p, workspace=ws_v)
            return
        ix = a.variant == "indexed"
        r_ = mds.markov_draft_loop_ex(base, w1, w2_step, anchor, idx_bk if ix else None, spos,
                                      s_temp if ix else temp, s_seed if ix else seeds, cache, toks,
                                      row_mapping=rmap if ix else None, draft_lse=lse,
                                      fp64_gumbel=a.variant == "fp64", workspace=ws_d, events=events, w2_tiled=tiled)
        if events is not None:
            launches.append(r_[1])
        if ix:
            mds.rejection_verify_indexed(target, cache, toks, idx_b, s_temp, s_seed, apos, out, nacc,
                                         row_mapping=rmap, draft_lse=lse, top_p=top_p, workspace=ws_v)
        else:
            mds.rejection_verify(target, cache, toks, temp, seeds, apos, out, nacc, draft_lse=lse,
                                 top_p=top_p, workspace=ws_v)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    starts, ends = [ev() for _ in range(a.steps)], [ev() for _ in range(a.steps)]
    kev = [(ev(), ev()) for _ in range(a.steps)]
    launches = []
    # the timed steps: nothing but the step between the events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        if not a.no_flush:
            flush.sum()
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    # the same steps again, the library recording events around the dominant
    # kernel's launches (those records sit between kernels, so these steps
    # are not the timed ones)
    for i in range(a.steps):
        if not a.no_flush:
            flush.sum()
        step(kev[i])
    torch.cuda.synchronize()
    draft_span_ms = np.array([b.elapsed_time(e) for b, e in kev])  # all launches of the dominant kernel in a call
    n_launch = launches[-1]

    # back to back, caches warm
    w0, w1e = ev(), ev()
    w0.record(stream)
    for _ in range(a.steps):
        step()
    w1e.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1e) / a.steps

    ms = float(np.mean(step_ms))
    tokens = B * K
    s_b = 2 if wl.base_dtype == "bf16" else 4
    s_c = 2 if wl.cache_dtype == "bf16" else 4
    draft_step_b, draft_b, verify_b = algorithmic_bytes(B, K, V, r, s_base=s_b, s_cache=s_c, top_p=top_p is not None)
    kern_avg_ms = float(np.mean(draft_span_ms)) / n_launch
    bytes_per_launch = draft_b / n_launch
    if a.variant == "topk":
        bytes_per_launch, draft_b = topk_bytes(B, K, V, r, a.topk)
    if a.variant == "lmhead":
        bytes_per_launch = lm_head_bytes(B * K, V, a.hidden)
        draft_b += bytes_per_launch
    if a.variant == "lmhead_fused":
        bytes_per_launch = draft_b = fused_draft_bytes(B, K, V, r, a.hidden, s_base=s_b, s_cache=s_c)
    achieved = bytes_per_launch / (kern_avg_ms * 1e-3) / 1e9
    step_gbps = (draft_b + verify_b) / (ms * 1e-3) / 1e9
    acc_len = float((nacc.float() + 1).mean().item())
    traffic = recorded_traffic("draft_wave_kernel_hbm_traffic_V200064_B32.md",
                               ("draft_wave.hip", "mds_device.h", "mds_internal.h"))
    if a.variant == "topk":
        traffic = recorded_traffic("topk_chunk_kernel_hbm_traffic_V200064_B32.md",
                                   ("draft_topk.hip", "mds_device.h", "mds_internal.h"))
    if a.variant == "lmhead":
        traffic = recorded_traffic("lm_head_kernel_hbm_traffic_V200064_B32.md",
                                   ("lm_head.hip", "mds_device.h", "mds_internal.h"))
    if (B != 32 or a.workload != "headline_v200064" or a.variant not in ("plain", "topk", "lmhead")
            or (a.variant == "plain" and not tiled)
            or (a.variant == "topk" and a.topk != 64) or (a.variant == "lmhead" and a.hidden != 4096)):
        traffic = None
    status = mds.workspace_status(ws_d) | mds.workspace_status(ws_v)

    res = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{a.workload}: Markov draft loop + rejection verify, V={V} r={r} K={K} B={B}, "
                               + ("bf16 base/cache, fp32 target, top-p 0.95, T~U[0.7,1.0]" if wl.top_p is not None
                                  else f"{wl.base_dtype} base, {wl.cache_dtype} cache, fp32 target") + ", bf16 w1/w2"
                               + {"plain": "", "indexed": ", request-state slots + row "
                               "mapping", "fp64": ", float64 Gumbel",
                               "topk": f", top-k Markov drafting k={a.topk}",
                               "lmhead": f", base logits from the draft LM head (H={a.hidden}, bf16)",
                               "lmhead_fused": f", the draft LM head (H={a.hidden}, bf16) with step 0 fused, "
                               "one call"}[a.variant],
                   "V": V, "r": r, "K": K, "B": B, "variant": a.variant,
                   "w2_layout": "tiled" if tiled else "row-major",
                   **({"topk": a.topk} if a.variant == "topk" else {}),
                   **({"hidden": a.hidden} if a.variant in ("lmhead", "lmhead_fused") else {}),
                   "cache_flushed_between_steps": not a.no_flush},
        "hbm": {"algorithmic_bytes_per_step": draft_b + verify_b, "achieved_GBps": step_gbps,
                "peak_GBps": HBM_PEAK_GBPS, "frac": step_gbps / HBM_PEAK_GBPS},
        "roofline": {"kernel": ("topk_chunk_kernel (base logits streamed once, -inf cache rows, chunk top-k)"
                                if a.variant == "topk" else
                                "lm_head_kernel (draft LM head, bf16 MFMA, lm_head streamed once)"
                                if a.variant == "lmhead" else
                                "the draft call from hidden states (LM head with step 0 fused, steps 1..K-1, "
                                "finalize): all its launches"
                                if a.variant == "lmhead_fused" else
                                "draft_wave_kernel (one Markov step, w2 streamed)"),
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "bytes_per_launch": bytes_per_launch, "avg_launch_us": kern_avg_ms * 1e3,
                     "launches": int(n_launch * a.steps),
                     **({"mfma_TFLOPs": 2.0 * B * K * V * a.hidden / (kern_avg_ms * 1e-3) / 1e12,
                         "mfma_peak_TFLOPs": 2500.0} if a.variant == "lmhead" else {})},
        "warm": {"ms_per_step": warm_ms, "value": tokens / (warm_ms * 1e-3)},
        "w2_tiling_ms": tile_ms,
        "step_ms_p10_p50_p90": [float(np.percentile(step_ms, q)) for q in (10, 50, 90)],
        "draft_kernels_ms": float(np.mean(draft_span_ms)),
        "acceptance_length": acc_len,
        "status_word": status,
        "timed_wall_s": wall,
    }
    if a.copy_calibration:
        # an elementwise kernel (a same-size tensor copy would go to a DMA
        # engine, which the shader counters do not see)
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            flush.sum()
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = {"read": src.numel() * 4, "write": dst.numel() * 4}
    if not a.no_cpu_baseline:
        kw = {"topk": a.topk} if a.variant == "topk" else ({"fp64_gumbel": True} if a.variant == "fp64" else {})
        if a.variant in ("lmhead", "lmhead_fused"):
            # the LM head dominates the oracle's time: at most 16 requests, once
            res["cpu_baseline"] = cpu_baseline(wl, min(a.cpu_sample, 16), repeats=1, lm=(hid_np, lm_np))
        else:
            res["cpu_baseline"] = cpu_baseline(wl, min(a.cpu_sample, B), **kw)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
