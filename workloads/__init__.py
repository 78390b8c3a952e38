"""Seeded synthetic inputs for the Markov draft loop and rejection verification.

This module only draws inputs. It holds none of the method's arithmetic: no
projection, no noise hash, no sampling, no softmax. Both the CPU oracle
(``oracle/``) and the GPU path consume what it returns, so neither depends on
the other.

The five workloads mirror the shapes and value distributions of the serving
setups on the pages (DSpark drafts of a 200k-vocabulary model with K=7 draft
steps and 1..128 concurrent requests, PR "vocab-parallel DSpark Markov
sampling", sections Part 1 and Claims). The pages measure with trained models
on GSM8K / SPEED-Bench / agentic prompts; those only shape the logits, so
seeded Gaussian/Zipf logits of the same shapes stand in for them.

Every workload carries K+1 base rows per request: rows 0..K-1 are the draft
base logits of the K Markov steps and row K exists only so that the target
for the bonus position can be derived the same way (target row j = base row j
+ Gaussian noise).

Per-request values come from a generator keyed by (master seed, request index),
so the first B requests of a workload are the same at every B: a workload at
B=8 is a prefix of the one at B=128.
"""
from __future__ import annotations

import dataclasses
import functools

import numpy as np

__all__ = ["WORKLOADS", "Workload", "make_workload", "bf16_bits", "bf16_bits_to_f32", "HEADLINE_BATCHES",
           "ODD_VOCAB_BATCHES", "make_lm_head"]

HEADLINE_BATCHES = (1, 8, 32, 128)
ODD_VOCAB_BATCHES = (1, 2, 3, 4, 5, 7, 8, 16, 31, 32, 33, 64, 96, 127, 128)


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    desc: str
    V: int
    r: int
    K: int
    B: int  # default batch
    base_dtype: str  # "f32" | "bf16"
    cache_dtype: str  # "f32" | "bf16"
    base_std: float
    w_std: float
    target_std: float
    master: int  # seed material of the generators
    top_p: float | None = None
    boost: bool = False  # 5% of the columns of each request raised by 6
    zipf: bool = False  # Zipf-shaped offsets (rank^-1.1 scaled to +10) on the base logits
    temp: str = "one"  # "one", "fixed" (T = 1, seed 0, position 100), "u0.6-1.2", "u0.7-1.0", "greedy_quarter"
    planted: bool = False  # exact ties between blocks, NaN columns, zero w2 rows


WORKLOADS: dict[str, WorkloadSpec] = {
    "tiny_v4096": WorkloadSpec("tiny V=4096 r=64 K=3 B=1", 4096, 64, 3, 1, "f32", "f32", 3.0, 0.05, 0.5, 0,
                               temp="fixed"),
    "boosted_v32000": WorkloadSpec("V=32000 r=128 K=5 B=8 boosted", 32000, 128, 5, 8, "f32", "f32", 3.0, 0.02, 1.0,
                                   2, boost=True, temp="u0.6-1.2"),
    "zipf_top_p_v151936": WorkloadSpec("V=151936 r=256 K=7 B=32 bf16 zipf top-p", 151936, 256, 7, 32, "bf16", "bf16",
                                       4.0, 0.02, 0.8, 3, top_p=0.95, zipf=True, temp="u0.7-1.0"),
    "headline_v200064": WorkloadSpec("V=200064 r=256 K=7 fp32", 200064, 256, 7, 32, "f32", "f32", 3.0, 0.02, 1.0, 4),
    "odd_vocab_v50017": WorkloadSpec("odd vocabulary V=50017 r=192 K=7", 50017, 192, 7, 32, "f32", "f32", 3.0, 0.05,
                                     0.5, 5, temp="greedy_quarter", planted=True),
}


@dataclasses.dataclass
class Workload:
    name: str
    V: int
    r: int
    K: int
    B: int
    base_dtype: str
    cache_dtype: str
    base: np.ndarray  # [B, K+1, V] float32, or uint16 bf16 bit patterns when base_dtype == "bf16"
    w1: np.ndarray  # [V, r] uint16 bf16 bit patterns
    w2: np.ndarray  # [V, r] uint16 bf16 bit patterns
    anchor_tokens: np.ndarray  # [B] int32, the previous token of draft step 0
    anchor_pos: np.ndarray  # [B] int64, position P0 of the anchor token
    seeds: np.ndarray  # [B] int64 per-request sampling seed
    temperature: np.ndarray  # [B] float32, 0 marks a greedy request
    target: np.ndarray  # [B*(K+1), V] float32, row b*(K+1)+j
    top_p: np.ndarray | None  # [B] float32 or None
    nan_rows: list = dataclasses.field(default_factory=list)  # [(b, k, cols)] draft base rows holding NaN
    tie_cols: tuple = ()  # columns whose w2 rows are zero (bias exactly 0)
    tie_requests: tuple = ()  # greedy requests whose tie columns were set to row max + 5

    @property
    def draft_base(self) -> np.ndarray:
        """[B, K, V] view of the draft rows (row K is the bonus row's base)."""
        return self.base[:, : self.K]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even, via torch's conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


@functools.lru_cache(maxsize=4)
def _weights(wname: str):
    spec = WORKLOADS[wname]
    rng = np.random.default_rng([spec.master, 0])
    w1 = rng.standard_normal((spec.V, spec.r), dtype=np.float32) * np.float32(spec.w_std)
    w2 = rng.standard_normal((spec.V, spec.r), dtype=np.float32) * np.float32(spec.w_std)
    tie_cols: tuple = ()
    if spec.planted:
        # Four columns in distinct 1024-column blocks plus a second column in
        # the first one's block; their w2 rows are zero, so the Markov bias
        # there is exactly 0 whatever the previous token.
        tie_cols = (1029, 9000, 23555, 50016, 1500)
        w2[list(tie_cols)] = 0.0
    w1b, w2b = bf16_bits(w1), bf16_bits(w2)
    w1b.setflags(write=False)
    w2b.setflags(write=False)
    return w1b, w2b, tie_cols


@functools.lru_cache(maxsize=2)
def _zipf_offsets(wname: str) -> np.ndarray:
    spec = WORKLOADS[wname]
    rng = np.random.default_rng([spec.master, 2])
    perm = rng.permutation(spec.V)
    off = np.empty(spec.V, dtype=np.float32)
    off[perm] = (10.0 * np.arange(1, spec.V + 1, dtype=np.float64) ** -1.1).astype(np.float32)
    return off


def _request(wname: str, b: int):
    """Per-request draws: base rows, target rows, temperature, seed, position, anchor."""
    spec = WORKLOADS[wname]
    V, K = spec.V, spec.K
    rng = np.random.default_rng([spec.master, 1, b])
    base = rng.standard_normal((K + 1, V), dtype=np.float32) * np.float32(spec.base_std)
    if spec.boost:
        boosted = rng.choice(V, size=V // 20, replace=False)
        base[:, boosted] += np.float32(6.0)
    if spec.zipf:
        base += _zipf_offsets(wname)[None, :]
    noise = rng.standard_normal((K + 1, V), dtype=np.float32) * np.float32(spec.target_std)
    if spec.temp == "fixed":
        temp, seed, pos = 1.0, 0, 100
    else:
        seed = int(rng.integers(0, 2**63, dtype=np.int64))
        pos = int(rng.integers(1, 2**20))
        if spec.temp == "u0.6-1.2":
            temp = float(rng.uniform(0.6, 1.2))
        elif spec.temp == "u0.7-1.0":
            temp = float(rng.uniform(0.7, 1.0))
        elif spec.temp == "greedy_quarter":
            # a quarter of the requests are greedy (b = 3, 7, 11, ...), so
            # every batch of four or more holds one
            temp = 0.0 if b % 4 == 3 else 1.0
        else:
            temp = 1.0
    anchor = int(rng.integers(0, V))
    return base, noise, np.float32(temp), seed, pos, anchor, rng


def make_workload(wname: str, B: int | None = None) -> Workload:
    """Build the named workload (a key of WORKLOADS) at batch ``B`` (default: its own)."""
    spec = WORKLOADS[wname]
    B = spec.B if B is None else int(B)
    if B < 1:
        raise ValueError("B must be >= 1")
    V, K = spec.V, spec.K
    w1, w2, tie_cols = _weights(wname)
    base_bits = spec.base_dtype == "bf16"
    base = np.empty((B, K + 1, V), dtype=np.uint16 if base_bits else np.float32)
    target = np.empty((B * (K + 1), V), dtype=np.float32)
    temps = np.empty(B, np.float32)
    seeds = np.empty(B, np.int64)
    pos = np.empty(B, np.int64)
    anchors = np.empty(B, np.int32)
    nan_rows = []
    tie_requests = []
    for b in range(B):
        rb, noise, t, s, p, a, rng = _request(wname, b)
        if base_bits:
            bits = bf16_bits(rb)
            base[b] = bits
            rb_f = bf16_bits_to_f32(bits)
        else:
            base[b] = rb
            rb_f = rb
        target[b * (K + 1):(b + 1) * (K + 1)] = rb_f + noise
        temps[b], seeds[b], pos[b], anchors[b] = t, s, p, a
        if spec.planted:
            # exact ties in every other greedy request: the tie columns carry
            # the row maximum + 5 in every base row and every target row
            if t == 0.0 and (b // 4) % 2 == 0:
                tie_requests.append(b)
                for j in range(K + 1):
                    base[b, j, list(tie_cols)] = base[b, j].max() + np.float32(5.0)
                    row = target[b * (K + 1) + j]
                    row[list(tie_cols)] = row.max() + np.float32(5.0)
            # NaN columns in 2% of the draft rows, injected after the target
            # was derived; request 6 always has one so batches of 8+ do
            for k in range(K):
                if (b == 6 and k == 2) or rng.uniform() < 0.02:
                    cols = np.sort(rng.choice(V, size=int(rng.integers(1, 4)), replace=False))
                    base[b, k, cols] = np.nan
                    nan_rows.append((b, k, tuple(int(c) for c in cols)))
    top_p = None if spec.top_p is None else np.full(B, spec.top_p, np.float32)
    return Workload(name=wname, V=V, r=spec.r, K=K, B=B, base_dtype=spec.base_dtype,
                    cache_dtype=spec.cache_dtype, base=base, w1=w1, w2=w2, anchor_tokens=anchors,
                    anchor_pos=pos, seeds=seeds, temperature=temps, target=target, top_p=top_p,
                    nan_rows=nan_rows, tie_cols=tie_cols, tie_requests=tuple(tie_requests))


def make_custom(V: int, r: int, K: int, B: int, *, seed: int = 0, base_std: float = 3.0, w_std: float = 0.05,
                target_std: float = 0.5, temperature: float = 1.0, base_dtype: str = "f32",
                cache_dtype: str = "f32", top_p: float | None = None) -> Workload:
    """Small seeded workload of arbitrary shape (tile/tail coverage in tests)."""
    rng = np.random.default_rng([seed, 7, V, r, K, B])
    w1 = bf16_bits(rng.standard_normal((V, r), dtype=np.float32) * np.float32(w_std))
    w2 = bf16_bits(rng.standard_normal((V, r), dtype=np.float32) * np.float32(w_std))
    rb = rng.standard_normal((B, K + 1, V), dtype=np.float32) * np.float32(base_std)
    if base_dtype == "bf16":
        base = bf16_bits(rb)
        rb = bf16_bits_to_f32(base)
    else:
        base = rb
    target = (rb + rng.standard_normal((B, K + 1, V), dtype=np.float32) * np.float32(target_std)).reshape(
        B * (K + 1), V)
    return Workload(name=f"custom V={V} r={r} K={K} B={B}", V=V, r=r, K=K, B=B, base_dtype=base_dtype,
                    cache_dtype=cache_dtype, base=base, w1=w1, w2=w2,
                    anchor_tokens=rng.integers(0, V, size=B).astype(np.int32),
                    anchor_pos=rng.integers(1, 2**20, size=B).astype(np.int64),
                    seeds=rng.integers(0, 2**63, size=B, dtype=np.int64),
                    temperature=np.full(B, temperature, np.float32), target=target,
                    top_p=None if top_p is None else np.full(B, top_p, np.float32))


def make_lm_head(rows: int, V: int, H: int, *, seed: int = 0, logit_std: float = 3.0):
    """Seeded draft LM-head inputs: hidden [rows, H] and lm_head [V, H] as bf16 bit patterns.

    hidden ~ N(0, 1) and lm_head ~ N(0, logit_std^2 / H), so the logits
    hidden @ lm_head^T are ~N(0, logit_std^2) like the workloads' base logits.
    Generated in row chunks to bound host memory.
    """
    rng = np.random.default_rng([seed, 11, rows, V, H])
    hidden = bf16_bits(rng.standard_normal((rows, H), dtype=np.float32))
    lm = np.empty((V, H), np.uint16)
    scale = np.float32(logit_std / np.sqrt(H))
    step = max(1, (1 << 24) // H)
    for v0 in range(0, V, step):
        v1 = min(V, v0 + step)
        lm[v0:v1] = bf16_bits(rng.standard_normal((v1 - v0, H), dtype=np.float32) * scale)
    return hidden, lm
