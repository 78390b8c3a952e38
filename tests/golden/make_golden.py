"""Writes tests/golden/tiny_v4096_oracle.json from the CPU oracle only.

The file locks the oracle's outputs on the tiny workload (V=4096, r=64, K=3,
B=1) so that any later change to the oracle's arithmetic shows up as a
failing test and has to be justified. Run from the repository root:
    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def compute():
    wl = workloads.make_workload("tiny_v4096")
    d = oracle.draft_loop(wl.draft_base, wl.base_dtype, wl.w1, wl.w2, wl.anchor_tokens, wl.anchor_pos, wl.seeds,
                          wl.temperature, wl.cache_dtype)
    v = oracle.verify(wl.target, d["cache"], wl.cache_dtype, d["tokens"], wl.temperature, wl.top_p, wl.seeds,
                      wl.anchor_pos)
    return {
        "workload": "tiny V=4096 r=64 K=3 B=1, master seed 0",
        "draft_tokens": d["tokens"].tolist(),
        "draft_margin": [[round(float(x), 9) for x in row] for row in d["margin"]],
        "draft_lse": [[round(float(x), 9) for x in row] for row in d["lse"]],
        "cache_sha256": hashlib.sha256(np.ascontiguousarray(d["cache"]).tobytes()).hexdigest(),
        "cache_first8": [float(x) for x in d["cache"][0, 0, :8]],
        "out_tokens": v["out_tokens"].tolist(),
        "num_accepted": v["num_accepted"].tolist(),
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_v4096_oracle.json")
    with open(out, "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", out)
