"""The oracle still reproduces the stored outputs that tests/golden/make_golden.py
wrote from it on the tiny workload (a lock against unjustified changes)."""
import json
import os

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_reproduces_golden():
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "golden", "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    with open(os.path.join(HERE, "golden", "tiny_v4096_oracle.json")) as f:
        want = json.load(f)
    got = mg.compute()
    for k in ("draft_tokens", "out_tokens", "num_accepted", "cache_sha256", "cache_first8"):
        assert got[k] == want[k], k
    for k in ("draft_margin", "draft_lse"):
        flat_g = [x for row in got[k] for x in row]
        flat_w = [x for row in want[k] for x in row]
        assert flat_g == pytest.approx(flat_w, abs=1e-8), k
