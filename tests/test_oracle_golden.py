"""The oracle still produces the sums stored by tests/golden/make_oracle_golden.py."""
import json
import os

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_stored_sums():
    with open(os.path.join(HERE, "golden", "oracle_small.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        c = synth.random_clip(case["width"], case["height"], case["bpc"], case["frames"],
                              case["seed"], case["kind"])
        sums, hm = oracle.clip(c.ref, c.dist, case["bpc"])
        assert [[int(v) for v in r] for r in sums] == case["sums"], case["kind"]
        assert [int(v) for v in hm] == case["has_motion"]
    c = synth.make_clip("c1", 3)
    sums, hm = oracle.clip(c.ref, c.dist, 8)
    assert [[int(v) for v in r] for r in sums] == g["c1_first3"]["sums"]


def test_oracle_v2_matches_stored_sums():
    with open(os.path.join(HERE, "golden", "oracle_small.json")) as f:
        g = json.load(f)
    assert len(g["v2_cases"]) >= 4
    for case in g["v2_cases"]:
        c = synth.random_clip(case["width"], case["height"], case["bpc"], case["frames"],
                              case["seed"], case["kind"])
        sums, hm = oracle.clip_v2(c.ref, c.dist, case["bpc"])
        assert [[int(v) for v in r] for r in sums] == case["sums"], (case["kind"], case["bpc"])
        assert [int(v) for v in hm] == case["has_motion"]
