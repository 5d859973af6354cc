"""Write oracle_small.json: oracle sums for small seeded clips (calls only the oracle and synth).

Run from the repository root:  python tests/golden/make_oracle_golden.py
The stored sums guard the oracle against unintended changes; a deliberate change to its arithmetic
regenerates this file in the same commit, naming the passage or reading that justifies it.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

CASES = [
    ("uniform", 3, 3, 8, 3, 1),
    ("uniform", 7, 5, 10, 3, 2),
    ("checker", 17, 9, 8, 2, 3),
    ("extreme", 33, 18, 10, 3, 4),
    ("impulse", 64, 20, 8, 4, 5),
]

# motion v2 (the filter of the frame difference) at 8, 10, 12 and 16 bits
V2_CASES = [
    ("uniform", 9, 7, 8, 3, 11),
    ("extreme", 17, 9, 10, 3, 12),
    ("checker", 12, 10, 12, 3, 13),
    ("uniform", 21, 11, 16, 3, 14),
    ("extreme", 8, 6, 16, 3, 15),
]


def main():
    out = {"cases": []}
    for kind, w, h, bpc, f, seed in CASES:
        c = synth.random_clip(w, h, bpc, f, seed, kind)
        sums, hm = oracle.clip(c.ref, c.dist, bpc)
        out["cases"].append({"kind": kind, "width": w, "height": h, "bpc": bpc, "frames": f,
                             "seed": seed, "sums": [[int(v) for v in r] for r in sums],
                             "has_motion": [int(v) for v in hm]})
    out["v2_cases"] = []
    for kind, w, h, bpc, f, seed in V2_CASES:
        c = synth.random_clip(w, h, bpc, f, seed, kind)
        sums, hm = oracle.clip_v2(c.ref, c.dist, bpc)
        out["v2_cases"].append({"kind": kind, "width": w, "height": h, "bpc": bpc, "frames": f,
                                "seed": seed, "sums": [[int(v) for v in r] for r in sums],
                                "has_motion": [int(v) for v in hm]})
    c = synth.make_clip("c1", 3)
    sums, hm = oracle.clip(c.ref, c.dist, 8)
    out["c1_first3"] = {"sums": [[int(v) for v in r] for r in sums],
                        "has_motion": [int(v) for v in hm]}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
