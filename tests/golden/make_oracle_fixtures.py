"""Write oracle regression fixtures (calls only oracle/ and the generator).

    python tests/golden/make_oracle_fixtures.py

Output: tests/golden/oracle_tiny_1k.json with the 1K tiny workload's kept-block
counts, density and a few block scores, so that a later change in the
oracle's arithmetic shows up as a diff.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from rr_workloads import generate, get_config  # noqa: E402


def main():
    w = get_config(0)
    g = generate(w)
    A = oracle.block_scores(g["q"], g["k"], w.B, w.S)
    keep, cnt, _ = oracle.select(A, w.tau)
    out = {
        "workload": w.name, "seed": w.seed, "B": w.B, "S": w.S, "tau": w.tau,
        "counts": cnt.tolist(),
        "density": float(keep.sum()) / (w.Hq * w.nb * (w.nb + 1) / 2),
        "A_head0_row7": A[0, 7].tolist(),
        "A_head5_row3": A[5, 3, :4].tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_1k.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
