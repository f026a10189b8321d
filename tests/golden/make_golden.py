"""Writes the stored expected values under tests/golden/ from the fp64 oracle only.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402

# (K, B_f, r) of the five workloads: a single sequence at V=32000, the temperature
# sweep at V=32000, the headline B=64 V=128256, the high-temperature B=256 V=128256
# and the large-batch B=512 V=151936 case.
WORKLOAD_FANOUT = [(4, 16, 0.7), (5, 32, 0.6), (8, 64, 0.7), (6, 96, 0.8), (4, 32, 0.5)]


def main():
    rows = []
    for K, Bf, r in WORKLOAD_FANOUT:
        F, gap = oracle.fanout(K, Bf, r)
        rows.append({"K": K, "Bf": Bf, "r": r, "F": F.tolist(), "min_remainder_gap": gap})
    out = {
        "source": "written by tests/golden/make_golden.py from the fp64 oracle (oracle.fanout)",
        "rule": "geometric fan-out F_k proportional to r^k under budget B_f, largest remainder",
        "rows": rows,
    }
    with open(os.path.join(HERE, "fanout_workloads.json"), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")


if __name__ == "__main__":
    main()
