"""Writes tests/golden/flag_counts.json: the oracle's integer-parity exception counts
(sequences flagged E1..E5) on the parity inputs of tests/parity_cases.py -- the
workloads at full size, the c1 rounds, the edge cases, the masked vocabularies and the
random configurations.  Calls only oracle/ (and the seeded input generators).  The
GPU parity tests compare every sequence the oracle leaves unflagged and check that the
flagged count equals the stored one.

Run from the repository root:  python tests/golden/make_flag_counts.py
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, os.path.dirname(HERE))

import parity_cases as pc  # noqa: E402


def _count(c, out):
    cnt = pc.exception_counts(c.oracle_round())
    cnt["sequences"] = c.B
    out[c.label] = cnt
    return cnt


def main():
    cases = {}
    for label, *_ in pc.FULL_CASES:
        t = time.time()
        print("%-14s %s  (%.1f s)" % (label, _count(pc.full_case(label), cases), time.time() - t), flush=True)
    tot = {"sequences": pc.C1_ROUNDS}
    for rnd in range(pc.C1_ROUNDS):
        cnt = pc.exception_counts(pc.c1_case(rnd).oracle_round())
        for k, v in cnt.items():
            tot[k] = tot.get(k, 0) + v
    cases["c1 rounds"] = tot
    print("c1 rounds      %s" % tot, flush=True)
    for label, *_ in pc.EDGE_CASES:
        print("%-20s %s" % (label, _count(pc.edge_case(label), cases)), flush=True)
    for label, *_ in pc.MASK_CASES:
        print("%-20s %s" % (label, _count(pc.mask_case(label), cases)), flush=True)
    rsum = {}
    for i in range(pc.N_RANDOM):
        c = pc.random_case(i)
        cnt = _count(c, cases)
        for k, v in cnt.items():
            rsum[k] = rsum.get(k, 0) + v
    print("random configs total %s" % rsum, flush=True)
    out = {"source": "written by tests/golden/make_flag_counts.py from the fp64 oracle",
           "rule": "a sequence is flagged when the oracle sets any of E1..E5 for it; flagged sequences "
                   "are left out of the integer comparison",
           "cases": cases}
    with open(os.path.join(HERE, "flag_counts.json"), "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
        fh.write("\n")


if __name__ == "__main__":
    main()
