"""The stored exception counts (tests/golden/flag_counts.json) still follow from the
oracle: recomputed here for the cases the CPU finishes in seconds (c2 at each
temperature, the edge and mask cases, every fourth random configuration).  The
full-size cases are recomputed by the GPU parity tests, which run the oracle on them
anyway."""
import json
import os

import pytest

import parity_cases as pc

with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "flag_counts.json")) as fh:
    STORED = json.load(fh)["cases"]

CASES = ([("full", c[0]) for c in pc.FULL_CASES if c[1] == "c2"] + [("edge", c[0]) for c in pc.EDGE_CASES] +
         [("mask", c[0]) for c in pc.MASK_CASES] + [("random", i) for i in range(0, pc.N_RANDOM, 4)])


@pytest.mark.parametrize("kind,key", CASES, ids=[str(c[1]) for c in CASES])
def test_stored_counts(kind, key):
    c = {"full": pc.full_case, "edge": pc.edge_case, "mask": pc.mask_case, "random": pc.random_case}[kind](key)
    got = pc.exception_counts(c.oracle_round())
    want = {k: v for k, v in STORED[c.label].items() if k != "sequences"}
    assert got == want, (c.label, got, want)
    assert STORED[c.label]["sequences"] == c.B
