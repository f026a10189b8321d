"""Pins of the oracle's n-gram fallback speculator (prompt lookup over the
sequence's own context) against hand-worked cases, Python's own substring search
(str.rfind), the closed form of the periodic copy and numpy's Philox.  CPU only."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _philox_token(seed, rnd, b, j, V, purpose):
    bg = np.random.Philox(key=np.array([seed, purpose], dtype=np.uint64),
                          counter=np.array([rnd - 1, b, j, 0], dtype=np.uint64))
    return ((int(bg.random_raw(1)[0]) >> 32) * V) >> 32


def test_ngram_hand_worked_cases(orc):
    """Cases worked by hand (tests/golden/ngram_cases.json, each with its reason)."""
    with open(os.path.join(GOLDEN, "ngram_cases.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        t, n, e, err = orc.ngram_fallback(c["K"], 100, np.array([c["hist"]]), [len(c["hist"])],
                                          np.array([c["draft"]]), [c["k"]], [c["bonus"]], None,
                                          c["n_min"], c["n_max"], 1, 2)
        assert t[0].tolist() == c["tokens"], c["why"]
        assert (n[0], e[0], err[0]) == (c["n"], c["e"], 0), c["why"]


def _rfind_match(ctx, n_min, n_max):
    """(n, e) by Python's substring search: tokens become one code point each; the
    last occurrence of the suffix n-gram inside ctx[:-1] (so that it ends at L-2 at
    the latest), longest n first."""
    s = "".join(chr(x) for x in ctx)
    L = len(s)
    for n in range(min(n_max, L - 1), n_min - 1, -1):
        start = s.rfind(s[L - n:], 0, L - 1)
        if start >= 0:
            return n, start + n - 1
    return 0, -1


def test_ngram_matches_substring_search(orc):
    """Random contexts over 2..4 symbols (many repeats), ragged histories, every
    k in [0, K]: (n, e) equals str.rfind's; the proposal is c[e + 1 + (j mod P)]
    with period P = L - 1 - e (the closed form of copying on over one's own
    output); with no match the tokens are numpy Philox's uniform words."""
    rng = np.random.default_rng(31)
    seed, rnd, V = 77, 5, 4
    for trial in range(60):
        B, K = 24, int(rng.integers(1, 7))
        ld = int(rng.integers(1, 40))
        alphabet = int(rng.integers(2, 5))
        hist = rng.integers(0, alphabet, (B, ld)).astype(np.int32)
        hl = rng.integers(0, ld + 1, B).astype(np.int32)
        draft = rng.integers(0, alphabet, (B, K)).astype(np.int32)
        acc = rng.integers(0, K + 1, B).astype(np.int32)
        bonus = rng.integers(0, alphabet, B).astype(np.int32)
        n_min = int(rng.integers(1, 4))
        n_max = int(rng.integers(n_min, 8))
        t, n, e, err = orc.ngram_fallback(K, V, hist, hl, draft, acc, bonus, None, n_min, n_max, seed, rnd,
                                          b_base=trial * B)
        assert np.all(err == 0)
        for b in range(B):
            ctx = hist[b, :hl[b]].tolist() + draft[b, :acc[b]].tolist() + [int(bonus[b])]
            ne = _rfind_match(ctx, n_min, n_max)
            assert (n[b], e[b]) == ne, (ctx, n_min, n_max)
            if ne[0]:
                P = len(ctx) - 1 - ne[1]
                assert t[b].tolist() == [ctx[ne[1] + 1 + (j % P)] for j in range(K)]
            else:
                assert t[b].tolist() == [_philox_token(seed, rnd, trial * B + b, j, V, orc.PURPOSE_FALLBACK)
                                         for j in range(K)]


def test_ngram_no_match_equals_uniform_fallback(orc):
    """With no repeated n-gram (distinct tokens) the proposal is exactly the cache
    lookup's uniform fallback draft of the same (seed, round, b)."""
    B, K, V = 16, 5, 1000
    hist = np.arange(B * 30, dtype=np.int32).reshape(B, 30)
    hl = np.full(B, 30, np.int32)
    acc = np.zeros(B, np.int32)
    bonus = np.arange(B, dtype=np.int32) + 5000
    t, n, e, err = orc.ngram_fallback(K, V, hist, hl, np.zeros((B, K)), acc, bonus, None, 1, 4, 9, 3)
    assert np.all(n == 0) and np.all(e == -1)
    F = np.array([1, 0, 0, 0, 0, 0], dtype=np.int32)
    ids = np.full((B, 1), -7, np.int32)
    _, _, fb, _ = orc.cache_lookup(K, V, F, ids, acc, bonus, 1, 9, 3)
    assert np.array_equal(t, fb)


def test_ngram_hits_invalid_and_next_draft(orc):
    """A hit gets tokens -1 and keeps its next draft; an out-of-range k or history
    length is an error bit with tokens -1 (and next draft -1); misses get the
    proposal in both outputs."""
    K, V = 3, 50
    hist = np.array([[1, 2, 3, 1, 2], [1, 2, 3, 1, 2], [1, 2, 3, 1, 2], [1, 2, 3, 1, 2]], np.int32)
    hl = np.array([5, 5, 5, 6], np.int32)
    acc = np.array([0, 0, 4, 0], np.int32)
    bonus = np.array([3, 3, 3, 3], np.int32)
    hit = np.array([0, 1, 0, 0], np.uint8)
    nd = np.full((4, K), 42, np.int32)
    t, n, e, err = orc.ngram_fallback(K, V, hist, hl, np.zeros((4, K)), acc, bonus, hit, 1, 3, 1, 1,
                                      next_draft=nd)
    # context [1,2,3,1,2,3]: [1,2,3] ends at e=2; period 3
    assert t[0].tolist() == [1, 2, 3] and (n[0], e[0]) == (3, 2) and nd[0].tolist() == [1, 2, 3]
    assert t[1].tolist() == [-1] * K and nd[1].tolist() == [42] * K and (n[1], e[1]) == (0, -1)
    assert t[2].tolist() == [-1] * K and err[2] == orc.ERR_LEN_RANGE and nd[2].tolist() == [-1] * K
    assert t[3].tolist() == [-1] * K and err[3] == orc.ERR_HIST_RANGE
    assert err[0] == 0 and err[1] == 0


def test_ngram_mutations_fail_a_pin(orc):
    """The substring-search pin separates the reading from its plausible slips:
    the earliest instead of the latest occurrence, the shortest instead of the
    longest n, and an occurrence allowed to end at the last position."""
    rng = np.random.default_rng(5)
    ctxs = [rng.integers(0, 3, int(rng.integers(3, 30))).tolist() for _ in range(300)]

    def earliest(ctx, n_min, n_max):
        s = "".join(chr(x) for x in ctx)
        for n in range(min(n_max, len(s) - 1), n_min - 1, -1):
            start = s.find(s[len(s) - n:], 0, len(s) - 1)
            if start >= 0:
                return n, start + n - 1
        return 0, -1

    def shortest(ctx, n_min, n_max):
        s = "".join(chr(x) for x in ctx)
        for n in range(n_min, min(n_max, len(s) - 1) + 1):
            start = s.rfind(s[len(s) - n:], 0, len(s) - 1)
            if start >= 0:
                return n, start + n - 1
        return 0, -1

    def self_match(ctx, n_min, n_max):
        s = "".join(chr(x) for x in ctx)
        for n in range(min(n_max, len(s)), n_min - 1, -1):
            start = s.rfind(s[len(s) - n:])
            if start >= 0:
                return n, start + n - 1
        return 0, -1

    for wrong in (earliest, shortest, self_match):
        assert any(wrong(c, 1, 4) != _rfind_match(c, 1, 4) for c in ctxs)


def test_planted_contexts_match_at_the_plant(orc):
    """The bench's planted histories (workloads.plant_contexts): every planted sequence
    matches with n = n_max, at the plant or later, and the unplanted rows keep their
    original histories."""
    from lossless_rejection_sampling_ssd_amd.workloads import make_histories, plant_contexts
    B, L, V, K, n = 12, 512, 1000, 4, 5
    hist, lens = make_histories(B, L, V, seed=9)
    rng = np.random.default_rng(3)
    draft = rng.integers(0, V, (B, K)).astype(np.int32)
    k = rng.integers(0, K + 1, B).astype(np.int32)
    bonus = rng.integers(0, V, B).astype(np.int32)
    rows = np.arange(0, B, 2)
    h2 = plant_contexts(hist, lens, draft, k, bonus, n, rows)
    _, mn, me, err = orc.ngram_fallback(K, V, h2, lens, draft, k, bonus, None, 2, n, 1, 1)
    assert not err.any()
    for b in range(B):
        if b in rows:
            assert mn[b] == n and me[b] >= lens[b] // 2 + n - 1, b
        else:
            assert (h2[b] == hist[b]).all()
