"""Pins of the oracle's integer-parity exception flags (E1, E2, E3, E5).

The flags name the sequences whose integer outputs the GPU comparison leaves out, so
a flag that fires too often would hollow out every parity test and one that never
fires would let rounding decide a test.  Each case below is built by hand on a two-
or three-token vocabulary so that the quantity a flag tests lands just inside or just
outside its band.  The quantity is recomputed here from the fp32 logits in numpy
fp64 and the uniforms come from numpy's own Philox4x64-10 (not from the oracle), so
these pins do not restate the oracle's arithmetic.

Bands (the parity rule of the round):
  E1  |u_i - p_i(d_i)/q'_i(d_i)| < 1e-5 at a tested position i <= min(k, K-1);
  E2  u within CDF_TIE_EPS of one of the two normalised CDF steps around the
      sampled id (draft sampler and bonus);
  E3  residual mass Z_r < 1e-5 after a rejection (k < K);
  E5  a tested p_i(d_i) or q'_i(d_i) below 1e-30 from a finite logit.
A final test compiles mutated copies of ssd_oracle.c (a wrong band, the
min(1, ratio) slip, flags after the first rejection, the -inf exemption dropped,
one side of the CDF gap dropped) and checks that each one fails a pin here.
"""
import os

import numpy as np
import pytest

SEED = 0x7E57
ACCEPT, BONUS, DRAFT = 0, 1, 2


# --------------------------------------------------------------------------- helpers
def u_np(seed, rnd, purpose, b, i):
    """U(seed, rnd, b, i, purpose) from numpy's Philox4x64-10: the first output word
    of counter (rnd, b, i, 0) under key (seed, purpose), top 24 bits times 2^-24
    (numpy increments the counter before producing a block)."""
    assert rnd >= 1
    g = np.random.Philox(key=np.array([seed, purpose], np.uint64),
                         counter=np.array([rnd - 1, b, i, 0], np.uint64))
    return (int(g.random_raw(1)[0]) >> 40) / 2.0**24


def us_over_rounds(seed, purpose, b, i, r0, n):
    """u for rounds r0 .. r0+n-1 at (b, i): consecutive numpy Philox blocks advance
    counter word 0, which is the round."""
    g = np.random.Philox(key=np.array([seed, purpose], np.uint64),
                         counter=np.array([r0 - 1, b, i, 0], np.uint64))
    w0 = g.random_raw(4 * n)[0::4]
    return (w0 >> np.uint64(40)).astype(np.float64) / 2.0**24


def logit_for(t):
    """fp32 logit z with sigmoid(z) ~ t (softmax of [z, 0] puts t on id 0)."""
    return np.float32(np.log(t) - np.log1p(-t))


def p0_of(z):
    """id-0 probability of softmax([z, 0]) in fp64 from the fp32 logit."""
    z = float(np.float32(z))
    return 1.0 / (1.0 + np.exp(-z)) if np.isfinite(z) else (1.0 if z > 0 else 0.0)


def softmax64(row):
    z = np.asarray(row, np.float32).astype(np.float64)
    m = z.max()
    e = np.exp(z - m)
    return e / e.sum()


def find_round(lo, hi, purpose, bs, i=0, r0=1, n=200000):
    """The first round r >= r0 whose uniforms at (b, i) lie in (lo, hi) for every b
    in bs."""
    ok = np.ones(n, bool)
    for b in bs:
        u = us_over_rounds(SEED, purpose, b, i, r0, n)
        ok &= (u > lo) & (u < hi)
    hits = np.nonzero(ok)[0]
    assert hits.size, "no round found"
    return r0 + int(hits[0])


# --------------------------------------------------------------------------- E1, E5: verify
# One sequence per case, K = 2, V = 2, draft tokens d = (0, 0).  Row i of the draft is
# [a_i, 0] and of the target [c_i, 0]; with F = (0, 0, 0) q' = q, so the ratio at
# position i is sigmoid(c_i) / sigmoid(a_i).
E1_DELTAS = [(+5e-6, True), (-5e-6, True), (+9e-6, True), (-9e-6, True),
             (+1.1e-5, False), (-1.1e-5, False), (+2e-5, False), (-2e-5, False)]


def _verify(orc, zq, zp, d, F, C, rnd):
    T = 1.0
    ps = orc.softmax(zp, T)
    qs = orc.softmax(zq, T)
    ids, mass = orc.build_cache(zq, T, F)
    Z, _ = orc.saguaro(zq, T, F, ids, mass, C)
    acc, aprob, err, exc = orc.verify(zp, zq, T, d, ps, qs, F, ids, Z, C, SEED, rnd)
    return acc, aprob, err, exc


def _e1_cases():
    """(zq, zp, d, expected flag, expected accepted length) of the E1 cases, all at one
    round whose uniforms at position 0 lie in (0.1, 0.6) (and above 0.45 at position
    0 of the after-rejection case)."""
    n = len(E1_DELTAS)
    bs = list(range(n + 2))
    rnd = find_round(0.1, 0.6, ACCEPT, bs)
    zq = np.zeros((n + 2, 3, 2), np.float32)
    zp = np.zeros((n + 2, 3, 2), np.float32)
    # position 1 of every case accepts far from any tie: q(0) = sigmoid(-3), p(0) = 1/2
    zq[:, 1, 0] = -3.0
    d = np.zeros((n + 2, 2), np.int32)
    want_flag, want_k = [], []
    for b, (delta, flag) in enumerate(E1_DELTAS):
        u = u_np(SEED, rnd, ACCEPT, b, 0)
        zp[b, 0, 0] = logit_for(0.5 * (u + delta))
        ratio = p0_of(zp[b, 0, 0]) / 0.5
        assert abs(abs(u - ratio) - abs(delta)) < 1e-7, (b, u, ratio)
        want_flag.append(flag)
        want_k.append(2 if u < ratio else 0)
    # after a clear rejection at position 0, a near-tie at position 1 is not tested
    b = n
    u0, u1 = u_np(SEED, rnd, ACCEPT, b, 0), u_np(SEED, rnd, ACCEPT, b, 1)
    zp[b, 0, 0] = logit_for(0.5 * (u0 - 0.08))
    zq[b, 1, 0] = 0.0
    zp[b, 1, 0] = logit_for(0.5 * (u1 + 5e-6))
    assert abs(p0_of(zp[b, 1, 0]) / 0.5 - u1 - 5e-6) < 1e-7
    want_flag.append(False)
    want_k.append(0)
    # after a clear acceptance at position 0, a near-tie at position 1 is tested
    b = n + 1
    u0, u1 = u_np(SEED, rnd, ACCEPT, b, 0), u_np(SEED, rnd, ACCEPT, b, 1)
    zp[b, 0, 0] = logit_for(0.5 * min(u0 + 0.3, 1.6))
    zq[b, 1, 0] = 0.0
    zp[b, 1, 0] = logit_for(0.5 * (u1 + 5e-6))
    want_flag.append(True)
    want_k.append(2)
    return zq, zp, d, rnd, np.array(want_flag), np.array(want_k)


def check_e1_band(orc):
    """E1 fires exactly for |u - ratio| < 1e-5 at tested positions (0.9x and 1.1x of
    the band on both sides of u, and 0.5x / 2x)."""
    zq, zp, d, rnd, want_flag, want_k = _e1_cases()
    F = np.zeros(3, np.int32)
    acc, aprob, err, exc = _verify(orc, zq, zp, d, F, 1.0, rnd)
    assert np.array_equal(acc, want_k), (acc, want_k)
    got = (exc & orc.E1_ACCEPT_TIE) != 0
    assert np.array_equal(got, want_flag), (got, want_flag)
    assert not np.any(err)


def check_e1_uses_qprime(orc):
    """With the draft token cached (F_0 = 1, C = 0.5) the tested ratio is p / q' with
    q'(0) = C q(0) / (1 - (1 - C) q(0)) = 1/3 at q(0) = 1/2, not p / q."""
    rnd = find_round(0.1, 0.6, ACCEPT, [0, 1])
    zq = np.zeros((2, 3, 2), np.float32)
    zp = np.zeros((2, 3, 2), np.float32)
    zq[:, 1, 0] = -3.0
    d = np.zeros((2, 2), np.int32)
    C = 0.5
    qp0 = C * 0.5 / (1.0 - (1.0 - C) * 0.5)
    for b, delta in enumerate((5e-6, 2e-5)):
        u = u_np(SEED, rnd, ACCEPT, b, 0)
        zp[b, 0, 0] = logit_for(qp0 * (u + delta))
        assert abs(p0_of(zp[b, 0, 0]) / qp0 - u - delta) < 1e-7
    F = np.array([1, 0, 0], np.int32)
    acc, aprob, err, exc = _verify(orc, zq, zp, d, F, C, rnd)
    got = (exc & orc.E1_ACCEPT_TIE) != 0
    assert got.tolist() == [True, False], got
    assert acc.tolist() == [2, 2]


def check_e1_ratio_above_one(orc):
    """A uniform within 1e-5 of 1 and a ratio of 1.5: accepted with room to spare, not
    flagged (|u - 1.5| ~ 0.5; the slip min(1, ratio) would flag it)."""
    rnd = find_round(1.0 - 5e-6, 1.0, ACCEPT, [0], n=4000000)
    zq = np.zeros((1, 3, 2), np.float32)
    zp = np.zeros((1, 3, 2), np.float32)
    zq[0, 1, 0] = -3.0
    zp[0, 0, 0] = logit_for(0.75)  # ratio 1.5 against q(0) = 1/2
    acc, aprob, err, exc = _verify(orc, zq, zp, np.zeros((1, 2), np.int32), np.zeros(3, np.int32), 1.0, rnd)
    assert acc[0] == 2 and exc[0] == 0, (acc, exc)


def check_e5_band(orc):
    """E5: a tested probability below 1e-30 from a finite logit (target or draft side)
    is flagged; -inf (probability exactly 0), 1e-29, and an untested position are not."""
    rnd = find_round(0.2, 0.8, ACCEPT, list(range(7)))
    cases = [  # (zp row 0, zq row 0, zp row 1 (tested only after an acceptance), flag)
        (np.log(1e-31), 0.0, 0.0, True),            # p ~ 1e-31 * 2
        (np.log(1e-29), 0.0, 0.0, False),           # p ~ 2e-29 > 1e-30
        (-np.inf, 0.0, 0.0, False),                 # masked: p = 0 in any precision
        (0.0, np.log(1e-31), 0.0, True),            # q' ~ 1e-31 (accepted: ratio huge)
        (0.0, -np.inf, 0.0, False),                 # q' = 0: an error bit, not E5
        (-6.0, 0.0, np.log(1e-31), False),          # rejected at 0; position 1 untested
        (6.0, 0.0, np.log(1e-31), True),            # accepted at 0; position 1 tested
    ]
    B = len(cases)
    zq = np.zeros((B, 3, 2), np.float32)
    zp = np.zeros((B, 3, 2), np.float32)
    zq[:, 1, 0] = -3.0  # position 1 accepts far from a tie unless its target is tiny
    want = []
    for b, (p0, q0, p1, flag) in enumerate(cases):
        zp[b, 0, 0], zq[b, 0, 0], zp[b, 1, 0] = p0, q0, p1
        want.append(flag)
    acc, aprob, err, exc = _verify(orc, zq, zp, np.zeros((B, 2), np.int32), np.zeros(3, np.int32), 1.0, rnd)
    got = (exc & orc.E5_TINY_PROB) != 0
    assert got.tolist() == want, (got, want)
    assert err[4] == orc.ERR_QPRIME_ZERO and acc[4] == 0
    assert acc[2] == 0 and acc[5] == 0 and acc[3] == 2
    assert not np.any(exc & orc.E1_ACCEPT_TIE)


# --------------------------------------------------------------------------- E2: inverse CDF
def _e2_deltas(eps):
    return [(0.5 * eps, True), (-0.5 * eps, True), (0.9 * eps, True), (-0.9 * eps, True),
            (1.1 * eps, False), (-1.1 * eps, False), (2.5 * eps, False), (-2.5 * eps, False)]


def check_e2_draft_sampler(orc):
    """Draft sampler, V = 2: q'(0) = u + delta puts the CDF step at distance |delta|
    from u, on either side; flagged iff |delta| < CDF_TIE_EPS.  Each case is drawn
    once with id 0 uncached (q' = q) and once cached (F_0 = 1, C = 0.5, where id 0
    holds the larger logit), so that q' differs from q."""
    eps = orc.CDF_TIE_EPS
    C = 0.5
    for cached in (False, True):
        for delta, flag in _e2_deltas(eps):
            rnd = find_round(0.4, 0.9, DRAFT, [0])
            u = u_np(SEED, rnd, DRAFT, 0, 0)
            t = u + delta
            zq = np.zeros((1, 2, 2), np.float32)
            if not cached:
                zq[0, 0, 0] = logit_for(t)
                qp0 = p0_of(zq[0, 0, 0])
            else:  # q'(0) = C q / (1 - (1 - C) q), q > 1/2 so that id 0 is the top-1
                q = t / (C + (1.0 - C) * t)
                zq[0, 0, 0] = logit_for(q)
                q = p0_of(zq[0, 0, 0])
                qp0 = C * q / (1.0 - (1.0 - C) * q)
            assert abs(qp0 - t) < 2e-8, (qp0, t)
            F = np.array([1 if cached else 0, 0], np.int32)
            ids, mass = orc.build_cache(zq, 1.0, F)
            Z, _ = orc.saguaro(zq, 1.0, F, ids, mass, C)
            d, flags = orc.draft_sample(zq, 1.0, F, ids, Z, C, SEED, rnd)
            assert d[0, 0] == (0 if u < qp0 else 1), (cached, delta, d)
            assert bool(flags[0, 0]) == flag, (cached, delta, flags)


def check_e2_bonus_all_accepted(orc):
    """Bonus after all K accepted (w = p_K, Z_r = 1), V = 2: p_K(0) = u + delta."""
    eps = orc.CDF_TIE_EPS
    deltas = _e2_deltas(eps)
    B = len(deltas)
    K = 1
    rnd = find_round(0.2, 0.8, BONUS, list(range(B)), i=K)
    zq = np.zeros((B, K + 1, 2), np.float32)
    zp = np.zeros((B, K + 1, 2), np.float32)
    want_b = []
    for b, (delta, flag) in enumerate(deltas):
        u = u_np(SEED, rnd, BONUS, b, K)
        zp[b, K, 0] = logit_for(u + delta)
        assert abs(p0_of(zp[b, K, 0]) - u - delta) < 2e-8
        want_b.append(0 if u < p0_of(zp[b, K, 0]) else 1)
    want_f = [f for _, f in deltas]
    _bonus_check(orc, zq, zp, np.full(B, K, np.int32), rnd, want_b, want_f)


def check_e2_bonus_residual(orc):
    """Bonus after a rejection at position 0 (w = max(p - q, 0)), V = 3: q =
    softmax([0, 0, 2]) and p chosen so that w = (w0, 0.2, 0) with
    w0 / (w0 + 0.2) = u + delta, i.e. the first CDF step at distance |delta| from u."""
    eps = orc.CDF_TIE_EPS
    deltas = _e2_deltas(eps)
    B = len(deltas)
    rnd = find_round(0.2, 0.55, BONUS, list(range(B)))
    zq = np.zeros((B, 2, 3), np.float32)
    zp = np.zeros((B, 2, 3), np.float32)
    zq[:, 0, 2] = 2.0
    q = softmax64(zq[0, 0])
    want_b = []
    for b, (delta, flag) in enumerate(deltas):
        u = u_np(SEED, rnd, BONUS, b, 0)
        t = u + delta
        w1 = 0.2
        w0 = t * w1 / (1.0 - t)
        p0, p1 = q[0] + w0, q[1] + w1
        p2 = 1.0 - p0 - p1
        assert p2 < q[2]
        zp[b, 0] = np.array([np.log(p0 / p2), np.log(p1 / p2), 0.0], np.float32)
        p = softmax64(zp[b, 0])
        w = np.maximum(p - q, 0.0)
        c0 = w[0] / w.sum()
        assert w[2] == 0.0 and abs(c0 - t) < 2e-7, (b, c0, t)
        want_b.append(0 if u < c0 else 1)
    want_f = [f for _, f in deltas]
    _bonus_check(orc, zq, zp, np.zeros(B, np.int32), rnd, want_b, want_f)


def _bonus_check(orc, zq, zp, acc, rnd, want_b, want_f):
    T, C = 1.0, 1.0
    K = zq.shape[1] - 1
    F = np.zeros(K + 1, np.int32)
    ps, qs = orc.softmax(zp, T), orc.softmax(zq, T)
    ids, mass = orc.build_cache(zq, T, F)
    Z, _ = orc.saguaro(zq, T, F, ids, mass, C)
    bonus, zr, _, err, exc = orc.residual_sample(zp, zq, T, ps, qs, F, ids, Z, C, acc, SEED, rnd)
    assert bonus.tolist() == want_b, (bonus, want_b)
    got = (exc & orc.E2_CDF_TIE) != 0
    assert got.tolist() == want_f, (got, want_f)
    assert not np.any(exc & orc.E3_DEGENERATE_RESIDUAL)


# --------------------------------------------------------------------------- E3: residual mass
def check_e3_band(orc):
    """E3: after a rejection (k = 0 < K = 1), V = 2, q = (1/2, 1/2) and p(0) = 1/2 + z
    give the residual w = (z, 0) with Z_r = z; flagged iff z < 1e-5.  Identical rows
    (Z_r = 0 exactly) are flagged and fall back to p; all accepted (k = K) is never
    flagged."""
    zs = [(5e-6, True), (9e-6, True), (1.1e-5, False), (2e-5, False), (1e-3, False)]
    B = len(zs) + 2
    zq = np.zeros((B, 2, 2), np.float32)
    zp = np.zeros((B, 2, 2), np.float32)
    acc = np.zeros(B, np.int32)
    want = []
    for b, (z, flag) in enumerate(zs):
        zp[b, 0, 0] = logit_for(0.5 + z)
        assert abs(p0_of(zp[b, 0, 0]) - 0.5 - z) < 2e-9 + 1e-4 * z
        want.append(flag)
    zp[len(zs), 0] = zq[len(zs), 0] = np.array([0.3, -0.2], np.float32)  # p == q: Z_r = 0
    want.append(True)
    zp[len(zs) + 1, 1, 0] = logit_for(0.5 + 5e-6)  # k = K: w = p_K
    zq[len(zs) + 1, 1, 0] = 0.0
    acc[len(zs) + 1] = 1
    want.append(False)
    T, C = 1.0, 1.0
    F = np.zeros(2, np.int32)
    ps, qs = orc.softmax(zp, T), orc.softmax(zq, T)
    ids, mass = orc.build_cache(zq, T, F)
    Z, _ = orc.saguaro(zq, T, F, ids, mass, C)
    bonus, zr, _, err, exc = orc.residual_sample(zp, zq, T, ps, qs, F, ids, Z, C, acc, SEED, 3)
    got = (exc & orc.E3_DEGENERATE_RESIDUAL) != 0
    assert got.tolist() == want, (got, want, zr)
    for b, (z, _) in enumerate(zs):
        assert abs(zr[b] - (p0_of(zp[b, 0, 0]) - 0.5)) < 1e-14 and bonus[b] == 0
    # Z_r = 0: the bonus is drawn from p (both ids possible), the mass reported is 1
    assert abs(zr[len(zs)] - 1.0) < 1e-15


CHECKS = [check_e1_band, check_e1_uses_qprime, check_e1_ratio_above_one, check_e5_band, check_e2_draft_sampler,
          check_e2_bonus_all_accepted, check_e2_bonus_residual, check_e3_band]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_exception_pin(orc, check):
    check(orc)


def test_band_constants(orc):
    """The bands the pins above bracket: E1 and E3 at 1e-5 (the parity rule), E2 at the
    derived CDF_TIE_EPS, which the rule caps at 1e-5."""
    assert 0 < orc.CDF_TIE_EPS <= 1e-5


# --------------------------------------------------------------------------- mutations
SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "ssd_oracle.c")

MUTANTS = [
    ("E1 band 2e-5", "#define ORC_TIE_EPS 1e-5", "#define ORC_TIE_EPS 2e-5"),
    ("E1 band 5e-6", "#define ORC_TIE_EPS 1e-5", "#define ORC_TIE_EPS 5e-6"),
    ("E1 against min(1, ratio)", "if (fabs(u - ratio) < ORC_TIE_EPS)",
     "if (fabs(u - (ratio < 1.0 ? ratio : 1.0)) < ORC_TIE_EPS)"),
    ("E1/E5 after the first rejection", "if (k == K) {\n                    /* no earlier rejection",
     "if (1) {\n                    /* no earlier rejection"),
    ("E3 band 1e-6", "#define ORC_RESID_EPS 1e-5", "#define ORC_RESID_EPS 1e-6"),
    ("E5 flags -inf", "(p < ORC_TINY && !isinf(zpd))", "(p < ORC_TINY)"),
    ("E5 band 1e-28", "#define ORC_TINY 1e-30", "#define ORC_TINY 1e-28"),
    ("E2 gap on one side only", "*gap = a < c ? a : c;", "*gap = a;"),
    ("E2 gap unnormalised", "double a = fabs(run / total - u), c = fabs(prev / total - u);",
     "double a = fabs(run - u), c = fabs(prev - u);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutants_fail_a_pin(orc, tmp_path, name, old, new):
    """A plausible slip in the flag logic fails at least one pin above."""
    text = open(SRC).read()
    assert text.count(old) == 1, name
    path = orc.compile_variant(text.replace(old, new), str(tmp_path / "mut.so"))
    saved = orc._lib
    orc._lib = orc.load_library(path)
    try:
        failed = []
        for check in CHECKS:
            try:
                check(orc)
            except AssertionError:
                failed.append(check.__name__)
    finally:
        orc._lib = saved
    assert failed, "mutant '%s' passes every pin" % name


def test_e2_band_mutation_fails_a_pin(orc):
    """The E2 band is a parameter of the oracle's calls: a band 1.2x too wide or 0.8x
    too narrow fails a pin."""
    saved = orc.CDF_TIE_EPS
    for scale in (1.2, 0.8):
        orc.CDF_TIE_EPS = saved * scale
        try:
            with pytest.raises(AssertionError):
                for check in (check_e2_draft_sampler, check_e2_bonus_all_accepted, check_e2_bonus_residual):
                    # the cases are rebuilt around the true band
                    _with_band(check, orc, saved)
        finally:
            orc.CDF_TIE_EPS = saved


def _with_band(check, orc, true_eps):
    """Runs an E2 check whose cases sit around true_eps while the oracle is called
    with whatever orc.CDF_TIE_EPS holds."""
    used = orc.CDF_TIE_EPS

    class View:
        def __getattr__(self, k):
            if k == "CDF_TIE_EPS":
                return true_eps
            return getattr(orc, k)

    v = View()
    # residual_sample / draft_sample read orc.CDF_TIE_EPS as their default band
    assert orc.CDF_TIE_EPS == used
    check(v)
