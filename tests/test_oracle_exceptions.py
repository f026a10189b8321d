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
  E2  a uniform of a draw within its band of one of the two normalised CDF steps
      around its pick, at the block level (u1) or the id level (u2); the band is
      derived per draw from the arithmetic of the GPU path, at least CDF_TIE_EPS
      (draft sampler and bonus);
  E3  residual mass Z_r < 1e-5 after a rejection (k < K);
  E5  a tested p_i(d_i) or q'_i(d_i) below 1e-30 from a finite logit.
A final test compiles mutated copies of ssd_oracle.c (a wrong band, the
min(1, ratio) slip, flags after the first rejection, the -inf exemption dropped,
one side of the CDF gap dropped, the band's random part dropped, the levels' uniforms
swapped) and checks that each one fails a pin here.
"""
import os

import numpy as np
import pytest

SEED = 0x7E57
ACCEPT, BONUS, DRAFT = 0, 1, 2


# --------------------------------------------------------------------------- helpers
def u_np(seed, rnd, purpose, b, i, w3=0):
    """U(seed, rnd, b, i, purpose) from numpy's Philox4x64-10: the first output word
    of counter (rnd, b, i, w3) under key (seed, purpose), top 24 bits times 2^-24
    (numpy increments the counter before producing a block); w3 = 1 gives a draw's
    second uniform."""
    assert rnd >= 1
    g = np.random.Philox(key=np.array([seed, purpose], np.uint64),
                         counter=np.array([rnd - 1, b, i, w3], np.uint64))
    return (int(g.random_raw(1)[0]) >> 40) / 2.0**24


def us_over_rounds(seed, purpose, b, i, r0, n, w3=0):
    """u for rounds r0 .. r0+n-1 at (b, i): consecutive numpy Philox blocks advance
    counter word 0, which is the round."""
    g = np.random.Philox(key=np.array([seed, purpose], np.uint64),
                         counter=np.array([r0 - 1, b, i, w3], np.uint64))
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


def find_round(lo, hi, purpose, bs, i=0, r0=1, n=200000, w3=0, also=None):
    """The first round r >= r0 whose uniforms (counter word w3) at (b, i) lie in
    (lo, hi) for every b in bs, and, with also = (w3', lo', hi'), whose uniforms of
    word w3' lie in (lo', hi')."""
    ok = np.ones(n, bool)
    for b in bs:
        u = us_over_rounds(SEED, purpose, b, i, r0, n, w3)
        ok &= (u > lo) & (u < hi)
        if also is not None:
            u = us_over_rounds(SEED, purpose, b, i, r0, n, also[0])
            ok &= (u > also[1]) & (u < also[2])
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


# --------------------------------------------------------------------------- E2: the draws
# A draw takes u1 (last counter word 0) for its block of 512 ids and u2 (word 1) for
# the id within the block.  Each case puts one CDF step at a distance delta from the
# uniform of one level: at the id level V = 2 or 3 (a single block), at the block level
# V = 1024 with mass on id 0 (block 0) and id 1023 (block 1) only, so that the id level
# has one id per block and nothing to decide.  delta is a multiple of the band the
# oracle reports for the draw (probed at delta = 0); the gap it reports must equal
# |step - u| recomputed here from the fp32 logits, the band must lie in the range the
# arithmetic of the GPU path gives for such rows (a few fp32 ulps, about 3e-7), and
# the flag must fire exactly for |delta| below the band.
E2_FACTORS = [(0.5, True), (-0.5, True), (0.9, True), (-0.9, True),
              (1.1, False), (-1.1, False), (2.5, False), (-2.5, False)]
LEVELS = {"id": (2, 1), "block": (1024, 0)}  # level -> (V, counter word of its uniform)


def _u_of(rnd, purpose, b, i, w3):
    return u_np(SEED, rnd, purpose, b, i, w3)


def _round_for_level(purpose, w3, i=0, lo=0.4, hi=0.9):
    """A round whose uniform of the tested level lies in (lo, hi) and whose other
    uniform lies in (0.1, 0.9), away from the steps 0 and 1 of a one-entry level."""
    return find_round(lo, hi, purpose, [0], i=i, w3=w3, also=(1 - w3, 0.1, 0.9))


def _check_e2_info(info, level, t, u, flag):
    """info = (gap of u1, band of u1, gap of u2, band of u2) of one draw."""
    lv = 0 if level == "block" else 1
    gap, band = info[2 * lv], info[2 * lv + 1]
    assert abs(gap - abs(t - u)) < 1e-12, (level, gap, t, u)
    assert 5e-8 < band < 2e-6, (level, band)
    assert info[2 * (1 - lv)] > 0.09 and info[2 * (1 - lv) + 1] < 1e-5, info
    assert (gap < band) == flag, (level, gap, band, flag)


def _draft_row(V, t, cached, C):
    """Draft logits over V ids whose reweighted law holds t on id 0 and 1 - t on id
    V - 1 (the rest masked); cached: id 0 is the cached top-1 (F_0 = 1) with weight C.
    Returns the row and q'(0) recomputed in fp64 from its fp32 logits."""
    z = np.full(V, -np.inf, np.float32)
    z[V - 1] = 0.0
    if not cached:
        z[0] = logit_for(t)
        return z, p0_of(z[0])
    q = t / (C + (1.0 - C) * t)  # q'(0) = C q / (1 - (1 - C) q), q > 1/2: id 0 is the top-1
    z[0] = logit_for(q)
    q = p0_of(z[0])
    return z, C * q / (1.0 - (1.0 - C) * q)


def check_e2_draft_sampler(orc):
    """Draft sampler at both levels, each case drawn once with id 0 uncached (q' = q)
    and once cached (F_0 = 1, C = 0.5), so that q' differs from q."""
    C = 0.5
    for level, (V, w3) in LEVELS.items():
        rnd = _round_for_level(DRAFT, w3)
        u = _u_of(rnd, DRAFT, 0, 0, w3)
        for cached in (False, True):
            F = np.array([1 if cached else 0, 0], np.int32)

            def draw(t):
                zq = np.zeros((1, 2, V), np.float32)
                zq[0, 0], qp0 = _draft_row(V, t, cached, C)
                ids, mass = orc.build_cache(zq, 1.0, F)
                Z, _ = orc.saguaro(zq, 1.0, F, ids, mass, C)
                d, flags, e2 = orc.draft_sample(zq, 1.0, F, ids, Z, C, SEED, rnd, want_gaps=True)
                return qp0, d[0, 0], bool(flags[0, 0]), e2[0, 0]

            band = draw(u)[3][2 * w3 + 1]
            for f, flag in E2_FACTORS:
                qp0, d, got, info = draw(u + f * band)
                assert abs(qp0 - u - f * band) < 0.05 * band, (level, cached, f, qp0, u)
                assert d == (0 if u < qp0 else V - 1), (level, cached, f, d)
                assert got == flag, (level, cached, f, info)
                _check_e2_info(info, level, qp0, u, flag)


def check_e2_bonus_all_accepted(orc):
    """Bonus after all K = 1 accepted (w = p_K) at both levels: p_K(0) = u + delta on
    id 0 and the rest on id V - 1."""
    K = 1
    for level, (V, w3) in LEVELS.items():
        rnd = _round_for_level(BONUS, w3, i=K, lo=0.2, hi=0.8)
        u = _u_of(rnd, BONUS, 0, K, w3)

        def draw(t):
            zq = np.zeros((1, K + 1, V), np.float32)
            zp = np.zeros((1, K + 1, V), np.float32)
            zp[0, K], p0 = _draft_row(V, t, False, 1.0)
            return (p0,) + _bonus(orc, zq, zp, np.full(1, K, np.int32), rnd)

        band = draw(u)[4][2 * w3 + 1]
        for f, flag in E2_FACTORS:
            p0, bonus, got, zr, info = draw(u + f * band)
            assert abs(p0 - u - f * band) < 0.05 * band
            assert bonus == (0 if u < p0 else V - 1), (level, f, bonus)
            assert got == flag, (level, f, info)
            _check_e2_info(info, level, p0, u, flag)


def check_e2_bonus_residual(orc):
    """Bonus after a rejection at position 0 (w = max(p - q, 0)) at both levels: ids
    (a, b, c) = (0, 1, 2) of V = 3 (id level) or (0, 1023, 512) of V = 1024 (block
    level, a and b in different blocks, c beside b's block); q puts logits (0, 0, 2)
    on them and p is chosen so that w = (w_a, 0.2, 0) with w_a / (w_a + 0.2) = u +
    delta, i.e. the first CDF step of the level at distance |delta| from u."""
    for level, V, w3 in (("id", 3, 1), ("block", 1024, 0)):
        ia, ib, ic = (0, 1, 2) if V == 3 else (0, 1023, 512)
        rnd = _round_for_level(BONUS, w3, lo=0.2, hi=0.55)
        u = _u_of(rnd, BONUS, 0, 0, w3)
        zq = np.full((1, 2, V), -np.inf, np.float32)
        zq[0, :, [ia, ib, ic]] = np.array([0.0, 0.0, 2.0], np.float32)[:, None]
        q = softmax64(zq[0, 0, [ia, ib, ic]])

        def draw(t):
            w1 = 0.2
            w0 = t * w1 / (1.0 - t)
            p0, p1 = q[0] + w0, q[1] + w1
            p2 = 1.0 - p0 - p1
            assert p2 < q[2]
            zp = np.full((1, 2, V), -np.inf, np.float32)
            zp[0, :, [ia, ib, ic]] = np.array([np.log(p0 / p2), np.log(p1 / p2), 0.0], np.float32)[:, None]
            w = np.maximum(softmax64(zp[0, 0, [ia, ib, ic]]) - q, 0.0)
            assert w[2] == 0.0
            return (w[0] / w.sum(),) + _bonus(orc, zq, zp, np.zeros(1, np.int32), rnd)

        band = draw(u)[4][2 * w3 + 1]
        for f, flag in E2_FACTORS:
            c0, bonus, got, zr, info = draw(u + f * band)
            assert abs(c0 - u - f * band) < 0.05 * band, (level, f, c0, u)
            assert bonus == (ia if u < c0 else ib), (level, f, bonus)
            assert got == flag, (level, f, info)
            _check_e2_info(info, level, c0, u, flag)


def _bonus(orc, zq, zp, acc, rnd):
    """(bonus, E2 flag, Z_r, (gap, band) info) of one sequence at T = 1, C = 1."""
    T, C = 1.0, 1.0
    K = zq.shape[1] - 1
    F = np.zeros(K + 1, np.int32)
    ps, qs = orc.softmax(zp, T), orc.softmax(zq, T)
    ids, mass = orc.build_cache(zq, T, F)
    Z, _ = orc.saguaro(zq, T, F, ids, mass, C)
    bonus, zr, _, err, exc, e2 = orc.residual_sample(zp, zq, T, ps, qs, F, ids, Z, C, acc, SEED, rnd,
                                                     want_bands=True)
    assert not np.any(exc & orc.E3_DEGENERATE_RESIDUAL) and not np.any(err)
    return int(bonus[0]), bool(exc[0] & orc.E2_CDF_TIE), float(zr[0]), e2[0]


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
    """The bands the pins above bracket: E1 and E3 at 1e-5 (the parity rule); the floor
    CDF_TIE_EPS of the per-draw E2 bands is capped by the rule at 1e-5."""
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
    ("E2 band without its random part", "#define ORC_CDF_SIGMAS 6.0", "#define ORC_CDF_SIGMAS 0.0"),
    ("E2 draft uniforms swapped", "draft[bi] = draw_two_level(w, V, u1, u2, &blk, gap);",
     "draft[bi] = draw_two_level(w, V, u2, u1, &blk, gap);"),
    ("E2 bonus uniforms swapped", "bonus[b] = draw_two_level(w, V, u1, u2, &blk, gap);",
     "bonus[b] = draw_two_level(w, V, u2, u1, &blk, gap);"),
    ("E2 second uniform from counter word 0", "philox_word(seed, round, purpose, b, i, 1)",
     "philox_word(seed, round, purpose, b, i, 0)"),
    ("E2 blocks of 1024 ids", "#define ORC_BLOCK 512", "#define ORC_BLOCK 1024"),
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
