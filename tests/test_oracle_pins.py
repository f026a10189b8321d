"""Pins of the fp64 oracle against things other than itself: numpy library
routines, an independent generator implementation, brute force and closed forms.
CPU only."""
import itertools
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_logits(rng, B, K, V, scale=2.0, dtype="f32"):
    z = (rng.standard_normal((B, K + 1, V)) * scale).astype(np.float32)
    if dtype == "bf16":
        # round-to-nearest-even to bf16 bits (the oracle widens them exactly)
        u = z.view(np.uint32).astype(np.uint64)
        rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        return rounded
    return z


def _widen(z):
    if z.dtype == np.uint16:
        return (z.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return z.astype(np.float64)


# --------------------------------------------------------------------------- RNG
def test_philox_matches_numpy(orc):
    """P11: Philox4x64-10 equals numpy's independent implementation (numpy's
    generator increments its counter before producing a block)."""
    rng = np.random.default_rng(1)
    for _ in range(50):
        ctr = rng.integers(1, 2**63, size=4, dtype=np.uint64)
        key = rng.integers(0, 2**63, size=2, dtype=np.uint64)
        mine = orc.philox4x64_10(ctr, key)
        bg = np.random.Philox(key=key, counter=ctr - np.array([1, 0, 0, 0], dtype=np.uint64))
        assert np.array_equal(mine, bg.random_raw(4))


def test_uniform_definition_and_ks(orc):
    """P11: u = (first word >> 40) * 2^-24 from numpy's Philox; uniform on [0,1)."""
    seed, rnd = 0x55D3, 17
    us = []
    for b in range(40):
        for i in range(50):
            u = orc.uniform(seed, rnd, orc.PURPOSE_ACCEPT, b, i)
            bg = np.random.Philox(key=np.array([seed, orc.PURPOSE_ACCEPT], dtype=np.uint64),
                                  counter=np.array([rnd - 1, b, i, 0], dtype=np.uint64))
            w0 = int(bg.random_raw(1)[0])
            assert u == (w0 >> 40) / 2.0**24
            assert orc.uniform_u32(seed, rnd, orc.PURPOSE_ACCEPT, b, i) == w0 >> 32
            us.append(u)
            # a draw's second uniform: last counter word 1
            bg = np.random.Philox(key=np.array([seed, orc.PURPOSE_BONUS], dtype=np.uint64),
                                  counter=np.array([rnd - 1, b, i, 1], dtype=np.uint64))
            assert orc.uniform2(seed, rnd, orc.PURPOSE_BONUS, b, i) == (int(bg.random_raw(1)[0]) >> 40) / 2.0**24
    from scipy import stats
    assert stats.kstest(us, "uniform").pvalue > 1e-3


# --------------------------------------------------------------------------- fan-out
def _lr_bruteforce(K, Bf, r):
    """Largest-remainder apportionment characterised independently: among all
    floor/ceil roundings of f_k = Bf r^k / sum r^j that sum to Bf, the one with the
    smallest L1 distance to f; among equals the one rounding lower k up first."""
    w = np.array([r**k for k in range(K + 1)])
    f = Bf * w / w.sum()
    fl = np.floor(f).astype(int)
    best = None
    for ups in itertools.product([0, 1], repeat=K + 1):
        F = fl + np.array(ups)
        if F.sum() != Bf:
            continue
        cost = np.abs(F - f).sum()
        key = (round(cost, 12), tuple(-u for u in ups))
        if best is None or key < best[0]:
            best = (key, F)
    return best[1], f


@pytest.mark.parametrize("K,Bf,r", [(4, 16, 0.7), (5, 32, 0.6), (8, 64, 0.7), (6, 96, 0.8),
                                    (4, 32, 0.5), (3, 10, 1.0), (1, 0, 0.3), (7, 5, 0.9), (2, 7, 0.25)])
def test_fanout_largest_remainder(orc, K, Bf, r):
    """P6: sum F = Bf, F non-increasing in k, |F_k - f_k| < 1, and F is the L1-closest
    integer rounding of the geometric shares (brute force)."""
    F, gap = orc.fanout(K, Bf, r)
    ref, f = _lr_bruteforce(K, Bf, r)
    assert F.sum() == Bf
    assert np.all(np.diff(F) <= 0)
    assert np.all(np.abs(F - f) < 1)
    if gap > 1e-9:
        assert np.array_equal(F, ref)


def test_fanout_golden(orc):
    """P6: the fan-out of the five workloads, stored by tests/golden/make_golden.py."""
    with open(os.path.join(GOLDEN, "fanout_workloads.json")) as fh:
        g = json.load(fh)
    for row in g["rows"]:
        F, _ = orc.fanout(row["K"], row["Bf"], row["r"])
        assert F.tolist() == row["F"]


# --------------------------------------------------------------------------- softmax
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [0.0, 0.5, 1.0, 1.7])
def test_softmax_matches_numpy(orc, dtype, T):
    """P1 / P10: softmax equals numpy exp((z - max)/T) / sum; greedy equals np.argmax
    (first maximum); sum p = 1."""
    rng = np.random.default_rng(2)
    z = _rand_logits(rng, 3, 2, 257, 3.0, dtype)
    m, s, a, probs = orc.softmax(z, T, want_probs=True)
    zz = _widen(z)
    ref_arg = np.argmax(zz, axis=-1)
    assert np.array_equal(a, ref_arg)
    assert np.array_equal(m, zz.max(-1))
    if T > 0:
        e = np.exp((zz - zz.max(-1, keepdims=True)) / T)
        ref = e / e.sum(-1, keepdims=True)
        np.testing.assert_allclose(probs, ref, rtol=0, atol=1e-15)
    else:
        ref = np.zeros_like(zz)
        np.put_along_axis(ref, ref_arg[..., None], 1.0, axis=-1)
        assert np.array_equal(probs, ref)
    np.testing.assert_allclose(probs.sum(-1), 1.0, atol=1e-13)


def test_softmax_ties_and_padded_rows(orc):
    """Greedy ties go to the lower id; a row stride larger than V is honoured."""
    z = np.zeros((1, 2, 16), dtype=np.float32)
    z[0, 0, [3, 9]] = 5.0
    z[0, 1, :] = -1.0
    _, _, a, _ = orc.softmax(z, 0.0)
    assert a.tolist() == [[3, 0]]
    big = np.full((2, 3, 40), np.nan, dtype=np.float32)
    rng = np.random.default_rng(3)
    big[:, :, :33] = rng.standard_normal((2, 3, 33))
    view = big[:, :, :33]
    m1, s1, a1, _ = orc.softmax(view, 1.0)
    m2, s2, a2, _ = orc.softmax(np.ascontiguousarray(view), 1.0)
    assert np.array_equal(a1, a2) and np.array_equal(m1, m2) and np.array_equal(s1, s2)


# --------------------------------------------------------------------------- cache
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topF_matches_lexsort(orc, dtype):
    """P8: S_k = the first F_k ids of np.lexsort((ids, -z)); M_k = sum of q over them."""
    rng = np.random.default_rng(4)
    K, V = 4, 300
    z = _rand_logits(rng, 3, K, V, 2.0, dtype)
    if dtype == "bf16":
        # heavy bf16 ties: quantise further so many equal values appear
        z = (z & 0xFFE0).astype(np.uint16)
    F, _ = orc.fanout(K, 40, 0.6)
    T = 0.9
    ids, mass = orc.build_cache(z, T, F)
    zz = _widen(z)
    _, _, _, probs = orc.softmax(z, T, want_probs=True)
    O = np.concatenate([[0], np.cumsum(F)])
    for b in range(3):
        for k in range(K + 1):
            order = np.lexsort((np.arange(V), -zz[b, k]))
            ref = order[:F[k]]
            assert ids[b, O[k]:O[k + 1]].tolist() == ref.tolist()
            np.testing.assert_allclose(mass[b, k], probs[b, k, ref].sum(), atol=1e-14)


def test_topF_greedy_mass(orc):
    """At T = 0 the cached mass is 1 when F_k >= 1 (the argmax is cached first) and 0
    when F_k = 0."""
    rng = np.random.default_rng(5)
    z = _rand_logits(rng, 2, 3, 50)
    F = np.array([3, 0, 2, 1], dtype=np.int32)
    ids, mass = orc.build_cache(z, 0.0, F)
    assert mass.tolist() == [[1.0, 0.0, 1.0, 1.0]] * 2
    assert ids[:, 0].tolist() == np.argmax(z[:, 0], -1).tolist()


# --------------------------------------------------------------------------- Saguaro
@pytest.mark.parametrize("C", [0.2, 0.5, 1.0])
def test_saguaro_invariants(orc, C):
    """P7: sum q' = 1; q'/q is C/Z on S_k and 1/Z elsewhere; C = 1 gives q' = q."""
    rng = np.random.default_rng(6)
    K, V, T = 3, 120, 1.0
    z = _rand_logits(rng, 2, K, V)
    F, _ = orc.fanout(K, 20, 0.7)
    ids, mass = orc.build_cache(z, T, F)
    Z, qp = orc.saguaro(z, T, F, ids, mass, C, want_qprime=True)
    _, _, _, q = orc.softmax(z, T, want_probs=True)
    np.testing.assert_allclose(qp.sum(-1), 1.0, atol=1e-13)
    O = np.concatenate([[0], np.cumsum(F)])
    for b in range(2):
        for k in range(K + 1):
            S = set(ids[b, O[k]:O[k + 1]].tolist())
            ratio = qp[b, k] / q[b, k]
            for x in range(V):
                want = (C if x in S else 1.0) / Z[b, k]
                assert abs(ratio[x] - want) < 1e-12 * max(1.0, want)
            np.testing.assert_allclose(Z[b, k], 1 - (1 - C) * q[b, k, list(S)].sum(), atol=1e-14)
    if C == 1.0:
        np.testing.assert_allclose(qp, q, atol=1e-15)


def test_saguaro_empty_cache_is_identity(orc):
    """F_k = 0 leaves q'_k = q_k."""
    rng = np.random.default_rng(7)
    z = _rand_logits(rng, 1, 2, 40)
    F = np.array([0, 0, 0], dtype=np.int32)
    ids, mass = orc.build_cache(z, 1.0, F)
    Z, qp = orc.saguaro(z, 1.0, F, ids, mass, 0.3, want_qprime=True)
    _, _, _, q = orc.softmax(z, 1.0, want_probs=True)
    assert np.all(Z == 1.0)
    np.testing.assert_allclose(qp, q, atol=1e-15)


# --------------------------------------------------------------------------- residual / sampler
def _setup(orc, rng, B, K, V, T, C, Bf=12, r=0.7, scale=2.0, corr_noise=0.8):
    zq = (rng.standard_normal((B, K + 1, V)) * scale).astype(np.float32)
    zp = (zq + rng.standard_normal((B, K + 1, V)) * corr_noise).astype(np.float32)
    F, _ = orc.fanout(K, Bf, r)
    ids, mass = orc.build_cache(zq, T, F)
    Z, qp = orc.saguaro(zq, T, F, ids, mass, C, want_qprime=True)
    ps = orc.softmax(zp, T, want_probs=True)
    qs = orc.softmax(zq, T, want_probs=True)
    return zp, zq, F, ids, mass, Z, qp, ps, qs


def _u_np(seed, rnd, purpose, b, i, w3):
    bg = np.random.Philox(key=np.array([seed, purpose], dtype=np.uint64),
                          counter=np.array([rnd - 1, b, i, w3], dtype=np.uint64))
    return (int(bg.random_raw(1)[0]) >> 40) / 2.0**24


def _two_level(w, u1, u2, block=512):
    """The two-level draw with numpy's searchsorted: the block of 512 ids from the
    running block masses at u1, then the id within it from its running sums at u2."""
    W = np.array([w[s:s + block].sum() for s in range(0, w.shape[0], block)])
    b = int(np.searchsorted(np.cumsum(W), u1 * W.sum(), side="right"))
    wb = w[b * block:(b + 1) * block]
    return b * block + int(np.searchsorted(np.cumsum(wb), u2 * W[b], side="right"))


@pytest.mark.parametrize("T", [0.8, 1.0])
def test_residual_invariants_and_searchsorted(orc, T):
    """P5 / P9: w >= 0 and sums to Z_r; after a rejection w(d_k) = 0 and bonus != d_k;
    the bonus equals the two-level draw by np.searchsorted (blocks of 512 ids, V = 1100:
    two whole blocks and a ragged one) with the uniforms from numpy's Philox."""
    rng = np.random.default_rng(8)
    B, K, V, C = 64, 3, 1100, 0.4
    zp, zq, F, ids, mass, Z, qp, ps, qs = _setup(orc, rng, B, K, V, T, C)
    seed, rnd = 99, 3
    d, _ = orc.draft_sample(zq, T, F, ids, Z, C, seed, rnd)
    acc, aprob, err, exc = orc.verify(zp, zq, T, d, ps, qs, F, ids, Z, C, seed, rnd)
    assert np.all(err == 0)
    bonus, zr, resid, err2, exc2 = orc.residual_sample(zp, zq, T, ps, qs, F, ids, Z, C, acc, seed, rnd,
                                                       want_resid=True)
    p = ps[3]
    n_rej = 0
    for b in range(B):
        k = acc[b]
        w = resid[b]
        assert np.all(w >= 0)
        np.testing.assert_allclose(w.sum(), zr[b], rtol=1e-12)
        if k < K:
            n_rej += 1
            ref = np.maximum(p[b, k] - qp[b, k], 0.0)
            np.testing.assert_allclose(w, ref, atol=1e-15)
            assert w[d[b, k]] == 0.0
            assert bonus[b] != d[b, k]
        else:
            np.testing.assert_allclose(w, p[b, K], atol=1e-15)
        j = _two_level(w, _u_np(seed, rnd, orc.PURPOSE_BONUS, b, k, 0), _u_np(seed, rnd, orc.PURPOSE_BONUS, b, k, 1))
        if not (exc2[b] & orc.E2_CDF_TIE):
            assert bonus[b] == j
    assert n_rej > 10
    assert len(set((bonus // 512).tolist())) == 3


def test_residual_greedy_and_bad_len(orc):
    """At T = 0 the bonus is argmax p_k; an accepted length outside [0, K] is an
    error with bonus -1."""
    rng = np.random.default_rng(9)
    B, K, V = 5, 2, 30
    zp, zq, F, ids, mass, Z, qp, ps, qs = _setup(orc, rng, B, K, V, 0.0, 0.5)
    acc = np.array([0, 1, 2, 3, -1], dtype=np.int32)
    bonus, zr, _, err, _ = orc.residual_sample(zp, zq, 0.0, ps, qs, F, ids, Z, 0.5, acc, 1, 1)
    for b in range(3):
        assert bonus[b] == np.argmax(zp[b, acc[b]])
    assert bonus[3] == -1 and bonus[4] == -1
    assert err[3] == orc.ERR_LEN_RANGE and err[4] == orc.ERR_LEN_RANGE


def test_draft_sampler_searchsorted(orc):
    """P9 for the draft sampler: d_i is the two-level draw from q'_i by np.searchsorted
    (V = 1300: two whole blocks of 512 and a ragged one)."""
    rng = np.random.default_rng(10)
    B, K, V, T, C = 20, 3, 1300, 1.0, 0.5
    zp, zq, F, ids, mass, Z, qp, ps, qs = _setup(orc, rng, B, K, V, T, C)
    d, flags = orc.draft_sample(zq, T, F, ids, Z, C, 5, 6)
    for b in range(B):
        for i in range(K):
            j = _two_level(qp[b, i], _u_np(5, 6, orc.PURPOSE_DRAFT, b, i, 0), _u_np(5, 6, orc.PURPOSE_DRAFT, b, i, 1))
            if not flags[b, i]:
                assert d[b, i] == j
    assert len(set((d // 512).ravel().tolist())) == 3
    dg, _ = orc.draft_sample(zq, 0.0, F, ids, Z, C, 5, 6)
    assert np.array_equal(dg, np.argmax(zq[:, :K], -1))


# --------------------------------------------------------------------------- verify
def test_verify_bruteforce(orc):
    """Accepted length is the first i with u_i >= p_i(d_i)/q'_i(d_i) (python loop over
    the oracle's own probabilities and numpy's Philox words); accept_prob =
    min(1, ratio); bad tokens are errors that reject."""
    rng = np.random.default_rng(11)
    B, K, V, T, C, seed, rnd = 40, 4, 25, 1.0, 0.5, 7, 11
    zp, zq, F, ids, mass, Z, qp, ps, qs = _setup(orc, rng, B, K, V, T, C)
    d = rng.integers(0, V, size=(B, K)).astype(np.int32)
    d[3, 2] = V + 5
    d[4, 0] = -1
    acc, aprob, err, exc = orc.verify(zp, zq, T, d, ps, qs, F, ids, Z, C, seed, rnd)
    p = ps[3]
    for b in range(B):
        k = K
        for i in range(K):
            x = d[b, i]
            if not (0 <= x < V):
                ratio, ok = 0.0, False
            else:
                ratio, ok = p[b, i, x] / qp[b, i, x], True
            bg = np.random.Philox(key=np.array([seed, 0], dtype=np.uint64),
                                  counter=np.array([rnd - 1, b, i, 0], dtype=np.uint64))
            u = (int(bg.random_raw(1)[0]) >> 40) / 2.0**24
            np.testing.assert_allclose(aprob[b, i], min(1.0, ratio), rtol=1e-12)
            if k == K and not (ok and u < ratio):
                k = i
        if not (exc[b] & orc.E1_ACCEPT_TIE):
            assert acc[b] == k
    assert err[3] == orc.ERR_TOKEN_RANGE and err[4] == orc.ERR_TOKEN_RANGE
    assert acc[4] == 0


def test_verify_greedy(orc):
    """T = 0: accept iff d_i = argmax p_i."""
    rng = np.random.default_rng(12)
    B, K, V = 30, 4, 6
    zp, zq, F, ids, mass, Z, qp, ps, qs = _setup(orc, rng, B, K, V, 0.0, 0.5)
    ap = np.argmax(zp, -1)
    d = np.where(rng.random((B, K)) < 0.7, ap[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    acc, aprob, err, _ = orc.verify(zp, zq, 0.0, d, ps, qs, F, ids, Z, 0.5, 1, 1)
    for b in range(B):
        k = next((i for i in range(K) if d[b, i] != ap[b, i]), K)
        assert acc[b] == k
        assert aprob[b].tolist() == [1.0 if d[b, i] == ap[b, i] else 0.0 for i in range(K)]


# --------------------------------------------------------------------------- lookup
def test_lookup_bruteforce(orc):
    """P12: hit = bonus in S_k by set membership, slot = O_k + position; uniform
    fallback = (U32 * V) >> 32 on a miss, -1 otherwise."""
    rng = np.random.default_rng(13)
    B, K, V = 200, 3, 20
    F = np.array([5, 3, 2, 0], dtype=np.int32)
    Bf = int(F.sum())
    ids = np.stack([rng.permutation(V)[:Bf] for _ in range(B)]).astype(np.int32)
    acc = rng.integers(0, K + 1, B).astype(np.int32)
    bonus = rng.integers(0, V, B).astype(np.int32)
    for mode in (0, 1):
        hit, slot, fb, err = orc.cache_lookup(K, V, F, ids, acc, bonus, mode, 3, 4)
        O = np.concatenate([[0], np.cumsum(F)])
        for b in range(B):
            S = ids[b, O[acc[b]]:O[acc[b] + 1]].tolist()
            h = bonus[b] in S
            assert hit[b] == h
            assert slot[b] == (O[acc[b]] + S.index(bonus[b]) if h else -1)
            for j in range(K):
                if h or not mode:
                    assert fb[b, j] == -1
                else:
                    u32 = orc.uniform_u32(3, 4, orc.PURPOSE_FALLBACK, b, j)
                    assert fb[b, j] == (u32 * V) >> 32
                    assert 0 <= fb[b, j] < V
        assert np.all(err == 0)
    assert 0 < hit.sum() < B


def test_cache_gather_matches_fancy_indexing(orc):
    """Pin of the next-draft gather: on a hit the cached continuation
    values[b, slot[b], :], on a miss the fallback tokens; a hit with a slot outside
    [0, Bf) is flagged and yields -1 (numpy fancy indexing as the reference)."""
    rng = np.random.default_rng(11)
    B, Bf, K = 40, 24, 6
    values = rng.integers(0, 50000, size=(B, Bf, K), dtype=np.int32)
    hit = (rng.random(B) < 0.5).astype(np.uint8)
    slot = np.where(hit == 1, rng.integers(0, Bf, size=B), -1).astype(np.int32)
    fb = rng.integers(-1, 50000, size=(B, K), dtype=np.int32)
    bad = [3, 7]
    hit[bad] = 1
    slot[3], slot[7] = Bf, -2
    nd, err = orc.cache_gather(values, hit, slot, fb)
    ok = (hit == 1) & (slot >= 0) & (slot < Bf)
    expect = np.where(ok[:, None], values[np.arange(B), np.clip(slot, 0, Bf - 1)], fb)
    expect[(hit == 1) & ~ok] = -1
    assert np.array_equal(nd, expect)
    assert np.array_equal(err != 0, (hit == 1) & ~ok)
    assert np.all(err[(hit == 1) & ~ok] == orc.ERR_SLOT_RANGE)


# --------------------------------------------------------------------------- fan-out statistics
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bonus_rank_is_sorted_position(orc, dtype):
    """Pin of the bonus rank: the position of the bonus token in draft row k sorted
    by numpy lexsort (logit descending, id ascending), with heavy ties (coarse
    logits), -inf entries and invalid (k, bonus) pairs; the histogram is numpy's
    add.at of the capped ranks."""
    rng = np.random.default_rng(21)
    B, K, V, R = 60, 3, 97, 10
    z = np.round(rng.standard_normal((B, K + 1, V)) * 2.0) / 2.0
    z[rng.random(z.shape) < 0.05] = -np.inf
    z = z.astype(np.float32)
    if dtype == "bf16":
        z = (z.view(np.uint32) >> 16).astype(np.uint16)  # exact: the values have short mantissas
    acc = rng.integers(-1, K + 2, B).astype(np.int32)
    bon = rng.integers(-2, V + 2, B).astype(np.int32)
    hist0 = rng.integers(0, 5, (K + 1, R + 1)).astype(np.uint32)
    rank, hist = orc.bonus_rank(z, acc, bon, R, hist=hist0.copy())
    zw = _widen(z)
    expect_hist = hist0.copy()
    for b in range(B):
        k, t = acc[b], bon[b]
        if not (0 <= k <= K and 0 <= t < V):
            assert rank[b] == -1
            continue
        order = np.lexsort((np.arange(V), -zw[b, k]))
        pos = int(np.nonzero(order == t)[0][0])
        assert rank[b] == pos, (b, k, t)
        np.add.at(expect_hist, (k, min(pos, R)), 1)
    assert np.array_equal(hist, expect_hist)
    assert (rank >= 0).sum() > B // 3


def test_bonus_rank_agrees_with_cache_membership(orc):
    """rank < F_k exactly when the token is among the F_k cached ids of row k (the
    cache build is an independent sort of the same row)."""
    rng = np.random.default_rng(22)
    B, K, V = 12, 4, 300
    z = _rand_logits(rng, B, K, V, dtype="bf16")
    F = np.array([9, 5, 3, 2, 1], np.int32)
    ids, _ = orc.build_cache(z, 1.0, F)
    O = np.concatenate([[0], np.cumsum(F)])
    for k in range(K + 1):
        for trial in range(6):
            tok = rng.integers(0, V, B).astype(np.int32)
            if trial % 2:
                tok = ids[:, O[k] + rng.integers(0, F[k])] if F[k] else tok
            rank, _ = orc.bonus_rank(z, np.full(B, k, np.int32), tok, 64)
            for b in range(B):
                assert (rank[b] < F[k]) == (tok[b] in ids[b, O[k]:O[k + 1]]), (k, b)


def _brute_fanout(hist, Bf, Fmax):
    K1, R1 = hist.shape
    cap = min(Fmax, R1 - 1)
    best, arg = None, None
    for F in itertools.product(range(cap + 1), repeat=K1):
        if sum(F) != Bf:
            continue
        v = sum(int(hist[k, :F[k]].sum()) for k in range(K1))
        if best is None or v > best or (v == best and F > arg):
            best, arg = v, F
    return arg, best


def test_fanout_optimize_brute_force(orc):
    """Pin of the fan-out optimiser: exhaustive search over every composition of Bf
    (the same objective, the same lexicographic rule among maximisers)."""
    rng = np.random.default_rng(23)
    n = 0
    for K1 in (1, 2, 3, 4):
        for R in (1, 3, 5):
            for Fmax in (2, 4, 8):
                cap = min(Fmax, R)
                for Bf in sorted({0, 1, cap, K1 * cap // 2, K1 * cap}):
                    hist = rng.integers(0, 6, (K1, R + 1)) * (rng.random((K1, R + 1)) < 0.7)
                    F, hits, total = orc.fanout_optimize(hist, Bf, Fmax)
                    aF, ahits = _brute_fanout(hist, Bf, Fmax)
                    assert tuple(int(x) for x in F) == aF, (K1, R, Fmax, Bf, hist)
                    assert hits == ahits and total == int(hist.sum())
                    n += 1
    assert n > 100
    assert orc.fanout_optimize(np.ones((3, 5)), 13, 4) is None
    assert orc.fanout_optimize(np.ones((3, 5)), -1, 4) is None


def test_fanout_optimize_special_cases(orc):
    """No data: the budget fills the shortest lengths first.  A coverage that falls
    off geometrically in both k and rank (every marginal distinct): the optimum
    equals greedy allocation by largest marginal, which is exact for concave
    coverage."""
    F, hits, total = orc.fanout_optimize(np.zeros((4, 9), np.int64), 13, 6)
    assert F.tolist() == [6, 6, 1, 0] and hits == 0 and total == 0
    K1, R, Bf, Fmax = 9, 64, 64, 64
    hist = np.array([[int(1e9 * 0.6 ** k * 0.83 ** j) + 3 * k + 7 * j for j in range(R + 1)]
                     for k in range(K1)], np.int64)
    F, hits, _ = orc.fanout_optimize(hist, Bf, Fmax)
    g = np.zeros(K1, int)
    for _ in range(Bf):
        k = max(range(K1), key=lambda k: hist[k, g[k]] if g[k] < min(R, Fmax) else -1)
        g[k] += 1
    assert hits == sum(int(hist[k, :g[k]].sum()) for k in range(K1))
    assert F.tolist() == g.tolist()
    assert F.sum() == Bf and np.all(np.diff(F) <= 0)


# --------------------------------------------------------------------------- fallback policy
def _model(**kw):
    m = dict(t_verify=1.0, t_primary=0.8, t_random=0.05, n_hit=3.0, n_primary=3.0, n_random=1.2)
    m.update(kw)
    return m


def test_fallback_no_miss_is_a_tie(orc):
    """h = 1 for every sequence: no round waits and both fallbacks deliver n_hit per
    sequence, so the throughputs are equal (B n_hit / t_verify) and the tie keeps
    the primary speculator."""
    m = _model()
    c, tp, tr = orc.fallback_choose(m, [1.0] * 17)
    assert c == orc.FALLBACK_NONE and tp == tr == 17 * 3.0 / 1.0


def test_fallback_closed_form_values(orc):
    """Throughputs written out by hand for B = 2, h = (0.5, 0.75)."""
    m = _model(t_verify=2.0, t_primary=1.0, t_random=0.25, n_hit=4.0, n_primary=3.0, n_random=1.0)
    c, tp, tr = orc.fallback_choose(m, [0.5, 0.75])
    p_miss = 1 - 0.375
    assert tp == pytest.approx((1.25 * 4 + 0.75 * 3) / (2 + p_miss * 1.0), rel=1e-15)
    assert tr == pytest.approx((1.25 * 4 + 0.75 * 1) / (2 + p_miss * 0.25), rel=1e-15)
    assert c == (orc.FALLBACK_UNIFORM if tr > tp else orc.FALLBACK_NONE)


def test_fallback_critical_batch_closed_form(orc):
    """With n_primary = n_hit = n, n_random = 0 and t_random = 0, random tokens win
    exactly when h^b < 1 - t_verify (1 - h) / (h t_primary), so
    b* = floor(ln(1 - t_verify (1 - h) / (h t_primary)) / ln h) + 1."""
    import math
    for h, tv, tpri in ((0.9, 1.0, 3.0), (0.97, 0.5, 4.0), (0.8, 1.0, 10.0), (0.995, 1.0, 2.5)):
        m = _model(t_verify=tv, t_primary=tpri, t_random=0.0, n_hit=2.0, n_primary=2.0, n_random=0.0)
        x = math.log(1 - tv * (1 - h) / (h * tpri)) / math.log(h)
        assert abs(x - round(x)) > 1e-6  # away from a boundary
        assert orc.fallback_critical_batch(m, h, 5000) == math.floor(x) + 1
    # a primary fallback that costs nothing is never beaten
    assert orc.fallback_critical_batch(_model(t_primary=0.0), 0.9, 500) == 0
