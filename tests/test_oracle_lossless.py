"""The lossless invariant and the acceptance laws, pinned on the oracle by exact
enumeration on tiny vocabularies and by Monte Carlo through the whole oracle round.

The summaries of "Speculative Speculative Decoding" (gist.science zh, technical
part, opening paragraph and section 5; the nl summary's conclusion) state that the
round is lossless: the emitted tokens follow the target law p.  With the draft
sampling from its Saguaro-reweighted law q', that means: conditioned on having
accepted the prefix t_0..t_{n-2}, the n-th emitted token follows p_{n-1}.
CPU only."""
import itertools

import numpy as np
import pytest


def _case(orc, rng, V, K, T, C, Bf, r):
    zq = (rng.standard_normal((1, K + 1, V)) * 1.5).astype(np.float32)
    zp = (zq + rng.standard_normal((1, K + 1, V)) * 1.2).astype(np.float32)
    F, _ = orc.fanout(K, Bf, r)
    F = np.minimum(F, V).astype(np.int32)  # a tiny vocabulary caps each share
    ids, mass = orc.build_cache(zq, T, F)
    Z, qp = orc.saguaro(zq, T, F, ids, mass, C, want_qprime=True)
    ps = orc.softmax(zp, T, want_probs=True)
    qs = orc.softmax(zq, T, want_probs=True)
    return zp, zq, F, ids, Z, qp[0], ps, qs


def _accept_probs(orc, zp, zq, T, ps, qs, F, ids, Z, C, K, V):
    """a[i, x] = min(1, p_i(x)/q'_i(x)) as the oracle's verify reports it."""
    a = np.zeros((K, V))
    for x in range(V):
        d = np.full((1, K), x, dtype=np.int32)
        _, aprob, _, _ = orc.verify(zp, zq, T, d, ps, qs, F, ids, Z, C, 0, 0)
        a[:, x] = aprob[0]
    return a


def _residual_laws(orc, zp, zq, T, ps, qs, F, ids, Z, C, K, V):
    """res[k] = the oracle's bonus law at accepted length k (w / Z_r)."""
    res = np.zeros((K + 1, V))
    for k in range(K + 1):
        _, zr, w, _, _ = orc.residual_sample(zp, zq, T, ps, qs, F, ids, Z, C,
                                              np.array([k], np.int32), 0, 0, want_resid=True)
        res[k] = w[0] / zr[0]
    return res


CASES = [(V, K, T, C) for V in (2, 3, 5) for K in (1, 2, 3) for T in (1.0, 0.6) for C in (0.3, 1.0)]


@pytest.mark.parametrize("V,K,T,C", CASES)
def test_lossless_exact_enumeration(orc, V, K, T, C):
    """P2: exact law of the emitted tokens, enumerating every draft block in V^K
    (probability prod q'_i(d_i)), every accepted length and every bonus token:
      P(round emits >= n tokens, first n = t) =
          prod_{i<n-1} min(p_i(t_i), q'_i(t_i)) * p_{n-1}(t_{n-1})."""
    rng = np.random.default_rng(1000 * V + 10 * K + int(10 * T) + int(10 * C))
    zp, zq, F, ids, Z, qp, ps, qs = _case(orc, rng, V, K, T, C, Bf=2 * V, r=0.7)
    p = ps[3][0]
    a = _accept_probs(orc, zp, zq, T, ps, qs, F, ids, Z, C, K, V)
    res = _residual_laws(orc, zp, zq, T, ps, qs, F, ids, Z, C, K, V)
    # law over emitted token tuples of each length n = k + 1
    law = {}
    for d in itertools.product(range(V), repeat=K):
        pd = np.prod([qp[i, d[i]] for i in range(K)])
        reach = 1.0
        for k in range(K + 1):
            if k < K:
                stop = reach * (1.0 - a[k, d[k]])
            else:
                stop = reach
            for y in range(V):
                t = tuple(d[:k]) + (y,)
                law[t] = law.get(t, 0.0) + pd * stop * res[k, y]
            if k < K:
                reach *= a[k, d[k]]
    # P(emits >= n and prefix t) = sum over emitted tuples extending t
    for n in range(1, K + 2):
        for t in itertools.product(range(V), repeat=n):
            got = sum(v for tt, v in law.items() if len(tt) >= n and tt[:n] == t)
            want = np.prod([min(p[i, t[i]], qp[i, t[i]]) for i in range(n - 1)]) * p[n - 1, t[n - 1]]
            assert abs(got - want) < 1e-12, (n, t, got, want)
    assert abs(sum(law.values()) - 1.0) < 1e-12


def test_lossless_monte_carlo_whole_round(orc):
    """P2 / P3 / P4 by sampling the whole oracle round with its Philox uniforms:
    first emitted token ~ p_0 (chi-square), E[accept_i | reached i] = sum_x
    min(p_i, q'_i), and P(k = j) = prod_{i<j} alpha_i (1 - alpha_j)."""
    from scipy import stats
    rng = np.random.default_rng(77)
    V, K, T, C, N = 8, 3, 1.0, 0.5, 60000
    zq1 = (rng.standard_normal((1, K + 1, V)) * 1.5).astype(np.float32)
    zp1 = (zq1 + rng.standard_normal((1, K + 1, V)) * 1.0).astype(np.float32)
    zq = np.ascontiguousarray(np.broadcast_to(zq1, (N, K + 1, V)))
    zp = np.ascontiguousarray(np.broadcast_to(zp1, (N, K + 1, V)))
    F, gap = orc.fanout(K, 6, 0.6)
    ids, mass = orc.build_cache(zq, T, F)
    Z, _ = orc.saguaro(zq, T, F, ids, mass, C)
    seed, rnd = 0xABC, 5
    d, _ = orc.draft_sample(zq, T, F, ids, Z, C, seed, rnd)
    out = orc.round_(zp, zq, T, F, C, d, seed, rnd, False, gap)
    p = orc.softmax(zp1, T, want_probs=True)[3][0]
    _, qp1 = orc.saguaro(zq1, T, F, ids[:1], mass[:1], C, want_qprime=True)
    qp1 = qp1[0]
    alpha = np.minimum(p, qp1).sum(-1)
    k = out.accept_len
    t0 = np.where(k >= 1, d[:, 0], out.bonus)
    obs = np.bincount(t0, minlength=V)
    exp_ = p[0] * N
    keep = exp_ > 5
    chi = ((obs[keep] - exp_[keep]) ** 2 / exp_[keep]).sum()
    assert stats.chi2.sf(chi, keep.sum() - 1) > 1e-4
    for i in range(K):
        reached = k >= i
        acc = (k[reached] > i).mean()
        n = reached.sum()
        sd = np.sqrt(alpha[i] * (1 - alpha[i]) / n)
        assert abs(acc - alpha[i]) < 4.5 * sd
    for j in range(K + 1):
        pj = np.prod(alpha[:j]) * ((1 - alpha[j]) if j < K else 1.0)
        sd = np.sqrt(pj * (1 - pj) / N)
        assert abs((k == j).mean() - pj) < 4.5 * sd
    # each emitted token at a later position, given it was reached, also follows p
    for i in range(1, K + 1):
        reached = k >= i
        ti = np.where(k[reached] > i, d[reached, i] if i < K else -1, out.bonus[reached])
        obs = np.bincount(ti, minlength=V)
        exp_ = p[i] * reached.sum()
        keep = exp_ > 5
        chi = ((obs[keep] - exp_[keep]) ** 2 / exp_[keep]).sum()
        assert stats.chi2.sf(chi, keep.sum() - 1) > 1e-4
    assert np.all(out.err == 0)


def test_saguaro_tradeoff_direction(orc):
    """Lowering C moves residual mass onto the cached tokens (the pages' stated
    purpose of Saguaro sampling) and lowers acceptance sum min(p, q')."""
    rng = np.random.default_rng(78)
    V, K, T = 64, 2, 1.0
    zq = (rng.standard_normal((1, K + 1, V)) * 2.0).astype(np.float32)
    zp = (zq + rng.standard_normal((1, K + 1, V)) * 1.0).astype(np.float32)
    F, _ = orc.fanout(K, 12, 0.7)
    ids, mass = orc.build_cache(zq, T, F)
    ps = orc.softmax(zp, T, want_probs=True)
    qs = orc.softmax(zq, T, want_probs=True)
    p = ps[3][0]
    prev_hit, prev_alpha = -1.0, 2.0
    for C in (1.0, 0.7, 0.4, 0.1):
        Z, qp = orc.saguaro(zq, T, F, ids, mass, C, want_qprime=True)
        alpha = np.minimum(p[0], qp[0, 0]).sum()
        _, zr, w, _, _ = orc.residual_sample(zp, zq, T, ps, qs, F, ids, Z, C, np.array([0], np.int32),
                                              0, 0, want_resid=True)
        hit = w[0, ids[0, :F[0]]].sum() / zr[0]
        assert hit >= prev_hit - 1e-12 and alpha <= prev_alpha + 1e-12
        prev_hit, prev_alpha = hit, alpha
