"""Parity of the HIP path (called through the C ABI) with the fp64 oracle on seeded
synthetic inputs.  Each test prints what names its case before the GPU step."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import lossless_rejection_sampling_ssd_amd as ssd
from lossless_rejection_sampling_ssd_amd.workloads import to_oracle_array

from gpu_helpers import PROB_ATOL, SUM_RTOL, compare_round, gpu_round, oracle_draft
import parity_cases as pc
from parity_cases import rand_logits as _rand

with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "flag_counts.json")) as _fh:
    FLAGS = json.load(_fh)["cases"]


def _check_flags(label, flagged):
    """The number of sequences the oracle flagged equals the stored count
    (tests/golden/flag_counts.json, written from the oracle alone)."""
    assert flagged == FLAGS[label]["flagged"], (label, flagged, FLAGS[label])

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def _case(msg):
    print("\n[case] " + msg, flush=True)


def _to_dev(z):
    """Device copy keeping the row stride of a padded view."""
    if z.is_contiguous():
        return z.cuda()
    B, K1, V = z.shape
    ld = z.stride(1)
    base = torch.empty((B, K1, ld), dtype=z.dtype)
    base[:, :, :V] = z
    base[:, :, V:] = float("nan")
    return base.cuda()[:, :, :V]


# ----------------------------------------------------------------------------- softmax
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,pad", [(7, 0), (1000, 0), (4099, 0), (20011, 0), (33000, 8), (5003, 3)])
@pytest.mark.parametrize("T", [0.0, 0.7, 1.0])
def test_softmax(dtype, V, pad, T):
    _case("softmax dtype=%s V=%d pad=%d T=%g" % (dtype, V, pad, T))
    B, K = 3, 2
    zq, zp = _rand(B, K, V, dtype, 11 + V, ld=V + pad if pad else None)
    z = _to_dev(zp)
    shape = ssd.shape_of(z, T)
    R = B * (K + 1)
    m = torch.zeros(R, device="cuda")
    s = torch.zeros(R, dtype=torch.float64, device="cuda")
    a = torch.zeros(R, dtype=torch.int32, device="cuda")
    probs = torch.zeros((B, K + 1, V), device="cuda")
    ssd.ssd_softmax(shape, z, m, s, a, probs)
    torch.cuda.synchronize()
    om, os_, oa, op = oracle.softmax(to_oracle_array(zp), T, want_probs=True)
    assert np.array_equal(m.cpu().numpy(), om.reshape(R).astype(np.float32))
    np.testing.assert_allclose(s.cpu().numpy(), os_.reshape(R), rtol=SUM_RTOL)
    assert np.array_equal(a.cpu().numpy(), oa.reshape(R))
    np.testing.assert_allclose(probs.cpu().numpy(), op, atol=PROB_ATOL, rtol=0)


# ----------------------------------------------------------------------------- cache
def _gpu_stats(z, T):
    shape = ssd.shape_of(z, T)
    R = shape.B * (shape.K + 1)
    m = torch.zeros(R, device="cuda")
    s = torch.zeros(R, dtype=torch.float64, device="cuda")
    a = torch.zeros(R, dtype=torch.int32, device="cuda")
    ssd.ssd_softmax(shape, z, m, s, a)
    return m, s, a


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V,F,kind", [
    (5000, [20, 14, 10, 7, 5], "gauss"),
    (5000, [64, 0, 3, 1, 0], "gauss"),
    (128256, [24, 19, 16, 13, 10], "quantised"),
    (3000, [40, 30, 20, 10, 5], "constant"),
    (128256, [30, 2, 1, 0, 1], "constant"),   # ties across many tiles: whole-key select
    (128256, [64, 40, 1, 0, 2], "gauss"),     # more candidates than register slots
    (9, [9, 4, 1, 0, 2], "gauss"),
    (20011, [1, 1, 1, 1, 1], "neginf"),
])
@pytest.mark.parametrize("T", [0.0, 1.0])
def test_build_cache(dtype, V, F, kind, T):
    _case("build_cache dtype=%s V=%d F=%s kind=%s T=%g" % (dtype, V, F, kind, T))
    B, K = 2, len(F) - 1
    zq, _ = _rand(B, K, V, dtype, 5 + V)
    if kind == "quantised":
        zq = (zq * 2).round() / 2          # many equal values: ties broken by id
    elif kind == "constant":
        zq = torch.full_like(zq, 1.25)     # every id ties: exact slow path
    elif kind == "neginf":
        zq[:, :, ::3] = float("-inf")
    z = zq.cuda()
    m, s, a = _gpu_stats(z, T)
    Bf = sum(F)
    ids = torch.zeros((B, Bf), dtype=torch.int32, device="cuda")
    mass = torch.zeros(B * (K + 1), dtype=torch.float64, device="cuda")
    ssd.ssd_build_cache(ssd.shape_of(z, T), z, m, s, F, ids, mass)
    torch.cuda.synchronize()
    oids, omass = oracle.build_cache(to_oracle_array(zq), T, np.array(F, np.int32))
    assert np.array_equal(ids.cpu().numpy(), oids)
    np.testing.assert_allclose(mass.cpu().numpy(), omass.reshape(-1), atol=PROB_ATOL, rtol=0)


# ----------------------------------------------------------------------------- Saguaro + draft
def _saguaro_draft_case(dtype, T, C, V, B, K, F):
    zq, _ = _rand(B, K, V, dtype, 21)
    z = zq.cuda()
    m, s, a = _gpu_stats(z, T)
    ids = torch.zeros((B, sum(F)), dtype=torch.int32, device="cuda")
    mass = torch.zeros(B * (K + 1), dtype=torch.float64, device="cuda")
    ssd.ssd_build_cache(ssd.shape_of(z, T), z, m, s, F, ids, mass)
    Z = torch.zeros(B * (K + 1), dtype=torch.float64, device="cuda")
    qp = torch.zeros((B, K + 1, V), device="cuda")
    d = torch.zeros((B, K), dtype=torch.int32, device="cuda")
    ssd.ssd_saguaro_reweight(ssd.shape_of(z, T), mass, C, Z, z, m, s, a, F, ids, qp, seed=77, round_=5, draft=d)
    torch.cuda.synchronize()
    zq_np = to_oracle_array(zq)
    oids, omass = oracle.build_cache(zq_np, T, np.array(F, np.int32))
    oZ, oqp = oracle.saguaro(zq_np, T, np.array(F, np.int32), oids, omass, C, want_qprime=True)
    np.testing.assert_allclose(Z.cpu().numpy(), oZ.reshape(-1), atol=PROB_ATOL, rtol=0)
    np.testing.assert_allclose(qp.cpu().numpy(), oqp, atol=PROB_ATOL, rtol=0)
    od, flags = oracle.draft_sample(zq_np, T, np.array(F, np.int32), oids, oZ, C, 77, 5)
    ok = flags == 0
    assert np.array_equal(d.cpu().numpy()[ok], od[ok])
    return int((~ok).sum())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,C", [(1.0, 0.5), (0.7, 0.2), (1.0, 1.0), (0.0, 0.5)])
def test_saguaro_and_draft(dtype, T, C):
    _case("saguaro dtype=%s T=%g C=%g" % (dtype, T, C))
    _saguaro_draft_case(dtype, T, C, 6007, 8, 3, [6, 3, 2, 1])


def test_draft_sampling_large_grid():
    """Draft sampling over 64 sequences x 8 positions of 20 pass-2 tiles each (10,240
    tiles, above the size from which pass 2 weighs every element as uncached first and
    the cached ids again), against the oracle."""
    _case("draft sampling, large grid")
    flagged = _saguaro_draft_case("bf16", 1.0, 0.5, 40000, 64, 8, [8, 4, 3, 2, 2, 1, 1, 1, 1])
    assert flagged == 0  # the oracle flags none of these 512 draws, so every one is compared


# ----------------------------------------------------------------------------- chain of the six calls
def _chain(zp, zq, T, F, C, draft, seed, rnd, fallback):
    """The six separate calls in the method's order (GPU)."""
    shape = ssd.shape_of(zp, T)
    B, K = shape.B, shape.K
    R = B * (K + 1)
    Bf = sum(F)
    pm, ps, pa = _gpu_stats(zp, T)
    qm, qs, qa = _gpu_stats(zq, T)
    ids = torch.zeros((B, max(Bf, 1)), dtype=torch.int32, device="cuda")
    mass = torch.zeros(R, dtype=torch.float64, device="cuda")
    ssd.ssd_build_cache(shape, zq, qm, qs, F, ids, mass)
    Z = torch.zeros(R, dtype=torch.float64, device="cuda")
    ssd.ssd_saguaro_reweight(shape, mass, C, Z)
    d = torch.as_tensor(np.ascontiguousarray(draft), dtype=torch.int32, device="cuda")
    acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    aprob = torch.zeros((B, K), device="cuda")
    err = torch.zeros(B, dtype=torch.int32, device="cuda")
    ssd.ssd_verify(shape, zp, zq, d, pm, ps, pa, qm, qs, F, ids, Z, C, seed, rnd, acc, aprob, err)
    bonus = torch.zeros(B, dtype=torch.int32, device="cuda")
    zr = torch.zeros(B, dtype=torch.float64, device="cuda")
    ssd.ssd_residual_sample(shape, zp, zq, pm, ps, pa, qm, qs, F, ids, Z, C, acc, seed, rnd, bonus, zr, err)
    hit = torch.zeros(B, dtype=torch.uint8, device="cuda")
    slot = torch.zeros(B, dtype=torch.int32, device="cuda")
    fb = torch.zeros((B, K), dtype=torch.int32, device="cuda")
    ssd.ssd_cache_lookup(B, K, shape.V, F, ids, acc, bonus, fallback, seed, rnd, hit, slot, fb, err)
    torch.cuda.synchronize()
    out = {"p_max": pm, "p_sum": ps, "p_argmax": pa, "q_max": qm, "q_sum": qs, "q_argmax": qa, "cache_ids": ids,
           "cache_mass": mass, "Z": Z, "accept_len": acc, "accept_prob": aprob, "bonus": bonus, "resid_mass": zr,
           "hit": hit, "slot": slot, "fallback_tokens": fb, "dev_err": err}
    return {k: v.cpu().numpy() for k, v in out.items()}


ROUND_CASES = [
    # (label, dtype, B, K, V, T, F, C, fallback, scale, noise)
    ("c1-like", "f32", 1, 4, 32000, 1.0, [6, 4, 3, 2, 1], 0.5, 0, 2.0, 0.7),
    ("c2-greedy", "f32", 16, 5, 32000, 0.0, [13, 8, 5, 3, 2, 1], 0.3, 0, 2.5, 0.8),
    ("c2-T0.7", "f32", 16, 5, 32000, 0.7, [13, 8, 5, 3, 2, 1], 0.3, 0, 2.5, 0.8),
    ("c3-small", "bf16", 12, 8, 40000, 1.0, [20, 14, 10, 7, 5, 3, 2, 2, 1], 0.5, 0, 3.0, 1.0),
    ("c5-small", "bf16", 24, 4, 151936, 1.0, [17, 8, 4, 2, 1], 0.5, 1, 2.0, 1.5),
    ("ragged", "bf16", 5, 2, 4101, 1.3, [9, 0, 4], 0.8, 1, 2.0, 0.6),
    ("tiny-V", "f32", 7, 3, 5, 1.0, [2, 1, 1, 1], 0.4, 1, 1.0, 0.5),
    ("K=1", "f32", 9, 1, 777, 0.9, [3, 2], 0.5, 1, 2.0, 0.5),
    ("Bf=0", "bf16", 4, 3, 3000, 1.0, [0, 0, 0, 0], 1.0, 1, 2.0, 0.8),
    ("K=16", "f32", 3, 16, 2000, 1.0, [4] * 17, 0.6, 0, 2.0, 0.3),
]


@pytest.mark.parametrize("case", ROUND_CASES, ids=[c[0] for c in ROUND_CASES])
def test_round_vs_oracle_and_chain(case):
    label, dtype, B, K, V, T, F, C, fb, scale, noise = case
    _case("round " + label)
    zq, zp = _rand(B, K, V, dtype, sum(map(ord, label)), scale, noise)
    seed, rnd = 0x1234 + B, 9
    zp_np, zq_np = to_oracle_array(zp), to_oracle_array(zq)
    draft, _ = oracle_draft(zp_np, zq_np, T, np.array(F, np.int32), C, seed, rnd)
    o = oracle.round_(zp_np, zq_np, T, np.array(F, np.int32), C, draft, seed, rnd, fb)
    zpd, zqd = zp.cuda(), zq.cuda()
    values = np.random.default_rng(B + K).integers(0, V, (B, sum(F), K)).astype(np.int32)
    g = gpu_round(zpd, zqd, T, F, C, draft, seed, rnd, fb, values=values)
    compare_round(g, o, K, sum(F), label=label, values=values)
    ch = _chain(zpd, zqd, T, F, C, draft, seed, rnd, fb)
    for k in ch:
        a, b = g[k], ch[k]
        if k == "cache_ids":
            a, b = a[:, :sum(F)], b[:, :sum(F)]
        assert np.array_equal(a, b), (label, k)
    t = lambda x: torch.as_tensor(np.ascontiguousarray(x), device="cuda")  # noqa: E731
    nd = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
    ssd.ssd_cache_gather(t(values), t(ch["hit"]), t(ch["slot"]), t(ch["fallback_tokens"]), nd)
    assert np.array_equal(nd.cpu().numpy(), g["next_draft"]), (label, "next_draft chain")
    g2 = gpu_round(zpd, zqd, T, F, C, draft, seed, rnd, fb, values=values)
    for k in g:
        assert np.array_equal(g[k], g2[k]), ("determinism", label, k)


@pytest.mark.parametrize("label", [c[0] for c in pc.EDGE_CASES])
def test_round_edge_cases(label):
    """The fused round against the oracle at the edges of the method: the largest
    fan-out share, heavy ties, near-greedy and flat temperatures, large logits, and
    rows where every logit is equal; the first and the last draft token forced to
    ids 0 and V - 1."""
    _case("edge " + label)
    c = pc.edge_case(label)
    o = c.oracle_round()
    g_ = gpu_round(c.zp.cuda(), c.zq.cuda(), c.T, c.F, c.C, c.draft, c.seed, c.rnd, c.fallback)
    _check_flags(label, compare_round(g_, o, c.K, sum(c.F), label=label))


def test_forced_paths():
    """All accepted (p = q, C = 1); rejection at position 0 (z_p(d_0) = -inf);
    invalid draft tokens; a bonus that cannot be cached (F = 0) misses."""
    B, K, V, T = 6, 4, 3001, 1.0
    zq, zp = _rand(B, K, V, "f32", 3)
    F = [5, 4, 3, 2, 1]
    zp_same = zq.clone()
    zp_np, zq_np = to_oracle_array(zp_same), to_oracle_array(zq)
    draft, _ = oracle_draft(zp_np, zq_np, T, np.array(F, np.int32), 1.0, 1, 1)
    _case("forced all-accept")
    g = gpu_round(zp_same.cuda(), zq.cuda(), T, F, 1.0, draft, 1, 1, 1)
    o = oracle.round_(zp_np, zq_np, T, np.array(F, np.int32), 1.0, draft, 1, 1, 1)
    compare_round(g, o, K, sum(F), label="all-accept")
    assert np.all(g["accept_len"] == K)
    _case("forced reject at 0")
    zp_rej = zp.clone()
    for b in range(B):
        zp_rej[b, 0, draft[b, 0]] = float("-inf")
    zp_np = to_oracle_array(zp_rej)
    g = gpu_round(zp_rej.cuda(), zq.cuda(), T, F, 0.5, draft, 1, 1, 1)
    o = oracle.round_(zp_np, zq_np, T, np.array(F, np.int32), 0.5, draft, 1, 1, 1)
    compare_round(g, o, K, sum(F), label="reject0")
    assert np.all(g["accept_len"] == 0)
    assert np.all(g["bonus"] != draft[:, 0])
    _case("forced invalid tokens")
    bad = draft.copy()
    bad[1, 0] = -3
    bad[2, 2] = V
    bad[3, 3] = V + 100
    g = gpu_round(zp.cuda(), zq.cuda(), T, F, 0.5, bad, 1, 1, 1)
    o = oracle.round_(to_oracle_array(zp), zq_np, T, np.array(F, np.int32), 0.5, bad, 1, 1, 1)
    compare_round(g, o, K, sum(F), label="invalid")
    assert g["dev_err"][1] & ssd.SSD_DEVERR_TOKEN_RANGE and g["accept_len"][1] == 0


def test_lookup_oracle_fed():
    """ssd_cache_lookup on oracle-made inputs: random caches, lengths (including out
    of range) and bonus tokens."""
    _case("lookup oracle-fed")
    rng = np.random.default_rng(3)
    B, K, V = 300, 4, 50
    F = [6, 4, 3, 0, 2]
    Bf = sum(F)
    ids = np.stack([rng.permutation(V)[:Bf] for _ in range(B)]).astype(np.int32)
    acc = rng.integers(-1, K + 2, B).astype(np.int32)
    bonus = rng.integers(0, V, B).astype(np.int32)
    for mode in (0, 1):
        oh, osl, ofb, oerr = oracle.cache_lookup(K, V, np.array(F, np.int32), ids, acc, bonus, mode, 5, 6)
        t = lambda x: torch.as_tensor(x, device="cuda")  # noqa: E731
        hit = torch.zeros(B, dtype=torch.uint8, device="cuda")
        slot = torch.zeros(B, dtype=torch.int32, device="cuda")
        fb = torch.zeros((B, K), dtype=torch.int32, device="cuda")
        err = torch.zeros(B, dtype=torch.int32, device="cuda")
        ssd.ssd_cache_lookup(B, K, V, F, t(ids), t(acc), t(bonus), mode, 5, 6, hit, slot, fb, err)
        torch.cuda.synchronize()
        assert np.array_equal(hit.cpu().numpy(), oh)
        assert np.array_equal(slot.cpu().numpy(), osl)
        assert np.array_equal(fb.cpu().numpy(), ofb)
        assert np.array_equal(err.cpu().numpy(), oerr)


def test_cache_gather_oracle_fed():
    """ssd_cache_gather on oracle-made inputs: hits, misses with uniform or -1
    fallback tokens, and hits whose slot lies outside [0, Bf)."""
    rng = np.random.default_rng(11)
    for B, K, Bf in ((300, 4, 15), (5, 16, 1), (4, 3, 0), (70000, 8, 40)):
        _case("gather oracle-fed B=%d K=%d Bf=%d" % (B, K, Bf))
        values = rng.integers(0, 128256, (B, Bf, K)).astype(np.int32)
        hit = (rng.random(B) < 0.6).astype(np.uint8) if Bf > 0 else np.zeros(B, np.uint8)
        slot = np.where(hit == 1, rng.integers(-2, Bf + 2, B), -1).astype(np.int32)
        fbt = rng.integers(-1, 128256, (B, K)).astype(np.int32)
        ond, oerr = oracle.cache_gather(values, hit, slot, fbt)
        t = lambda x: torch.as_tensor(np.ascontiguousarray(x), device="cuda")  # noqa: E731
        nd = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
        err = torch.zeros(B, dtype=torch.int32, device="cuda")
        ssd.ssd_cache_gather(t(values), t(hit), t(slot), t(fbt), nd, err)
        torch.cuda.synchronize()
        assert np.array_equal(nd.cpu().numpy(), ond)
        assert np.array_equal(err.cpu().numpy(), oerr)
        assert B < 100 or oerr.any()


RANK_CASES = [
    # (dtype, B, K, V, ld pad, R)
    ("f32", 7, 3, 5000, 0, 16),
    ("bf16", 9, 4, 40013, 5, 64),
    ("bf16", 64, 8, 128256, 0, 64),
    ("f32", 3, 1, 2, 0, 1),
    ("bf16", 5, 16, 4097, 3, 7),
]


@pytest.mark.parametrize("case", RANK_CASES, ids=lambda c: "%s-B%d-K%d-V%d-pad%d-R%d" % c)
def test_bonus_rank_oracle_fed(case):
    """ssd_bonus_rank against the oracle: heavy ties (coarse logits), -inf entries,
    ragged tails, unaligned rows, invalid (k, bonus); the histogram accumulates over
    two calls."""
    dtype, B, K, V, pad, R = case
    _case("bonus rank %s" % (case,))
    rng = np.random.default_rng(B * 7 + V)
    z = np.round(rng.standard_normal((B, K + 1, V + pad)) * 4.0) / 4.0
    z[rng.random(z.shape) < 0.03] = -np.inf
    z = z.astype(np.float32)
    zt = torch.from_numpy(z)
    if dtype == "bf16":
        zt = zt.to(torch.bfloat16)
    zt = zt[:, :, :V]
    z_np = to_oracle_array(zt)
    zd = zt.cuda() if pad == 0 else torch.empty((B, K + 1, V + pad), dtype=zt.dtype, device="cuda")[:, :, :V]
    if pad:
        zd.copy_(zt)
    shape = ssd.shape_of(zd, 1.0)
    hist = torch.zeros((K + 1, R + 1), dtype=torch.int32, device="cuda")
    ohist = np.zeros((K + 1, R + 1), np.uint32)
    for rep in range(2):
        acc = rng.integers(-1, K + 2, B).astype(np.int32)
        bon = rng.integers(-2, V + 2, B).astype(np.int32)
        top = np.argmax(z[:, :, :V], axis=2)  # some bonuses at the top of their row
        for b in range(0, B, 3):
            if 0 <= acc[b] <= K:
                bon[b] = top[b, acc[b]]
        rank = torch.full((B,), -9, dtype=torch.int32, device="cuda")
        ssd.ssd_bonus_rank(shape, zd, torch.as_tensor(acc, device="cuda"), torch.as_tensor(bon, device="cuda"), R,
                           rank, hist)
        torch.cuda.synchronize()
        orank, ohist = oracle.bonus_rank(z_np, acc, bon, R, hist=ohist)
        assert np.array_equal(rank.cpu().numpy(), orank), (case, rep)
        assert np.array_equal(hist.cpu().numpy().astype(np.uint32), ohist), (case, rep)


@pytest.mark.parametrize("B,K,V,dtype", [(4, 3, 999, "f32"), (130, 1, 130072, "bf16")],
                         ids=["small", "two-tile grid"])
def test_residual_bad_len_and_greedy(B, K, V, dtype):
    """ssd_residual_sample with accepted lengths outside [0, K] reports the error and
    returns -1, and leaves every other sequence's bonus as it is with valid lengths
    only; at T = 0 it returns argmax p_k.  The second case (8,320 pass-2 tiles on
    aligned rows) takes the two-tile bonus pass."""
    zq, zp = _rand(B, K, V, dtype, 8)
    F = [3, 2, 1, 1][:K + 1]
    bad = {2: -1, 3: K + 1}  # sequence: accepted length outside [0, K]
    for T in (1.0, 0.0):
        _case("residual bad len %s B=%d T=%g" % (dtype, B, T))
        zpd, zqd = zp.cuda(), zq.cuda()
        pm, ps, pa = _gpu_stats(zpd, T)
        qm, qs, qa = _gpu_stats(zqd, T)
        ids = torch.zeros((B, sum(F)), dtype=torch.int32, device="cuda")
        mass = torch.zeros(B * (K + 1), dtype=torch.float64, device="cuda")
        shape = ssd.shape_of(zpd, T)
        ssd.ssd_build_cache(shape, zqd, qm, qs, F, ids, mass)
        Z = torch.zeros(B * (K + 1), dtype=torch.float64, device="cuda")
        ssd.ssd_saguaro_reweight(shape, mass, 0.5, Z)
        good = torch.arange(B, dtype=torch.int32, device="cuda") % (K + 1)
        out = {}
        for name, acc in (("good", good), ("bad", good.clone())):
            if name == "bad":
                for b_, v_ in bad.items():
                    acc[b_] = v_
            bonus = torch.zeros(B, dtype=torch.int32, device="cuda")
            err = torch.zeros(B, dtype=torch.int32, device="cuda")
            ssd.ssd_residual_sample(shape, zpd, zqd, pm, ps, pa, qm, qs, F, ids, Z, 0.5, acc, 1, 2, bonus, None, err)
            torch.cuda.synchronize()
            out[name] = (bonus.cpu().numpy(), err.cpu().numpy())
        bo, eo = out["bad"]
        for b_ in bad:
            assert bo[b_] == -1 and eo[b_] == ssd.SSD_DEVERR_LEN_RANGE
        rest = np.array([b_ not in bad for b_ in range(B)])
        assert np.all(eo[rest] == 0) and np.all(out["good"][1] == 0)
        assert np.array_equal(bo[rest], out["good"][0][rest])
        assert np.all((bo[rest] >= 0) & (bo[rest] < V))
        if T == 0.0:
            ap = np.argmax(zp.float().numpy(), -1)  # bf16 widens exactly; lowest id on ties
            k = good.cpu().numpy()
            assert all(bo[b_] == ap[b_, k[b_]] for b_ in range(B) if rest[b_])


# ----------------------------------------------------------------------------- workloads
def test_c1_rounds():
    """The single-sequence workload: all of its rounds, each with its own logits and
    counter."""
    flagged = 0
    ws = ssd.Workspace()
    for rnd in range(pc.C1_ROUNDS):
        if rnd % 100 == 0:
            _case("c1 round %d" % rnd)
        c = pc.c1_case(rnd)
        o = c.oracle_round()
        g = gpu_round(c.zp.cuda(), c.zq.cuda(), c.T, c.F, c.C, c.draft, c.seed, c.rnd, c.fallback, ws=ws)
        flagged += compare_round(g, o, c.K, sum(c.F), label=c.label)
    _check_flags("c1 rounds", flagged)
    assert flagged <= max(1, pc.C1_ROUNDS // 1000)


@pytest.mark.parametrize("label", [c[0] for c in pc.FULL_CASES])
def test_full_size_whole_batch(label):
    """A workload's whole batch at its full size, in the launch configuration the
    benchmark times, against the oracle sequence by sequence (c4 at three of its
    (target spread, C) points, c2 on its own recipe at each temperature).  c3 odd V:
    V = 128257, so every row after the first starts off a 16-byte boundary.  At most
    max(1, 1e-3 B) sequences may be flagged; the count must equal the stored one.  The
    six separate calls, chained, must give the round's outputs bit for bit."""
    _case("full-size %s: inputs and oracle" % label)
    c = pc.full_case(label)
    w, F = c.w, np.array(c.F)
    o = c.oracle_round()
    _case("full-size %s: GPU round" % label)
    zpd, zqd = c.zp.cuda(), c.zq.cuda()
    g = gpu_round(zpd, zqd, c.T, c.F, c.C, c.draft, c.seed, c.rnd, c.fallback, values=c.values)
    flagged = compare_round(g, o, w.K, w.Bf, label=label, values=c.values)
    _check_flags(label, flagged)
    assert flagged <= max(1, w.B // 1000), (label, flagged)
    # properties that hold for every sequence
    assert np.all((g["accept_len"] >= 0) & (g["accept_len"] <= w.K))
    assert np.all((g["bonus"] >= 0) & (g["bonus"] < w.V))
    O = np.concatenate([[0], np.cumsum(F)])
    for b in range(w.B):
        k = g["accept_len"][b]
        S = g["cache_ids"][b, O[k]:O[k + 1]]
        assert g["hit"][b] == (g["bonus"][b] in S)
    assert np.all(g["dev_err"] == 0)
    # the six separate calls give the fused round's outputs bit for bit (at c4 and c5
    # the residual draw's pass runs two tiles per wave in both)
    _case("full-size %s: separate calls" % label)
    ch = _chain(zpd, zqd, c.T, c.F, c.C, c.draft, c.seed, c.rnd, c.fallback)
    for k in ch:
        a, b = g[k], ch[k]
        if k == "cache_ids":
            a, b = a[:, :w.Bf], b[:, :w.Bf]
        assert np.array_equal(a, b), (label, k)
    del ch
    # coverage statistics of this round: the bonus ranks below F_k exactly on a hit,
    # and every rank equals the oracle's
    _case("full-size %s: bonus rank" % label)
    zq = c.zq.cuda()
    rank = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    hist = torch.zeros((w.K + 1, 65), dtype=torch.int32, device="cuda")
    acc_d = torch.as_tensor(g["accept_len"], device="cuda")
    ssd.ssd_bonus_rank(ssd.shape_of(zq, c.T), zq, acc_d, torch.as_tensor(g["bonus"], device="cuda"), 64, rank, hist)
    torch.cuda.synchronize()
    rk = rank.cpu().numpy()
    assert np.array_equal(rk < F[g["accept_len"]], g["hit"] == 1)
    assert int(hist.sum()) == w.B
    orank, _ = oracle.bonus_rank(c.zq_np, g["accept_len"], g["bonus"], 64)
    assert np.array_equal(rk, orank), label


@pytest.mark.parametrize("label", [c[0] for c in pc.MASK_CASES])
def test_round_masked_vocabulary(label):
    """-inf logits (masked ids) in the fused round against the oracle: shared masks,
    target-only masks (draft tokens the target forbids are rejected with ratio 0),
    and a draft row with fewer finite ids than its cache share."""
    _case("mask " + label)
    c = pc.mask_case(label)
    o = c.oracle_round()
    g_ = gpu_round(c.zp.cuda(), c.zq.cuda(), c.T, c.F, c.C, c.draft, c.seed, c.rnd, c.fallback, values=c.values)
    _check_flags(label, compare_round(g_, o, c.K, sum(c.F), label=label, values=c.values))


@pytest.mark.parametrize("i", range(pc.N_RANDOM))
def test_round_random_configs(i):
    """The fused round against the oracle (and against itself chained through the six
    separate calls) over 96 seeded random configurations, row strides above V and
    masked vocabularies included."""
    c = pc.random_case(i)
    _case(c.label)
    zpd, zqd = _to_dev(c.zp), _to_dev(c.zq)
    Bf = sum(c.F)
    o = c.oracle_round()
    g = gpu_round(zpd, zqd, c.T, c.F, c.C, c.draft, c.seed, c.rnd, c.fallback, values=c.values)
    _check_flags(c.label, compare_round(g, o, c.K, Bf, label=c.label, values=c.values))
    ch = _chain(zpd, zqd, c.T, c.F, c.C, c.draft, c.seed, c.rnd, c.fallback)
    for k in ch:
        a, b = g[k], ch[k]
        if k == "cache_ids":
            a, b = a[:, :Bf], b[:, :Bf]
        assert np.array_equal(a, b), (c.label, k)


UNALIGNED_CASES = [
    # (label, dtype, B, K, V, base offset in elements): rows that do not start on a
    # 16-byte boundary are read as two aligned vectors and a byte shift
    ("odd vocabulary bf16", "bf16", 4, 3, 50257, 0),
    ("odd vocabulary f32", "f32", 3, 2, 50257, 0),
    ("shifted base bf16", "bf16", 3, 2, 128256, 1),
    ("shifted base f32", "f32", 2, 3, 40000, 3),
]


@pytest.mark.parametrize("case", UNALIGNED_CASES, ids=lambda c: c[0])
def test_round_unaligned_rows(case):
    """The fused round on rows whose start is not 16-byte aligned (an odd row stride, or
    a base pointer one or three elements into an allocation) against the oracle."""
    label, dtype, B, K, V, off = case
    _case("unaligned " + label)
    zq, zp = _rand(B, K, V, dtype, sum(map(ord, label)), 2.0, 0.8)
    F = [6, 4, 2, 1][:K + 1]
    while len(F) < K + 1:
        F.append(1)
    T, C, seed, rnd = 1.0, 0.5, 0xA11 + B, 4
    zp_np, zq_np = to_oracle_array(zp), to_oracle_array(zq)
    draft, _ = oracle_draft(zp_np, zq_np, T, np.array(F, np.int32), C, seed, rnd)
    o = oracle.round_(zp_np, zq_np, T, np.array(F, np.int32), C, draft, seed, rnd, 1)

    def dev(z):
        if off == 0:
            return z.cuda()
        flat = torch.empty(z.numel() + off, dtype=z.dtype, device="cuda")
        flat[:off] = float("nan")
        flat[off:] = z.reshape(-1).cuda()
        return flat[off:].view(z.shape)

    zpd, zqd = dev(zp), dev(zq)
    g = gpu_round(zpd, zqd, T, F, C, draft, seed, rnd, 1)
    compare_round(g, o, K, sum(F), label=label)
