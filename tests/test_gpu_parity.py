"""Parity of the HIP path (called through the C ABI) with the fp64 oracle on seeded
synthetic inputs.  Each test prints what names its case before the GPU step."""
import numpy as np
import pytest
import torch

import oracle
import lossless_rejection_sampling_ssd_amd as ssd
from lossless_rejection_sampling_ssd_amd.workloads import WORKLOADS, make_logits, scaled, to_oracle_array

from gpu_helpers import PROB_ATOL, SUM_RTOL, compare_round, gpu_round, oracle_draft

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def _case(msg):
    print("\n[case] " + msg, flush=True)


def _rand(B, K, V, dtype, seed, scale=2.0, noise=0.8, ld=None):
    g = torch.Generator().manual_seed(seed)
    zq = torch.randn((B, K + 1, V), generator=g) * scale
    zp = zq + torch.randn((B, K + 1, V), generator=g) * noise
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    zq, zp = zq.to(dt), zp.to(dt)
    if ld is not None and ld > V:
        def pad(z):
            o = torch.full((B, K + 1, ld), float("nan"), dtype=dt)
            o[:, :, :V] = z
            return o[:, :, :V]
        zq, zp = pad(zq), pad(zp)
    return zq, zp


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
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,C", [(1.0, 0.5), (0.7, 0.2), (1.0, 1.0), (0.0, 0.5)])
def test_saguaro_and_draft(dtype, T, C):
    V, B, K = 6007, 8, 3
    _case("saguaro dtype=%s T=%g C=%g" % (dtype, T, C))
    zq, _ = _rand(B, K, V, dtype, 21)
    F = [6, 3, 2, 1]
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


EDGE_CASES = [
    # (label, dtype, B, K, V, T, F, C, scale, noise, quantum)
    # F_k at its maximum, with coarse (heavily tied) draft logits: many tied candidates
    # per tile, the histogram select and the exact per-tile fallback
    ("F=64 ties", "bf16", 3, 2, 50000, 1.0, [64, 0, 0], 0.5, 1.0, 0.3, 0.5),
    ("F=64 smooth", "f32", 4, 1, 70001, 1.0, [64, 0], 0.3, 2.0, 0.5, 0.0),
    ("peaked T=0.05", "bf16", 6, 3, 20000, 0.05, [8, 4, 2, 1], 0.5, 2.0, 0.5, 0.0),
    ("flat T=5", "f32", 6, 3, 20000, 5.0, [8, 4, 2, 1], 0.5, 2.0, 0.5, 0.0),
    ("large logits", "f32", 5, 2, 9000, 1.0, [6, 3, 1], 0.5, 3000.0, 20.0, 0.0),
    ("all tied", "bf16", 4, 2, 6000, 1.0, [5, 3, 1], 0.5, 0.0, 0.0, 0.0),
    # more than 64 tiles per row (pass 1: 4096 bf16 / 2048 fp32 elements per tile):
    # the finalisation's general path and the bonus's multi-chunk scans
    ("V=300k bf16", "bf16", 3, 2, 300001, 1.0, [12, 6, 3], 0.5, 2.0, 0.5, 0.0),
    ("V=200k f32", "f32", 2, 3, 200003, 0.8, [9, 5, 3, 2], 0.6, 2.0, 0.5, 0.0),
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=lambda c: c[0])
def test_round_edge_cases(case):
    """The fused round against the oracle at the edges of the method: the largest
    fan-out share, heavy ties, near-greedy and flat temperatures, large logits, and
    rows where every logit is equal."""
    label, dtype, B, K, V, T, F, C, scale, noise, quantum = case
    _case("edge " + label)
    g = torch.Generator().manual_seed(sum(map(ord, label)))
    zq = torch.randn((B, K + 1, V), generator=g) * scale
    if quantum > 0:
        zq = torch.round(zq / quantum) * quantum
    zp = zq + torch.randn((B, K + 1, V), generator=g) * noise
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    zq, zp = zq.to(dt), zp.to(dt)
    zp_np, zq_np = to_oracle_array(zp), to_oracle_array(zq)
    seed, rnd = 0xED6E + B, 5
    draft, _ = oracle_draft(zp_np, zq_np, T, np.array(F, np.int32), C, seed, rnd)
    draft[0, 0] = 0
    draft[-1, -1] = V - 1
    o = oracle.round_(zp_np, zq_np, T, np.array(F, np.int32), C, draft, seed, rnd, 1)
    g_ = gpu_round(zp.cuda(), zq.cuda(), T, F, C, draft, seed, rnd, 1)
    flagged = compare_round(g_, o, K, sum(F), label=label)
    assert flagged < B, (label, flagged)  # the forced edge tokens may be flagged; the rest are compared


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


def test_residual_bad_len_and_greedy():
    """ssd_residual_sample with accepted lengths outside [0, K] reports the error and
    returns -1; at T = 0 it returns argmax p_k."""
    B, K, V = 4, 3, 999
    zq, zp = _rand(B, K, V, "f32", 8)
    F = [3, 2, 1, 1]
    for T in (1.0, 0.0):
        _case("residual bad len T=%g" % T)
        zpd, zqd = zp.cuda(), zq.cuda()
        pm, ps, pa = _gpu_stats(zpd, T)
        qm, qs, qa = _gpu_stats(zqd, T)
        ids = torch.zeros((B, sum(F)), dtype=torch.int32, device="cuda")
        mass = torch.zeros(B * (K + 1), dtype=torch.float64, device="cuda")
        shape = ssd.shape_of(zpd, T)
        ssd.ssd_build_cache(shape, zqd, qm, qs, F, ids, mass)
        Z = torch.zeros(B * (K + 1), dtype=torch.float64, device="cuda")
        ssd.ssd_saguaro_reweight(shape, mass, 0.5, Z)
        acc = torch.tensor([0, 3, -1, 4], dtype=torch.int32, device="cuda")
        bonus = torch.zeros(B, dtype=torch.int32, device="cuda")
        err = torch.zeros(B, dtype=torch.int32, device="cuda")
        ssd.ssd_residual_sample(shape, zpd, zqd, pm, ps, pa, qm, qs, F, ids, Z, 0.5, acc, 1, 2, bonus, None, err)
        torch.cuda.synchronize()
        bo = bonus.cpu().numpy()
        eo = err.cpu().numpy()
        assert bo[2] == -1 and bo[3] == -1
        assert eo[2] == ssd.SSD_DEVERR_LEN_RANGE and eo[3] == ssd.SSD_DEVERR_LEN_RANGE
        assert eo[0] == 0 and eo[1] == 0
        if T == 0.0:
            ap = np.argmax(zp.numpy(), -1)
            assert bo[0] == ap[0, 0] and bo[1] == ap[1, 3]


# ----------------------------------------------------------------------------- workloads
def test_c1_rounds():
    """The single-sequence workload: every round with its own logits and counter."""
    w = WORKLOADS["c1"]
    F, gap = oracle.fanout(w.K, w.Bf, w.r)
    flagged = 0
    n = 300
    ws = ssd.Workspace()
    for rnd in range(n):
        if rnd % 100 == 0:
            _case("c1 round %d" % rnd)
        zq, zp = make_logits(w, buffer=rnd)
        zp_np, zq_np = to_oracle_array(zp), to_oracle_array(zq)
        draft, _ = oracle_draft(zp_np, zq_np, 1.0, F, 0.5, w.seed, rnd)
        o = oracle.round_(zp_np, zq_np, 1.0, F, 0.5, draft, w.seed, rnd, False, gap)
        g = gpu_round(zp.cuda(), zq.cuda(), 1.0, F.tolist(), 0.5, draft, w.seed, rnd, 0, ws=ws)
        flagged += compare_round(g, o, w.K, w.Bf, label="c1 round %d" % rnd)
    assert flagged <= max(1, n // 100)


@pytest.mark.parametrize("name,C,sig,V", [("c3", 0.5, None, None), ("c4", 0.2, 1.65, None), ("c4", 0.8, 0.3, None),
                                          ("c5", 0.5, None, None), ("c3", 0.5, None, 128257)])
def test_full_size_sampled(name, C, sig, V):
    """The workload at its full size in the launch configuration the benchmark
    times; the oracle recomputes a sample of sequences one by one (their uniforms
    keep the global sequence index).  V = 128257: the headline shape with an odd
    vocabulary, so every row after the first starts off a 16-byte boundary."""
    w = WORKLOADS[name] if V is None else scaled(WORKLOADS[name], V=V)
    T = w.temps[0]
    _case("full-size %s C=%g sigma=%s: generate" % (name, C, sig))
    zq, zp = make_logits(w, target_sigma=sig, device="cuda")
    F, gap = oracle.fanout(w.K, w.Bf, w.r)
    rng = np.random.default_rng(w.seed)
    sample = np.sort(rng.choice(w.B, size=6, replace=False))
    seed, rnd = w.seed, 1
    draft = rng.integers(0, w.V, size=(w.B, w.K)).astype(np.int32)
    zp_h, zq_h = zp.cpu(), zq.cpu()
    per = {}
    for b in sample:
        zp_np = to_oracle_array(zp_h[b:b + 1])
        zq_np = to_oracle_array(zq_h[b:b + 1])
        d, _ = oracle_draft(zp_np, zq_np, T, F, C, seed, rnd, b_base=int(b))
        draft[b] = d[0]
        per[int(b)] = (zp_np, zq_np)
    _case("full-size %s: GPU round" % name)
    values = rng.integers(0, w.V, size=(w.B, w.Bf, w.K)).astype(np.int32)
    g = gpu_round(zp, zq, T, F.tolist(), C, draft, seed, rnd, int(w.fallback_uniform), values=values)
    _case("full-size %s: oracle on %s" % (name, sample.tolist()))
    for b in sample:
        zp_np, zq_np = per[int(b)]
        o = oracle.round_(zp_np, zq_np, T, F, C, draft[b:b + 1], seed, rnd, w.fallback_uniform, gap, int(b))
        K1 = w.K + 1
        gb = {k: (v[b * K1:(b + 1) * K1] if v.ndim == 1 and v.shape[0] == w.B * K1 else v[b:b + 1])
              for k, v in g.items()}
        compare_round(gb, o, w.K, w.Bf, label="%s b=%d" % (name, b), values=values[b:b + 1])
    # properties that hold for every sequence
    assert np.all((g["accept_len"] >= 0) & (g["accept_len"] <= w.K))
    assert np.all((g["bonus"] >= 0) & (g["bonus"] < w.V))
    O = np.concatenate([[0], np.cumsum(F)])
    for b in range(w.B):
        k = g["accept_len"][b]
        S = g["cache_ids"][b, O[k]:O[k + 1]]
        h = g["bonus"][b] in S
        assert g["hit"][b] == h
        if not h and w.fallback_uniform:
            assert np.all((g["fallback_tokens"][b] >= 0) & (g["fallback_tokens"][b] < w.V))
    nd, _ = oracle.cache_gather(values, g["hit"], g["slot"], g["fallback_tokens"])
    assert np.array_equal(g["next_draft"], nd)
    assert np.all(g["dev_err"] == 0)
    # coverage statistics of this round: the bonus ranks below F_k exactly on a hit
    _case("full-size %s: bonus rank" % name)
    rank = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    hist = torch.zeros((w.K + 1, 65), dtype=torch.int32, device="cuda")
    acc_d = torch.as_tensor(g["accept_len"], device="cuda")
    ssd.ssd_bonus_rank(ssd.shape_of(zq, T), zq, acc_d, torch.as_tensor(g["bonus"], device="cuda"), 64, rank, hist)
    torch.cuda.synchronize()
    rk = rank.cpu().numpy()
    assert np.array_equal(rk < F[g["accept_len"]], g["hit"] == 1)
    assert int(hist.sum()) == w.B
    for b in sample:
        orank, _ = oracle.bonus_rank(per[int(b)][1], g["accept_len"][b:b + 1], g["bonus"][b:b + 1], 64)
        assert rk[b] == orank[0], (name, b)


MASK_CASES = [
    # (label, dtype, B, K, V, T, F, C, frac_shared, frac_target_only, n_finite_row0)
    # a vocabulary mask shared by both models (banned ids)
    ("shared mask", "bf16", 6, 3, 30000, 1.0, [10, 6, 3, 1], 0.5, 0.5, 0.0, 0),
    # ids only the target masks: the draft proposes tokens of target probability 0
    ("target-only mask", "f32", 6, 3, 20000, 1.0, [8, 4, 2, 1], 0.5, 0.0, 0.3, 0),
    # a row with fewer finite ids than F_0 (the cache takes -inf ids, lower id first)
    ("F above finite ids", "bf16", 4, 2, 9000, 0.8, [20, 4, 2], 0.4, 0.2, 0.1, 7),
    # greedy with masks
    ("masked greedy", "f32", 5, 3, 12000, 0.0, [6, 3, 2, 1], 0.5, 0.4, 0.2, 0),
]


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: c[0])
def test_round_masked_vocabulary(case):
    """-inf logits (masked ids) in the fused round against the oracle: shared masks,
    target-only masks (draft tokens the target forbids are rejected with ratio 0),
    and a draft row with fewer finite ids than its cache share."""
    label, dtype, B, K, V, T, F, C, f_shared, f_target, n_fin = case
    _case("mask " + label)
    g = torch.Generator().manual_seed(sum(map(ord, label)))
    zq = torch.randn((B, K + 1, V), generator=g) * 2.0
    zp = zq + torch.randn((B, K + 1, V), generator=g) * 0.7
    shared = torch.rand((B, K + 1, V), generator=g) < f_shared
    target = torch.rand((B, K + 1, V), generator=g) < f_target
    zq[shared] = float("-inf")
    zp[shared | target] = float("-inf")
    # every row keeps one finite id in both models
    zq[:, :, 123 % V] = 1.0
    zp[:, :, 123 % V] = 1.0
    if n_fin:
        keep = torch.randperm(V, generator=g)[:n_fin]
        row = torch.full((V,), float("-inf"))
        row[keep] = torch.randn(n_fin, generator=g)
        zq[0, 0] = row
        zp[0, 0] = row + 0.1
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    zq, zp = zq.to(dt), zp.to(dt)
    zp_np, zq_np = to_oracle_array(zp), to_oracle_array(zq)
    seed, rnd = 0x3A5C + B, 2
    draft, _ = oracle_draft(zp_np, zq_np, T, np.array(F, np.int32), C, seed, rnd)
    o = oracle.round_(zp_np, zq_np, T, np.array(F, np.int32), C, draft, seed, rnd, 1)
    values = np.random.default_rng(B).integers(0, V, (B, sum(F), K)).astype(np.int32)
    g_ = gpu_round(zp.cuda(), zq.cuda(), T, F, C, draft, seed, rnd, 1, values=values)
    flagged = compare_round(g_, o, K, sum(F), label=label, values=values)
    assert flagged <= B // 2, (label, flagged)


def _random_round_config(i):
    """Seeded random configuration i: dtype, shape, row padding, temperature, an
    arbitrary fan-out (any split of B_f with 0 <= F_k <= 64, not only geometric), C,
    the fallback mode and, for about a quarter of them, a fraction of ids masked
    (-inf) in both models."""
    rng = np.random.default_rng(0xC0FFEE + i)
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    B = int(rng.integers(1, 9))
    K = int(rng.integers(1, 11))
    V = int(rng.choice([int(rng.integers(2, 300)), int(rng.integers(300, 9000)), int(rng.integers(9000, 60000))]))
    pad = int(rng.choice([0, 0, int(rng.integers(1, 40))]))
    T = float(rng.choice([0.0, 0.5, 1.0, 1.0, 1.6]))
    Fmax = min(V, 64)
    F = [int(rng.integers(0, min(Fmax, 24) + 1)) if rng.random() < 0.8 else 0 for _ in range(K + 1)]
    C = float(rng.choice([1.0, float(rng.uniform(0.05, 1.0))]))
    fb = int(rng.integers(0, 2))
    scale = float(rng.uniform(0.5, 4.0))
    noise = float(rng.uniform(0.1, 1.5))
    mask = float(rng.uniform(0.1, 0.6)) if rng.random() < 0.25 else 0.0
    return dtype, B, K, V, pad, T, F, C, fb, scale, noise, mask


@pytest.mark.parametrize("i", range(96))
def test_round_random_configs(i):
    """The fused round against the oracle (and against itself chained through the six
    separate calls) over 96 seeded random configurations, row strides above V and
    masked vocabularies included."""
    dtype, B, K, V, pad, T, F, C, fb, scale, noise, mask = _random_round_config(i)
    label = "random %d: %s B=%d K=%d V=%d pad=%d T=%g F=%s C=%.3f fb=%d mask=%.2f" % (
        i, dtype, B, K, V, pad, T, F, C, fb, mask)
    _case(label)
    zq, zp = _rand(B, K, V, dtype, 0xAB00 + i, scale, noise, ld=V + pad if pad else None)
    if mask > 0:
        g = torch.Generator().manual_seed(0xAB00 + i)
        m = torch.rand((B, K + 1, V), generator=g) < mask
        m[:, :, 0] = False  # every row keeps a finite id
        zq[m] = float("-inf")
        zp[m] = float("-inf")
    seed, rnd = 0x5EED + i, 100 + i
    zp_np, zq_np = to_oracle_array(zp), to_oracle_array(zq)
    Fa = np.array(F, np.int32)
    draft, _ = oracle_draft(zp_np, zq_np, T, Fa, C, seed, rnd)
    o = oracle.round_(zp_np, zq_np, T, Fa, C, draft, seed, rnd, fb)
    zpd, zqd = _to_dev(zp), _to_dev(zq)
    Bf = sum(F)
    values = np.random.default_rng(i).integers(0, V, (B, max(Bf, 1), K)).astype(np.int32)[:, :Bf]
    g = gpu_round(zpd, zqd, T, F, C, draft, seed, rnd, fb, values=values if Bf > 0 else None)
    compare_round(g, o, K, Bf, label=label, values=values if Bf > 0 else None)
    ch = _chain(zpd, zqd, T, F, C, draft, seed, rnd, fb)
    for k in ch:
        a, b = g[k], ch[k]
        if k == "cache_ids":
            a, b = a[:, :Bf], b[:, :Bf]
        assert np.array_equal(a, b), (label, k)


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
