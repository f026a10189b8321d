"""The host-only policies of the C ABI (fan-out from measured coverage, fallback
speculator by batch size) against the oracle, on the CPU: these entry points run on
the host and launch nothing."""
import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def ssd():
    import lossless_rejection_sampling_ssd_amd as m
    return m


@pytest.mark.parametrize("K,R,Fmax", [(1, 4, 4), (3, 8, 6), (8, 64, 64), (16, 64, 64), (16, 5, 64), (4, 64, 9)])
def test_fanout_optimize_matches_oracle(ssd, K, R, Fmax):
    rng = np.random.default_rng(K * 100 + R)
    cap = min(Fmax, R)
    for trial in range(12):
        shape = (K + 1, R + 1)
        if trial % 3 == 0:
            hist = rng.integers(0, 1000, shape)
        elif trial % 3 == 1:  # geometric-looking coverage with noise, like measured data
            hist = np.array([[int(5000 * 0.6 ** k * 0.85 ** j) for j in range(R + 1)] for k in range(K + 1)])
            hist = hist + rng.integers(0, 3, shape)
        else:  # sparse, many ties
            hist = rng.integers(0, 3, shape) * (rng.random(shape) < 0.2)
        for Bf in sorted({0, 1, cap, (K + 1) * cap // 3, (K + 1) * cap}):
            F, hits, total = ssd.ssd_fanout_optimize(K, Bf, Fmax, hist)
            oF, ohits, ototal = oracle.fanout_optimize(hist, Bf, Fmax)
            assert F == oF.tolist(), (K, R, Fmax, Bf, trial)
            assert (hits, total) == (ohits, ototal)


def test_fanout_optimize_rejects(ssd):
    h = np.ones((4, 9), np.uint32)
    for K, Bf, Fmax in ((3, 33, 64), (3, -1, 8), (0, 1, 8), (3, 4, -1), (3, 4, 65)):
        with pytest.raises(ssd.SSDError):
            ssd.ssd_fanout_optimize(K, Bf, Fmax, h if K == 3 else np.ones((K + 1, 9)))
    with pytest.raises(ssd.SSDError):
        ssd.ssd_fanout_optimize(3, 4, 8, np.ones((4, 66)))  # R = 65 > SSD_MAX_F


def _model(ssd, **kw):
    d = dict(t_verify=1.0, t_primary=0.8, t_random=0.05, n_hit=3.0, n_primary=3.0, n_random=1.2)
    d.update(kw)
    return ssd.ssd_fallback_model(**d), d


def test_fallback_choose_matches_oracle(ssd):
    rng = np.random.default_rng(5)
    seen = set()
    for trial in range(300):
        B = int(rng.integers(1, 300))
        m, d = _model(ssd, t_verify=float(rng.uniform(0.1, 2)), t_primary=float(rng.uniform(0, 3)),
                      t_random=float(rng.uniform(0, 0.3)), n_hit=float(rng.uniform(1, 5)),
                      n_primary=float(rng.uniform(1, 5)), n_random=float(rng.uniform(0.5, 2)))
        h = rng.uniform(0.6, 1.0, B) if trial % 2 else np.full(B, rng.uniform(0.9, 1.0))
        c, tp, tr = ssd.ssd_fallback_choose(m, h)
        oc, otp, otr = oracle.fallback_choose(d, h.tolist())
        assert tp == pytest.approx(otp, rel=1e-13) and tr == pytest.approx(otr, rel=1e-13)
        if abs(tp - tr) > 1e-12 * max(tp, tr):
            assert c == oc
        seen.add(c)
    assert seen == {ssd.SSD_FALLBACK_NONE, ssd.SSD_FALLBACK_UNIFORM}


def test_fallback_critical_batch_matches_oracle(ssd):
    rng = np.random.default_rng(6)
    found = 0
    for trial in range(40):
        m, d = _model(ssd, t_verify=float(rng.uniform(0.2, 2)), t_primary=float(rng.uniform(0.5, 4)),
                      t_random=float(rng.uniform(0, 0.2)), n_hit=3.0, n_primary=3.0,
                      n_random=float(rng.uniform(0.5, 2.5)))
        h = float(rng.uniform(0.9, 0.999))
        b = ssd.ssd_fallback_critical_batch(m, h, 400)
        assert b == oracle.fallback_critical_batch(d, h, 400)
        found += b > 0
    assert found > 5


def test_fallback_rejects(ssd):
    m, _ = _model(ssd)
    bad, _ = _model(ssd, t_verify=0.0)
    with pytest.raises(ssd.SSDError):
        ssd.ssd_fallback_choose(bad, [0.5])
    with pytest.raises(ssd.SSDError):
        ssd.ssd_fallback_choose(m, [1.5])
    with pytest.raises(ssd.SSDError):
        ssd.ssd_fallback_choose(m, [])
    with pytest.raises(ssd.SSDError):
        ssd.ssd_fallback_critical_batch(m, -0.1, 10)
    with pytest.raises(ssd.SSDError):
        ssd.ssd_fallback_critical_batch(m, 0.5, 0)
