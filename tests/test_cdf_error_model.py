"""Derivation of the E2 band (the inverse-CDF near-tie) from the arithmetic of the GPU
path, on the CPU.

The bonus is the smallest id whose running residual mass exceeds u times the total.
The GPU forms that running sum from fp32 terms, the oracle from fp64 ones, so the
two can pick different ids only when u lies within the GPU's CDF error of a step.
A worst-case bound of that error (every rounding of every term aligned) is about
2e-6, which is of the order of one token's whole step at these vocabularies and
would exclude most rows.  The error that occurs is far smaller, because it is a
weighted mean of many independent roundings.  This file measures it with a numpy
model of the kernels' arithmetic -- not a copy of the kernels, and not run on the
device it checks:

  * c = fp32(log2(e) / T); every term is exp2 of the fp32 exponent fma(z, c, -o)
    (one rounding) with an integer offset o = rint(fp32(m c)) from a running lane
    maximum, and exp2 carries a random relative error of up to one fp32 ulp (the
    accuracy of the hardware's exp2);
  * a lane sums its 8-element vectors as fp32 trees, then its 8 vector sums in fp32
    after rescaling to the new offset when the lane maximum grows (exact ldexp);
    lanes, waves and tiles merge in fp64 (pass 1's layout: a tile is 64 lanes x 8
    vectors of 16 bytes);
  * row normaliser, cached mass, Z, residual weights max(tp - tq rho, 0) and the
    running sums are fp64, as in the kernels.

Rows are the workloads' own recipes at full vocabulary, every position of every
sequence used as a bonus row (residual rows after a rejection, the target row when
all are accepted).  The measured error is compared with the E2 band the oracle
computes for each draw from the same error model (draw_bands in ssd_oracle.c).
"""
import numpy as np
import pytest
import torch

from lossless_rejection_sampling_ssd_amd.workloads import WORKLOADS, make_logits, scaled, to_oracle_array

LOG2E = 1.4426950408889634
BLOCK = 512  # ids per block of the two-level draw
F32 = np.float32


def _exp2f(x, rng):
    """exp2 of fp32 arguments rounded to fp32 after a random relative error of up to
    one fp32 ulp (2^-23 relative)."""
    x = np.asarray(x, np.float64)
    y = np.exp2(x)
    eps = rng.uniform(-1.0, 1.0, size=y.shape) * 2.0**-23
    return (y * (1.0 + eps)).astype(F32)


def _fma32(z, c, o):
    """fp32 fma(z, c, -o): the product of two fp32 values and an integer-valued offset
    are exact in fp64, so one rounding to fp32 is the fused result."""
    return (np.asarray(z, np.float64) * np.float64(c) - np.asarray(o, np.float64)).astype(F32)


def _offset(m, c):
    """rint(fp32(m c)), 0 for m = -inf."""
    mc = (np.asarray(m, np.float32) * F32(c)).astype(F32)
    o = np.rint(mc).astype(F32)
    return np.where(np.isneginf(m), F32(0), o)


def _row_stats(z, c, rng):
    """(m, s) of one row as the kernels form them: s = sum 2^{z c - o(m)}."""
    V = z.shape[0]
    N = 8 if z.dtype == np.dtype("uint16") else 4
    x = _widen(z)
    tile = 64 * 8 * N
    nt = -(-V // tile)
    pad = np.full(nt * tile, -np.inf, np.float32)
    pad[:V] = x
    # [tile, vector j, lane, element e] -> per lane, vectors in order
    lanes = pad.reshape(nt, 8, 64, N)
    m = np.full((nt, 64), -np.inf, np.float32)
    s = np.zeros((nt, 64), np.float32)
    o = np.zeros((nt, 64), np.float32)
    for j in range(8):
        v = lanes[:, j]                                     # [nt, 64, N]
        m = np.maximum(m, v.max(axis=2))
        on = _offset(m, c)
        s = np.ldexp(s, (o - on).astype(np.int32)).astype(F32)
        o = on
        t = _exp2f(_fma32(v, c, o[:, :, None]), rng)        # [nt, 64, N]
        w = N // 2
        while w >= 1:
            t = (t[:, :, :w] + t[:, :, w:2 * w]).astype(F32)
            w //= 2
        s = (s + t[:, :, 0]).astype(F32)
    mrow = m.max()
    orow = _offset(mrow, c)
    keep = ~np.isneginf(m)
    srow = np.sum(np.ldexp(s[keep].astype(np.float64), (o[keep] - orow).astype(np.int32)))
    # standard form: s_std = s_rel * 2^{o - m c}, the factor an fp32 exp2
    f = float(_exp2f(np.float32(float(orow) - float(mrow) * float(c)), rng))
    return float(mrow), srow * f, f


def _widen(z):
    if z.dtype == np.dtype("uint16"):
        return (z.astype(np.uint32) << 16).view(np.float32)
    return z.astype(np.float32)


def _row_terms(z, c, m, rng):
    """Per-element terms 2^{z c - o(m)} (fp32 model) and the offset factor."""
    o = _offset(np.float32(m), c)
    return _exp2f(_fma32(_widen(z), c, o), rng).astype(np.float64)


def _gpu_weights(zp, zq, k, K, T, C, S, rng):
    """The bonus row's draw weights as the GPU forms them (any common scale)."""
    c = F32(LOG2E / T)
    mp, sp, fp = _row_stats(zp, c, rng)
    mq, sq, fq = _row_stats(zq, c, rng)
    inv_p, inv_q = fp / sp, fq / sq
    tp = _row_terms(zp, c, mp, rng)
    if k == K:
        return tp
    tq = _row_terms(zq, c, mq, rng)
    M = float(np.sum(tq[S]) * inv_q)
    Z = 1.0 - (1.0 - C) * M
    rho = inv_q / Z / inv_p
    sel = np.full(tq.shape, rho)
    sel[S] = rho * C
    w = np.maximum(tp - tq * sel, 0.0)
    return w if w.sum() > 0.0 else tp


def _levels(w, blk):
    """Block masses and, for block blk, the within-block weights."""
    V = w.shape[0]
    nb = -(-V // BLOCK)
    W = np.array([w[b * BLOCK:min(V, (b + 1) * BLOCK)].sum() for b in range(nb)])
    return W, w[blk * BLOCK:min(V, (blk + 1) * BLOCK)]


def _steps(cum, i):
    """Normalised CDF just below and at entry i of the running sums cum."""
    lo = cum[i - 1] if i > 0 else 0.0
    return np.array([lo, cum[i]]) / cum[-1]


CASES = [
    # (workload, B, temperature, target sigma)
    ("c3", 6, 1.0, None),
    ("c4", 4, 1.2, 1.65),
    ("c4", 4, 1.2, 0.3),
    ("c5", 6, 1.0, None),
    ("c2", 12, 0.7, None),
    ("c2", 12, 1.0, None),
]


@pytest.mark.parametrize("name,B,T,sig", CASES, ids=["%s-T%g-%s" % (c[0], c[2], c[3]) for c in CASES])
def test_cdf_error_within_band(orc, name, B, T, sig):
    """On every bonus row of the workload, at both levels of the draw, the emulated GPU
    CDF at the two steps around the oracle's pick differs from the oracle's by less
    than half the E2 band the oracle computes for that draw and level, and by more than
    a twelfth of it somewhere (the band is not padded far beyond the error); and the
    bands are narrow enough that the chance of flagging a draw stays below 1e-3."""
    w = scaled(WORKLOADS[name], B=B)
    zq_t, zp_t = make_logits(w, buffer=7, target_sigma=sig)
    zp, zq = to_oracle_array(zp_t), to_oracle_array(zq_t)
    K = w.K
    C = w.Cs[len(w.Cs) // 2]
    F, _ = orc.fanout(K, w.Bf, w.r)
    ps, qs = orc.softmax(zp, T), orc.softmax(zq, T)
    ids, mass = orc.build_cache(zq, T, F)
    Z, _ = orc.saguaro(zq, T, F, ids, mass, C)
    O = np.concatenate([[0], np.cumsum(F)])
    rng = np.random.default_rng(11)
    worst, rows, p_flag = [0.0, 0.0], 0, []
    for k in range(K + 1):
        acc = np.full(B, k, np.int32)
        bonus, zr, resid, _, exc, e2 = orc.residual_sample(zp, zq, T, ps, qs, F, ids, Z, C, acc, w.seed, 3,
                                                           want_resid=True, want_bands=True)
        for b in range(B):
            if k < K and zr[b] < 1e-5:
                continue  # E3 rows are not compared
            j = int(bonus[b])
            blk = j // BLOCK
            g = _gpu_weights(zp[b, k], zq[b, k], k, K, T, C, ids[b, O[k]:O[k + 1]], rng)
            Wo, wo = _levels(resid[b], blk)
            Wg, wg = _levels(g, blk)
            e1 = np.max(np.abs(_steps(np.cumsum(Wg), blk) - _steps(np.cumsum(Wo), blk)))
            e2_ = np.max(np.abs(_steps(np.cumsum(wg), j - blk * BLOCK) - _steps(np.cumsum(wo), j - blk * BLOCK)))
            worst[0] = max(worst[0], e1 / e2[b, 1])
            worst[1] = max(worst[1], e2_ / e2[b, 3])
            # chance that u1 or u2 falls within its band of a step around its pick
            pb = Wo / Wo.sum()
            f = np.sum(np.minimum(pb, 2 * e2[b, 1]))
            for bb in np.nonzero(Wo > 0)[0]:
                wb = resid[b][bb * BLOCK:(bb + 1) * BLOCK]
                wb = wb[wb > 0] / wb.sum()
                f += pb[bb] * np.sum(np.minimum(wb, 2 * e2[b, 3]))
            p_flag.append(f)
            rows += 1
    print("%s T=%g sigma=%s: %d bonus rows, largest error / band: blocks %.3f, ids %.3f; mean flag chance %.2e" % (
        name, T, sig, rows, worst[0], worst[1], np.mean(p_flag)))
    assert rows >= B * K // 2
    assert max(worst) < 0.5, worst
    assert max(worst) > 1.0 / 12.0, worst
    assert np.mean(p_flag) < 1e-3
