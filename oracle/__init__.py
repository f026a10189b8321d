"""fp64 CPU oracle of one SSD / Saguaro verify-and-pre-speculate round.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path (the
HIP library under ``lossless_rejection_sampling_ssd_amd`` and its binding) never
imports it, and the two share no code.

This module is argument marshalling around ``ssd_oracle.c`` (plain C, IEEE double).
It takes numpy arrays: fp32 logits as ``float32``, bf16 logits as their raw 16-bit
patterns in ``uint16`` arrays, shaped ``[B, K+1, V]`` (a row stride ``ld`` larger
than V is passed through ``ld``).  See ``ssd_oracle.c`` for the method, the passages
of the two summaries of "Speculative Speculative Decoding" each step follows, and
every reading taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")

F32, BF16 = 0, 1
PURPOSE_ACCEPT, PURPOSE_BONUS, PURPOSE_DRAFT, PURPOSE_FALLBACK = 0, 1, 2, 3
BLOCK = 512  # ids per block of the two-level draw
ERR_TOKEN_RANGE, ERR_QPRIME_ZERO, ERR_LEN_RANGE, ERR_SLOT_RANGE, ERR_HIST_RANGE = 1, 2, 4, 8, 16
FALLBACK_NONE, FALLBACK_UNIFORM = 0, 1  # the primary speculator / uniform random tokens
E1_ACCEPT_TIE, E2_CDF_TIE, E3_DEGENERATE_RESIDUAL, E4_FANOUT_TIE, E5_TINY_PROB = 1, 2, 4, 8, 16
FANOUT_EPS = 1e-9
# Floor of the inverse-CDF near-tie band (E2) on the normalised CDF.  The band of
# each draw is computed by the oracle (draw_bands in ssd_oracle.c) from the arithmetic
# of the GPU path: this floor, plus the CDF shift between the temperature the GPU
# path samples at (it applies T as an fp32 scale) and T, plus six standard deviations
# of the random walk that independent per-term fp32 errors make of the running sum.
# tests/test_cdf_error_model.py checks the band against a CPU model of that
# arithmetic.
CDF_TIE_EPS = 1e-8


def build(force: bool = False) -> str:
    """Compile ``ssd_oracle.c`` with gcc (fp64, OpenMP over independent rows)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    """The oracle library; LRS_ORACLE_LIB names another build of ssd_oracle.c to load
    instead (the sanitizer test's instrumented one)."""
    global _lib
    if _lib is None:
        other = os.environ.get("LRS_ORACLE_LIB")
        if other:
            _lib = load_library(other)
        else:
            build()
            _lib = load_library(_LIB_PATH)
    return _lib


def compile_variant(src_text: str, out_path: str) -> str:
    """Compiles C source text with the oracle's flags into out_path (a shared
    library); the tests use it for mutated copies of ``ssd_oracle.c``."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", out_path, src, "-lm"])
    return out_path


def load_library(path: str) -> ctypes.CDLL:
    """Loads a build of ``ssd_oracle.c`` and declares its signatures."""
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, u64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
    L.orc_num_threads.argtypes = []
    L.orc_num_threads.restype = i32
    L.orc_set_num_threads.argtypes = [i32]
    L.orc_set_num_threads.restype = None
    L.orc_philox4x64_10.argtypes = [P, P, P]
    L.orc_uniform.argtypes = [u64, u64, i32, i64, i64]
    L.orc_uniform.restype = dbl
    L.orc_uniform2.argtypes = [u64, u64, i32, i64, i64]
    L.orc_uniform2.restype = dbl
    L.orc_uniform_u32.argtypes = [u64, u64, i32, i64, i64]
    L.orc_uniform_u32.restype = ctypes.c_uint32
    L.orc_fanout.argtypes = [i32, i32, dbl, P, P]
    L.orc_fanout.restype = i32
    L.orc_softmax.argtypes = [i32, i32, i32, i64, i32, P, dbl, P, P, P, P]
    L.orc_build_cache.argtypes = [i32, i32, i32, i64, i32, P, dbl, P, i32, P, P]
    L.orc_saguaro.argtypes = [i32, i32, i32, i64, i32, P, dbl, P, i32, P, P, dbl, P, P]
    L.orc_draft_sample.argtypes = [i32, i32, i32, i64, i32, P, dbl, P, i32, P, P, dbl, u64, u64, i64, dbl, P, P, P]
    L.orc_verify.argtypes = [i32, i32, i32, i64, i32, P, P, dbl, P, P, P, P, P, P, P, P, i32, P, P,
                             dbl, u64, u64, i64, P, P, P, P]
    L.orc_residual_sample.argtypes = [i32, i32, i32, i64, i32, P, P, dbl, P, P, P, P, P, P, P, i32, P,
                                      P, dbl, P, u64, u64, i64, dbl, P, P, P, P, P, P]
    L.orc_cache_lookup.argtypes = [i32, i32, i32, P, i32, P, P, P, i32, u64, u64, i64, P, P, P, P]
    L.orc_cache_gather.argtypes = [i32, i32, i32, P, P, P, P, P, P]
    L.orc_ngram_fallback.argtypes = [i32, i32, i32, P, i64, P, P, P, P, P, i32, i32, u64, u64, i64, P, P,
                                     P, P, P]
    L.orc_bonus_rank.argtypes = [i32, i32, i32, i64, i32, P, P, P, i32, P, P]
    L.orc_round.argtypes = [i32, i32, i32, i64, i32, P, P, dbl, P, i32, dbl, P, u64, u64, i64, dbl, i32,
                            P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _logit_info(z):
    """(dtype code, B, K, V, ld) of a logit array [B, K+1, V] (possibly a view with a
    larger row stride)."""
    if z.dtype == np.float32:
        code, item = F32, 4
    elif z.dtype == np.uint16:
        code, item = BF16, 2
    else:
        raise TypeError("logits must be float32 or uint16 (bf16 bit patterns)")
    if z.ndim != 3:
        raise ValueError("logits must be [B, K+1, V]")
    B, K1, V = z.shape
    if z.strides[2] != item or z.strides[1] % item or z.strides[0] != z.strides[1] * K1:
        raise ValueError("logits rows must be unit-stride with a uniform row stride")
    return code, B, K1 - 1, V, z.strides[1] // item


def _base(z):
    return z.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


def philox4x64_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.zeros(4, dtype=np.uint64)
    lib().orc_philox4x64_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed, round_, purpose, b, i) -> float:
    return lib().orc_uniform(seed, round_, purpose, b, i)


def uniform2(seed, round_, purpose, b, i) -> float:
    """The second uniform of a draw (Philox counter word 3 = 1): the id within the
    block the first one picked."""
    return lib().orc_uniform2(seed, round_, purpose, b, i)


def uniform_u32(seed, round_, purpose, b, i) -> int:
    return lib().orc_uniform_u32(seed, round_, purpose, b, i)


def fanout(K: int, Bf: int, r: float):
    """Returns (F [K+1] int32, smallest remainder gap)."""
    F = np.zeros(K + 1, dtype=np.int32)
    gap = ctypes.c_double(0.0)
    rc = lib().orc_fanout(K, Bf, r, _ptr(F), ctypes.byref(gap))
    if rc != 0:
        raise ValueError("bad fan-out arguments")
    return F, gap.value


def softmax(z, T: float, want_probs: bool = False):
    code, B, K, V, ld = _logit_info(z)
    R = B * (K + 1)
    m = np.zeros(R)
    s = np.zeros(R)
    a = np.zeros(R, dtype=np.int32)
    probs = np.zeros((B, K + 1, V)) if want_probs else None
    lib().orc_softmax(B, K, V, ld, code, _base(z), T, _ptr(m), _ptr(s), _ptr(a), _ptr(probs))
    shp = (B, K + 1)
    return m.reshape(shp), s.reshape(shp), a.reshape(shp), probs


def build_cache(zq, T: float, F):
    code, B, K, V, ld = _logit_info(zq)
    F = np.ascontiguousarray(F, dtype=np.int32)
    Bf = int(F.sum())
    ids = np.zeros((B, Bf), dtype=np.int32)
    mass = np.zeros((B, K + 1))
    lib().orc_build_cache(B, K, V, ld, code, _base(zq), T, _ptr(F), Bf, _ptr(ids), _ptr(mass))
    return ids, mass


def saguaro(zq, T: float, F, cache_ids, cache_mass, C: float, want_qprime: bool = False):
    code, B, K, V, ld = _logit_info(zq)
    F = np.ascontiguousarray(F, dtype=np.int32)
    cache_ids = np.ascontiguousarray(cache_ids, dtype=np.int32)
    cache_mass = np.ascontiguousarray(cache_mass, dtype=np.float64)
    Z = np.zeros((B, K + 1))
    qp = np.zeros((B, K + 1, V)) if want_qprime else None
    lib().orc_saguaro(B, K, V, ld, code, _base(zq), T, _ptr(F), int(F.sum()), _ptr(cache_ids),
                      _ptr(cache_mass), C, _ptr(Z), _ptr(qp))
    return Z, qp


def draft_sample(zq, T: float, F, cache_ids, Z, C: float, seed: int, round_: int, b_base: int = 0,
                 cdf_eps: float = None, want_gaps: bool = False):
    """Harness step: draft tokens sampled from the reweighted draft law q' by the
    two-level draw (see ``ssd_oracle.c``).  Returns (draft, E2 flags) or, with
    want_gaps, (draft, flags, e2) with e2 [B, K, 4] = (gap of u1, band of u1, gap of u2,
    band of u2): the distances of the two uniforms to the steps around the pick and
    the E2 bands they were compared with."""
    code, B, K, V, ld = _logit_info(zq)
    F = np.ascontiguousarray(F, dtype=np.int32)
    cache_ids = np.ascontiguousarray(cache_ids, dtype=np.int32)
    Z = np.ascontiguousarray(Z, dtype=np.float64)
    d = np.zeros((B, K), dtype=np.int32)
    flags = np.zeros((B, K), dtype=np.uint8)
    e2 = np.zeros((B, K, 4))
    eps = CDF_TIE_EPS if cdf_eps is None else cdf_eps
    lib().orc_draft_sample(B, K, V, ld, code, _base(zq), T, _ptr(F), int(F.sum()), _ptr(cache_ids),
                           _ptr(Z), C, seed, round_, b_base, eps, _ptr(d), _ptr(flags), _ptr(e2))
    return (d, flags, e2) if want_gaps else (d, flags)


def verify(zp, zq, T, draft, pstats, qstats, F, cache_ids, Z, C, seed, round_, b_base: int = 0):
    code, B, K, V, ld = _logit_info(zp)
    F = np.ascontiguousarray(F, dtype=np.int32)
    pm, ps, pa = (np.ascontiguousarray(x) for x in pstats[:3])
    qm, qs, qa = (np.ascontiguousarray(x) for x in qstats[:3])
    draft = np.ascontiguousarray(draft, dtype=np.int32)
    cache_ids = np.ascontiguousarray(cache_ids, dtype=np.int32)
    Z = np.ascontiguousarray(Z, dtype=np.float64)
    acc = np.zeros(B, dtype=np.int32)
    aprob = np.zeros((B, K))
    err = np.zeros(B, dtype=np.int32)
    exc = np.zeros(B, dtype=np.uint8)
    lib().orc_verify(B, K, V, ld, code, _base(zp), _base(zq), T, _ptr(draft), _ptr(pm), _ptr(ps), _ptr(pa),
                     _ptr(qm), _ptr(qs), _ptr(qa), _ptr(F), int(F.sum()), _ptr(cache_ids), _ptr(Z), C,
                     seed, round_, b_base, _ptr(acc), _ptr(aprob), _ptr(err), _ptr(exc))
    return acc, aprob, err, exc


def residual_sample(zp, zq, T, pstats, qstats, F, cache_ids, Z, C, accept_len, seed, round_,
                    want_resid: bool = False, b_base: int = 0, cdf_eps: float = None, want_bands: bool = False):
    """Bonus tokens by the two-level draw.  Returns (bonus, Z_r, weights or None, err,
    exc), and with want_bands also e2 [B, 4] = (gap of u1, band of u1, gap of u2, band
    of u2)."""
    code, B, K, V, ld = _logit_info(zp)
    F = np.ascontiguousarray(F, dtype=np.int32)
    pm, ps, pa = (np.ascontiguousarray(x) for x in pstats[:3])
    qm, qs, qa = (np.ascontiguousarray(x) for x in qstats[:3])
    cache_ids = np.ascontiguousarray(cache_ids, dtype=np.int32)
    Z = np.ascontiguousarray(Z, dtype=np.float64)
    accept_len = np.ascontiguousarray(accept_len, dtype=np.int32)
    bonus = np.zeros(B, dtype=np.int32)
    zr = np.zeros(B)
    resid = np.zeros((B, V)) if want_resid else None
    err = np.zeros(B, dtype=np.int32)
    exc = np.zeros(B, dtype=np.uint8)
    e2 = np.zeros((B, 4))
    eps = CDF_TIE_EPS if cdf_eps is None else cdf_eps
    lib().orc_residual_sample(B, K, V, ld, code, _base(zp), _base(zq), T, _ptr(pm), _ptr(ps), _ptr(pa),
                              _ptr(qm), _ptr(qs), _ptr(qa), _ptr(F), int(F.sum()), _ptr(cache_ids),
                              _ptr(Z), C, _ptr(accept_len), seed, round_, b_base, eps, _ptr(bonus), _ptr(zr),
                              _ptr(resid), _ptr(err), _ptr(exc), _ptr(e2))
    if want_bands:
        return bonus, zr, resid, err, exc, e2
    return bonus, zr, resid, err, exc


def cache_lookup(K, V, F, cache_ids, accept_len, bonus, fallback_uniform, seed, round_, b_base: int = 0):
    F = np.ascontiguousarray(F, dtype=np.int32)
    cache_ids = np.ascontiguousarray(cache_ids, dtype=np.int32)
    accept_len = np.ascontiguousarray(accept_len, dtype=np.int32)
    bonus = np.ascontiguousarray(bonus, dtype=np.int32)
    B = accept_len.shape[0]
    hit = np.zeros(B, dtype=np.uint8)
    slot = np.zeros(B, dtype=np.int32)
    fb = np.zeros((B, K), dtype=np.int32)
    err = np.zeros(B, dtype=np.int32)
    lib().orc_cache_lookup(B, K, V, _ptr(F), int(F.sum()), _ptr(cache_ids), _ptr(accept_len), _ptr(bonus),
                           int(bool(fallback_uniform)), seed, round_, b_base, _ptr(hit), _ptr(slot), _ptr(fb),
                           _ptr(err))
    return hit, slot, fb, err


def cache_gather(values, hit, slot, fallback_tokens):
    """Next round's draft [B, K] from the value store values [B, Bf, K] (int32): the
    cached continuation on a hit, the fallback tokens on a miss."""
    values = np.ascontiguousarray(values, dtype=np.int32)
    hit = np.ascontiguousarray(hit, dtype=np.uint8)
    slot = np.ascontiguousarray(slot, dtype=np.int32)
    fallback_tokens = np.ascontiguousarray(fallback_tokens, dtype=np.int32)
    B, Bf, K = values.shape
    nd = np.zeros((B, K), dtype=np.int32)
    err = np.zeros(B, dtype=np.int32)
    lib().orc_cache_gather(B, K, Bf, _ptr(values), _ptr(hit), _ptr(slot), _ptr(fallback_tokens), _ptr(nd),
                           _ptr(err))
    return nd, err


def ngram_fallback(K, V, hist, hist_len, draft, accept_len, bonus, hit, n_min, n_max, seed, round_,
                   b_base: int = 0, next_draft=None):
    """n-gram fallback speculator (prompt lookup over the context hist[b, :len_b] ++
    draft[b, :k] ++ [bonus]; see ``orc_ngram_fallback`` for the reading).  hist is
    int32 [B, ld_hist]; hit (uint8 [B]) or None (every sequence served).  Returns
    (tokens [B, K], match_n [B], match_end [B], err [B]); next_draft, when given, is
    updated in place for the served sequences."""
    hist = np.ascontiguousarray(hist, dtype=np.int32)
    B, ld = hist.shape
    hist_len = np.ascontiguousarray(hist_len, dtype=np.int32)
    draft = np.ascontiguousarray(draft, dtype=np.int32).reshape(B, K)
    accept_len = np.ascontiguousarray(accept_len, dtype=np.int32)
    bonus = np.ascontiguousarray(bonus, dtype=np.int32)
    hit_a = None if hit is None else np.ascontiguousarray(hit, dtype=np.uint8)
    if next_draft is not None:
        assert next_draft.dtype == np.int32 and next_draft.shape == (B, K) and next_draft.flags.c_contiguous
    tokens = np.zeros((B, K), dtype=np.int32)
    mn = np.zeros(B, dtype=np.int32)
    me = np.zeros(B, dtype=np.int32)
    err = np.zeros(B, dtype=np.int32)
    lib().orc_ngram_fallback(B, K, V, _ptr(hist), ld, _ptr(hist_len), _ptr(draft), _ptr(accept_len), _ptr(bonus),
                             _ptr(hit_a), n_min, n_max, seed, round_, b_base, _ptr(tokens), _ptr(next_draft),
                             _ptr(mn), _ptr(me), _ptr(err))
    return tokens, mn, me, err


def bonus_rank(zq, accept_len, bonus, R: int, hist=None):
    """Rank of each bonus token within draft row k = accept_len (cache order: larger
    logit first, ties to the lower id), -1 for an invalid (k, bonus); and the
    coverage histogram hist[K+1, R+1] (uint32, bin R = rank >= R), accumulated into
    `hist` when given."""
    code, B, K, V, ld = _logit_info(zq)
    accept_len = np.ascontiguousarray(accept_len, dtype=np.int32)
    bonus = np.ascontiguousarray(bonus, dtype=np.int32)
    rank = np.zeros(B, dtype=np.int32)
    if hist is None:
        hist = np.zeros((K + 1, R + 1), dtype=np.uint32)
    assert hist.dtype == np.uint32 and hist.shape == (K + 1, R + 1) and hist.flags.c_contiguous
    lib().orc_bonus_rank(B, K, V, ld, code, _base(zq), _ptr(accept_len), _ptr(bonus), R, _ptr(rank), _ptr(hist))
    return rank, hist


def fanout_optimize(hist, Bf: int, Fmax: int):
    """Fan-out that maximises the number of hits the coverage histogram predicts
    ([zh] section 2 Challenge 1 and [nl] section 3 A: the fan-out solves a
    constrained optimisation; the objective is a reading).

    hist [K+1, R+1]: sequences verified with acceptance length k whose bonus had rank
    j in the draft row k (bin R: rank >= R).  Caching F_k candidates at length k
    catches the ranks below F_k, so the predicted hits are
        H(F) = sum_k sum_{j < F_k} hist[k, j],
    maximised over integers 0 <= F_k <= min(Fmax, R) with sum_k F_k = Bf.  Among
    maximisers the lexicographically largest F (most candidates at the shortest
    lengths) is returned.  Exact integer dynamic programme over (k, budget left),
    written as plain loops.  Returns (F int32 [K+1], predicted hits, total count);
    None when Bf exceeds (K+1) * min(Fmax, R)."""
    hist = np.asarray(hist)
    K1, R1 = hist.shape
    R = R1 - 1
    cap = min(Fmax, R)
    if Bf < 0 or Bf > K1 * cap:
        return None
    # cov[k][f] = hits caught at length k by caching f candidates
    cov = [[0] * (cap + 1) for _ in range(K1)]
    for k in range(K1):
        run = 0
        for f in range(1, cap + 1):
            run += int(hist[k, f - 1])
            cov[k][f] = run
    # best[k][b]: most hits from lengths k..K with exactly b candidates (None: infeasible)
    best = [[None] * (Bf + 1) for _ in range(K1 + 1)]
    best[K1][0] = 0
    for k in range(K1 - 1, -1, -1):
        for b in range(Bf + 1):
            top = None
            for f in range(0, min(cap, b) + 1):
                rest = best[k + 1][b - f]
                if rest is None:
                    continue
                v = cov[k][f] + rest
                if top is None or v > top:
                    top = v
            best[k][b] = top
    F = np.zeros(K1, dtype=np.int32)
    b = Bf
    for k in range(K1):
        for f in range(min(cap, b), -1, -1):  # largest f that stays optimal
            rest = best[k + 1][b - f]
            if rest is not None and cov[k][f] + rest == best[k][b]:
                F[k] = f
                b -= f
                break
    return F, int(best[0][Bf]), int(hist.sum())


def fallback_throughputs(model, h):
    """Expected tokens per unit time of each fallback speculator for one round of a
    batch with hit probabilities h [B] ([zh] section 2 Challenge 3 and [nl] section
    3 C: on a miss the whole batch waits for the fallback; slow and accurate for
    small batches, fast and weak for large ones; the formula is a reading):
        P(any miss) = 1 - prod_b h_b
        time(f)     = t_verify + P(any miss) * t_f
        tokens(f)   = sum_b [h_b n_hit + (1 - h_b) n_f]
    model: mapping with t_verify, t_primary, t_random, n_hit, n_primary, n_random.
    Returns (primary, random)."""
    all_hit, hit_sum = 1.0, 0.0
    for hb in h:
        all_hit *= float(hb)
        hit_sum += float(hb)
    p_miss = 1.0 - all_hit
    miss_sum = len(h) - hit_sum
    out = []
    for t_f, n_f in ((model["t_primary"], model["n_primary"]), (model["t_random"], model["n_random"])):
        tokens = hit_sum * model["n_hit"] + miss_sum * n_f
        out.append(tokens / (model["t_verify"] + p_miss * t_f))
    return out[0], out[1]


def fallback_choose(model, h):
    """FALLBACK_UNIFORM (random tokens) when its throughput is strictly higher, else
    FALLBACK_NONE (the primary speculator)."""
    tp, tr = fallback_throughputs(model, h)
    return (FALLBACK_UNIFORM if tr > tp else FALLBACK_NONE), tp, tr


def fallback_critical_batch(model, h: float, b_max: int) -> int:
    """The smallest batch size b <= b_max whose batch of b sequences with hit
    probability h prefers random tokens; 0 if none (b*, read from [nl] section 3 C)."""
    for b in range(1, b_max + 1):
        if fallback_choose(model, [h] * b)[0] == FALLBACK_UNIFORM:
            return b
    return 0


@dataclass
class RoundResult:
    p_max: np.ndarray
    p_sum: np.ndarray
    p_arg: np.ndarray
    q_max: np.ndarray
    q_sum: np.ndarray
    q_arg: np.ndarray
    cache_ids: np.ndarray
    cache_mass: np.ndarray
    Z: np.ndarray
    accept_len: np.ndarray
    accept_prob: np.ndarray
    bonus: np.ndarray
    resid_mass: np.ndarray
    hit: np.ndarray
    slot: np.ndarray
    fallback_tokens: np.ndarray
    err: np.ndarray
    exc: np.ndarray
    e2: np.ndarray  # [B, 4]: gap and band of each of the bonus draw's two uniforms


def round_(zp, zq, T, F, C, draft, seed, round_idx, fallback_uniform, fanout_gap=None,
           b_base: int = 0, cdf_eps: float = None) -> RoundResult:
    """One whole round in the method's order.  ``exc`` holds the per-sequence
    exception bits E1..E5 decided from the oracle's own fp64 values."""
    code, B, K, V, ld = _logit_info(zp)
    code2, B2, K2, V2, ld2 = _logit_info(zq)
    if (code, B, K, V, ld) != (code2, B2, K2, V2, ld2):
        raise ValueError("p and q logits must have the same layout")
    F = np.ascontiguousarray(F, dtype=np.int32)
    Bf = int(F.sum())
    draft = np.ascontiguousarray(draft, dtype=np.int32)
    R = (B, K + 1)
    out = RoundResult(
        p_max=np.zeros(R), p_sum=np.zeros(R), p_arg=np.zeros(R, np.int32),
        q_max=np.zeros(R), q_sum=np.zeros(R), q_arg=np.zeros(R, np.int32),
        cache_ids=np.zeros((B, Bf), np.int32), cache_mass=np.zeros(R), Z=np.zeros(R),
        accept_len=np.zeros(B, np.int32), accept_prob=np.zeros((B, K)), bonus=np.zeros(B, np.int32),
        resid_mass=np.zeros(B), hit=np.zeros(B, np.uint8), slot=np.zeros(B, np.int32),
        fallback_tokens=np.zeros((B, K), np.int32), err=np.zeros(B, np.int32), exc=np.zeros(B, np.uint8),
        e2=np.zeros((B, 4)))
    o = out
    eps = CDF_TIE_EPS if cdf_eps is None else cdf_eps
    lib().orc_round(B, K, V, ld, code, _base(zp), _base(zq), T, _ptr(F), Bf, C, _ptr(draft), seed,
                    round_idx, b_base, eps, int(bool(fallback_uniform)), _ptr(o.p_max), _ptr(o.p_sum), _ptr(o.p_arg),
                    _ptr(o.q_max), _ptr(o.q_sum), _ptr(o.q_arg), _ptr(o.cache_ids), _ptr(o.cache_mass),
                    _ptr(o.Z), _ptr(o.accept_len), _ptr(o.accept_prob), _ptr(o.bonus), _ptr(o.resid_mass),
                    _ptr(o.hit), _ptr(o.slot), _ptr(o.fallback_tokens), _ptr(o.err), _ptr(o.exc),
                    _ptr(o.e2))
    if fanout_gap is not None and fanout_gap < FANOUT_EPS:
        o.exc |= E4_FANOUT_TIE
    return out
