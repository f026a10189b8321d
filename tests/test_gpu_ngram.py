"""Parity of the n-gram fallback speculator (HIP kernel through the C ABI) with the
oracle: proposals, match length and end, error bits and next draft bit-exact, on
synthetic histories with repeats, tiny alphabets, ragged and empty histories, long
histories and invalid inputs; and composed with the fused round's cache gather."""
import numpy as np
import pytest
import torch

import oracle
import lossless_rejection_sampling_ssd_amd as ssd
from lossless_rejection_sampling_ssd_amd.workloads import WORKLOADS, make_histories, make_logits, scaled, \
    to_oracle_array

from gpu_helpers import gpu_round, oracle_draft

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def _case(msg):
    print("\n[case] " + msg, flush=True)


def _spliced_tail(rng, hist, lens, K, V, frac=0.6):
    """draft [B, K], accept_len [B], bonus [B]: for a fraction of the sequences the
    accepted tokens and the bonus repeat a span of the history (so that a match
    exists), for the rest they are random ids."""
    B = hist.shape[0]
    draft = rng.integers(0, V, (B, K)).astype(np.int32)
    acc = rng.integers(0, K + 1, B).astype(np.int32)
    bonus = rng.integers(0, V, B).astype(np.int32)
    for b in range(B):
        n = int(lens[b])
        if n > K + 1 and rng.random() < frac:
            s = int(rng.integers(0, n - K - 1))
            draft[b] = hist[b, s:s + K]
            bonus[b] = hist[b, s + acc[b]]
    return draft, acc, bonus


def _run(V, hist, lens, draft, acc, bonus, hit, n_min, n_max, seed, rnd, next_draft=None):
    B, K = draft.shape
    d = lambda a, dt=torch.int32: torch.as_tensor(np.ascontiguousarray(a), dtype=dt, device="cuda")
    tok = torch.full((B, K), 7777, dtype=torch.int32, device="cuda")
    mn = torch.full((B,), 99, dtype=torch.int32, device="cuda")
    me = torch.full((B,), 99, dtype=torch.int32, device="cuda")
    err = torch.zeros(B, dtype=torch.int32, device="cuda")
    nd = None if next_draft is None else d(next_draft)
    hist_d = d(hist) if hist.shape[1] > 0 else torch.empty((B, 0), dtype=torch.int32, device="cuda")
    ssd.ssd_ngram_fallback(V, hist_d, d(lens), d(draft), d(acc), d(bonus), n_min, n_max, seed, rnd, tok,
                           hit=None if hit is None else d(hit, torch.uint8), next_draft=nd, match_n=mn,
                           match_end=me, dev_err=err)
    torch.cuda.synchronize()
    return (tok.cpu().numpy(), mn.cpu().numpy(), me.cpu().numpy(), err.cpu().numpy(),
            None if nd is None else nd.cpu().numpy())


def _check(V, hist, lens, draft, acc, bonus, hit, n_min, n_max, seed, rnd, label, with_next=True):
    B, K = draft.shape
    nd0 = np.full((B, K), 4242, np.int32) if with_next else None
    g_tok, g_n, g_e, g_err, g_nd = _run(V, hist, lens, draft, acc, bonus, hit, n_min, n_max, seed, rnd, nd0)
    o_nd = None if nd0 is None else nd0.copy()
    o_tok, o_n, o_e, o_err = oracle.ngram_fallback(K, V, hist, lens, draft, acc, bonus, hit, n_min, n_max, seed,
                                                   rnd, next_draft=o_nd)
    bad = np.nonzero((g_tok != o_tok).any(1) | (g_n != o_n) | (g_e != o_e))[0]
    assert bad.size == 0, (label, bad[:8], g_n[bad[:8]], o_n[bad[:8]], g_e[bad[:8]], o_e[bad[:8]])
    assert np.array_equal(g_err, o_err), label
    if with_next:
        assert np.array_equal(g_nd, o_nd), label
    return o_n


@pytest.mark.parametrize("B,K,L,V,n_min,n_max", [(512, 4, 4096, 151936, 2, 5), (64, 8, 2048, 128256, 1, 4),
                                                 (16, 16, 3000, 32000, 1, 16), (33, 1, 257, 32000, 3, 3)])
def test_ngram_synthetic_histories(B, K, L, V, n_min, n_max):
    _case("ngram synthetic B=%d K=%d L=%d V=%d n=%d..%d" % (B, K, L, V, n_min, n_max))
    hist, lens = make_histories(B, L, V, seed=0x55D0 + B)
    rng = np.random.default_rng(B * 31 + K)
    draft, acc, bonus = _spliced_tail(rng, hist, lens, K, V)
    hit = (rng.random(B) < 0.4).astype(np.uint8)
    n = _check(V, hist, lens, draft, acc, bonus, hit, n_min, n_max, 0x55D5, 3, "synthetic")
    served = hit == 0
    assert (n[served] > 0).any() and (n[served] == 0).any()  # both proposal kinds occur
    _check(V, hist, lens, draft, acc, bonus, None, n_min, n_max, 0x55D5, 4, "no hit mask", with_next=False)


@pytest.mark.parametrize("alphabet,ld", [(1, 700), (2, 700), (3, 700), (5, 700), (2, 20000), (4, 20000)])
def test_ngram_tiny_alphabets(alphabet, ld):
    """Many equal n-grams (ties on n broken by the latest end), ragged lengths from 0
    to past several 8192-end chunks (the scan stops after the chunk that reaches the
    longest possible match), every k."""
    _case("ngram tiny alphabet=%d ld=%d" % (alphabet, ld))
    rng = np.random.default_rng(alphabet + ld)
    B, K, V = 96, 6, 10
    hist = rng.integers(0, alphabet, (B, ld)).astype(np.int32)
    lens = rng.integers(0, ld + 1, B).astype(np.int32)
    lens[:6] = [0, 1, 2, 255, 256, min(8193, ld)]
    draft = rng.integers(0, alphabet, (B, K)).astype(np.int32)
    acc = rng.integers(0, K + 1, B).astype(np.int32)
    bonus = rng.integers(0, alphabet, B).astype(np.int32)
    for n_min, n_max in ((1, 1), (1, 16), (4, 9), (16, 16)):
        _check(V, hist, lens, draft, acc, bonus, None, n_min, n_max, 5, 6, "alphabet n=%d..%d" % (n_min, n_max))


def test_ngram_long_history_match_only_at_start():
    """Distinct tokens except a repeat of the final n-gram at the very start of a long
    history: the scan cannot stop early and must reach position 0."""
    _case("ngram long history")
    B, K, L, V = 8, 5, 70000, 1 << 20
    hist = np.tile(np.arange(100, 100 + L, dtype=np.int32), (B, 1))
    lens = np.full(B, L, np.int32)
    acc = np.zeros(B, np.int32)
    draft = np.zeros((B, K), np.int32)
    # context ends with [hist[L-2], hist[L-1], bonus]; plant that 3-gram at the start
    bonus = np.full(B, 5, np.int32)
    for b in range(B):
        hist[b, b:b + 3] = [hist[b, L - 2], hist[b, L - 1], 5]
    n = _check(V, hist, lens, draft, acc, bonus, None, 2, 6, 1, 1, "long")
    assert np.all(n == 3)


def test_ngram_invalid_inputs_and_empty_history():
    """accept_len outside [0, K] and history lengths outside [0, ld] set their error
    bits with tokens -1; ld_hist = 0 (no history) still matches within the draft."""
    _case("ngram invalid and empty")
    rng = np.random.default_rng(9)
    B, K, ld, V = 12, 4, 16, 50
    hist = rng.integers(0, 3, (B, ld)).astype(np.int32)
    lens = rng.integers(0, ld + 1, B).astype(np.int32)
    acc = rng.integers(0, K + 1, B).astype(np.int32)
    lens[0], lens[1], acc[2], acc[3] = -1, ld + 1, -2, K + 1
    draft = rng.integers(0, 3, (B, K)).astype(np.int32)
    bonus = rng.integers(0, 3, B).astype(np.int32)
    _check(V, hist, lens, draft, acc, bonus, None, 1, 3, 2, 2, "invalid")
    empty = np.zeros((B, 0), np.int32)
    acc2 = np.full(B, K, np.int32)
    _check(V, empty, np.zeros(B, np.int32), draft, acc2, bonus, None, 1, 3, 2, 2, "no history")


def test_ngram_after_fused_round():
    """The miss path of a whole round: the fused round (with the value store) writes
    the next draft of the hits, the n-gram speculator that of the misses; the result
    equals the oracle's round, gather and n-gram speculator in sequence."""
    _case("ngram after fused round (c5 recipe, B=64 V=20000)")
    w = scaled(WORKLOADS["c5"], B=64, V=20000)
    T, C = w.temps[0], w.Cs[0]
    F, gap = oracle.fanout(w.K, w.Bf, w.r)
    zq, zp = make_logits(w, buffer=0)
    zp_np, zq_np = to_oracle_array(zp), to_oracle_array(zq)
    draft, _ = oracle_draft(zp_np, zq_np, T, F, C, w.seed, 0)
    values = np.random.default_rng(w.seed).integers(0, w.V, (w.B, w.Bf, w.K)).astype(np.int32)
    g = gpu_round(zp.cuda(), zq.cuda(), T, F.tolist(), C, draft, w.seed, 0, 0, values=values)
    o = oracle.round_(zp_np, zq_np, T, F, C, draft, w.seed, 0, False, gap)
    ok = o.exc == 0
    assert np.array_equal(g["hit"][ok], o.hit[ok])
    hist, lens = make_histories(w.B, 1024, w.V, seed=w.seed)
    # GPU: n-gram speculator on the GPU round's own outcome, into its next draft
    d = lambda a, dt=torch.int32: torch.as_tensor(np.ascontiguousarray(a), dtype=dt, device="cuda")
    nd = d(g["next_draft"])
    tok = torch.zeros((w.B, w.K), dtype=torch.int32, device="cuda")
    ssd.ssd_ngram_fallback(w.V, d(hist), d(lens), d(draft), d(g["accept_len"]), d(g["bonus"]), 1, 4, w.seed, 0,
                           tok, hit=d(g["hit"], torch.uint8), next_draft=nd)
    torch.cuda.synchronize()
    # oracle: gather, then the n-gram speculator on the misses
    o_nd, _ = oracle.cache_gather(values, o.hit, o.slot, o.fallback_tokens)
    oracle.ngram_fallback(w.K, w.V, hist, lens, draft, o.accept_len, o.bonus, o.hit, 1, 4, w.seed, 0,
                          next_draft=o_nd)
    assert np.array_equal(nd.cpu().numpy()[ok], o_nd[ok])
    assert (o.hit[ok] == 0).any() and (o.hit[ok] == 1).any()
