"""The C-ABI library without a GPU: it loads, exports every symbol include/ssd.h
declares, its host-only fan-out matches the oracle, and every argument error is
reported on the host before any launch (no call here reaches a kernel)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

BAD = ctypes.c_void_p(0x1000)  # never dereferenced: each call below fails validation first


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(ssd_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def ssd():
    import lossless_rejection_sampling_ssd_amd as m
    return m


def test_exports_every_declared_symbol(ssd):
    names = _declared()
    assert "ssd_round" in names and "ssd_verify" in names and len(names) >= 11
    for n in names:
        assert hasattr(ssd.lib(), n), n
    assert set(names) == set(ssd.EXPORTED)


def test_status_strings(ssd):
    L = ssd.lib()
    assert L.ssd_status_string(0) == b"ok"
    assert L.ssd_status_string(1) == b"invalid argument"
    assert L.ssd_status_string(4) == b"workspace too small"


@pytest.mark.parametrize("K,Bf,r", [(4, 16, 0.7), (5, 32, 0.6), (8, 64, 0.7), (6, 96, 0.8), (4, 32, 0.5),
                                    (16, 1000, 0.93), (1, 0, 1.0), (3, 7, 0.2), (12, 40, 0.55)])
def test_host_fanout_matches_oracle(ssd, orc, K, Bf, r):
    F, gap = orc.fanout(K, Bf, r)
    if gap > orc.FANOUT_EPS:
        assert ssd.ssd_fanout(K, Bf, r) == F.tolist()


def test_fanout_rejects_bad_args(ssd):
    for args in [(0, 4, 0.5), (17, 4, 0.5), (4, -1, 0.5), (4, 4, 0.0), (4, 4, 1.5), (4, 4, float("nan"))]:
        with pytest.raises(ssd.SSDError) as ei:
            ssd.ssd_fanout(*args)
        assert ei.value.status == ssd.SSD_ERR_ARG


def _shape(ssd, B=2, K=3, V=100, ld=None, dtype=0, T=1.0):
    return ssd.ssd_shape(B, K, V, V if ld is None else ld, dtype, T)


def test_workspace_bytes(ssd):
    L = ssd.lib()
    s = _shape(ssd)
    assert L.ssd_workspace_bytes(ctypes.byref(s), 8) > 0
    for bad in [_shape(ssd, B=0), _shape(ssd, K=0), _shape(ssd, K=17), _shape(ssd, V=1), _shape(ssd, ld=50),
                _shape(ssd, dtype=3), _shape(ssd, T=-1.0), _shape(ssd, T=float("inf")), _shape(ssd, T=float("nan"))]:
        assert L.ssd_workspace_bytes(ctypes.byref(bad), 8) == 0
    # one pass-1 block per 4 tiles of each of the 2 B (K+1) rows: above 2^31 - 1 blocks
    # the shape is unsupported
    big = ssd.ssd_shape(1 << 30, 1, 100, 100, 0, 1.0)
    assert L.ssd_workspace_bytes(ctypes.byref(big), 8) == 0
    ok = ssd.ssd_shape(40000, 1, 100, 100, 0, 1.0)
    assert L.ssd_workspace_bytes(ctypes.byref(ok), 8) > 0


def _F(vals):
    return (ctypes.c_int32 * len(vals))(*vals)


def test_softmax_validation(ssd):
    L = ssd.lib()
    ws_ok = ctypes.c_void_p(0x100000)
    for s, lg, mx, sm, ws, nb, want in [
        (_shape(ssd, B=0), BAD, BAD, BAD, ws_ok, 1 << 30, ssd.SSD_ERR_ARG),
        (_shape(ssd, T=-0.5), BAD, BAD, BAD, ws_ok, 1 << 30, ssd.SSD_ERR_ARG),
        (_shape(ssd), None, BAD, BAD, ws_ok, 1 << 30, ssd.SSD_ERR_ARG),
        (_shape(ssd), BAD, None, BAD, ws_ok, 1 << 30, ssd.SSD_ERR_ARG),
        (_shape(ssd), BAD, BAD, None, ws_ok, 1 << 30, ssd.SSD_ERR_ARG),
        (_shape(ssd), BAD, BAD, BAD, None, 1 << 30, ssd.SSD_ERR_ARG),
        (_shape(ssd), BAD, BAD, BAD, ctypes.c_void_p(0x100010), 1 << 30, ssd.SSD_ERR_ARG),  # misaligned
        (_shape(ssd), BAD, BAD, BAD, ws_ok, 16, ssd.SSD_ERR_WORKSPACE),
        (_shape(ssd, K=20), BAD, BAD, BAD, ws_ok, 1 << 30, ssd.SSD_ERR_ARG),
    ]:
        assert L.ssd_softmax(ctypes.byref(s), lg, mx, sm, None, None, ws, nb, None) == want


def test_cache_and_round_validation(ssd):
    L = ssd.lib()
    s = _shape(ssd, K=3, V=100)
    ws = ctypes.c_void_p(0x100000)
    good_F = _F([3, 2, 2, 1])
    # sum F != Bf
    assert L.ssd_build_cache(ctypes.byref(s), BAD, BAD, BAD, good_F, 9, BAD, BAD, ws, 1 << 30, None) == ssd.SSD_ERR_ARG
    # negative share, share above V
    assert L.ssd_build_cache(ctypes.byref(s), BAD, BAD, BAD, _F([3, -1, 2, 4]), 8, BAD, BAD, ws, 1 << 30,
                             None) == ssd.SSD_ERR_ARG
    assert L.ssd_build_cache(ctypes.byref(s), BAD, BAD, BAD, _F([101, 0, 0, 0]), 101, BAD, BAD, ws, 1 << 30,
                             None) == ssd.SSD_ERR_ARG
    # share above the per-length limit of this build
    sV = _shape(ssd, K=3, V=1000)
    assert L.ssd_build_cache(ctypes.byref(sV), BAD, BAD, BAD, _F([65, 0, 0, 0]), 65, BAD, BAD, ws, 1 << 30,
                             None) == ssd.SSD_ERR_UNSUPPORTED
    # null F
    assert L.ssd_build_cache(ctypes.byref(s), BAD, BAD, BAD, None, 8, BAD, BAD, ws, 1 << 30, None) == ssd.SSD_ERR_ARG
    # Saguaro factor outside (0, 1]
    for C in (0.0, -0.5, 1.5, float("nan")):
        assert L.ssd_saguaro_reweight(ctypes.byref(s), BAD, C, BAD, None, None, None, None, None, 0, None, None,
                                      ssd.ssd_rng(0, 0), None, None, 0, None) == ssd.SSD_ERR_ARG
        assert L.ssd_verify(ctypes.byref(s), BAD, BAD, BAD, BAD, BAD, BAD, BAD, BAD, good_F, 8, BAD, BAD, C,
                            ssd.ssd_rng(0, 0), BAD, None, None, None) == ssd.SSD_ERR_ARG
    # greedy verify needs the target argmax
    s0 = _shape(ssd, K=3, V=100, T=0.0)
    assert L.ssd_verify(ctypes.byref(s0), BAD, BAD, BAD, BAD, BAD, None, BAD, BAD, good_F, 8, BAD, BAD, 0.5,
                        ssd.ssd_rng(0, 0), BAD, None, None, None) == ssd.SSD_ERR_ARG
    # the cached ids are read at every temperature: required whenever Bf > 0, greedy too
    for sv in (s0, s):
        assert L.ssd_verify(ctypes.byref(sv), BAD, BAD, BAD, BAD, BAD, BAD, BAD, BAD, good_F, 8, None, BAD, 0.5,
                            ssd.ssd_rng(0, 0), BAD, None, None, None) == ssd.SSD_ERR_ARG
    # dense outputs above 65535 rows are refused before anything is launched
    big = _shape(ssd, B=20000, K=3, V=100)
    assert L.ssd_softmax(ctypes.byref(big), BAD, BAD, BAD, None, BAD, ws, 1 << 40, None) == ssd.SSD_ERR_UNSUPPORTED
    assert L.ssd_saguaro_reweight(ctypes.byref(big), BAD, 0.5, BAD, BAD, BAD, BAD, None, good_F, 8, BAD, BAD,
                                  ssd.ssd_rng(0, 0), None, None, 0, None) == ssd.SSD_ERR_UNSUPPORTED
    # residual: missing outputs, small workspace
    assert L.ssd_residual_sample(ctypes.byref(s), BAD, BAD, BAD, BAD, BAD, BAD, BAD, good_F, 8, BAD, BAD, 0.5, BAD,
                                 ssd.ssd_rng(0, 0), None, None, None, ws, 1 << 30, None) == ssd.SSD_ERR_ARG
    assert L.ssd_residual_sample(ctypes.byref(s), BAD, BAD, BAD, BAD, BAD, BAD, BAD, good_F, 8, BAD, BAD, 0.5, BAD,
                                 ssd.ssd_rng(0, 0), BAD, None, None, ws, 8, None) == ssd.SSD_ERR_WORKSPACE
    # lookup: bad fallback mode, bad shape
    assert L.ssd_cache_lookup(2, 3, 100, good_F, 8, BAD, BAD, BAD, 7, ssd.ssd_rng(0, 0), BAD, BAD, BAD, None,
                              None) == ssd.SSD_ERR_ARG
    assert L.ssd_cache_lookup(2, 0, 100, good_F, 8, BAD, BAD, BAD, 0, ssd.ssd_rng(0, 0), BAD, BAD, BAD, None,
                              None) == ssd.SSD_ERR_ARG
    # fused round: required outputs missing, bad fallback
    out = ssd.ssd_round_out()
    assert L.ssd_round(ctypes.byref(s), BAD, BAD, BAD, good_F, 8, 0.5, ssd.ssd_rng(0, 0), 0, ctypes.byref(out), None,
                       ws, 1 << 30, None) == ssd.SSD_ERR_ARG
    for name in ("cache_ids", "accept_len", "bonus", "hit", "slot", "fallback_tokens"):
        setattr(out, name, 0x2000)
    assert L.ssd_round(ctypes.byref(s), BAD, BAD, BAD, good_F, 8, 0.5, ssd.ssd_rng(0, 0), 9, ctypes.byref(out), None,
                       ws, 1 << 30, None) == ssd.SSD_ERR_ARG
    assert L.ssd_round(ctypes.byref(s), BAD, BAD, None, good_F, 8, 0.5, ssd.ssd_rng(0, 0), 0, ctypes.byref(out), None,
                       ws, 1 << 30, None) == ssd.SSD_ERR_ARG
    assert L.ssd_round(ctypes.byref(s), BAD, BAD, BAD, good_F, 8, 0.5, ssd.ssd_rng(0, 0), 0, ctypes.byref(out), None,
                       ws, 64, None) == ssd.SSD_ERR_WORKSPACE
    # no-allocation round: the round's own checks come first; a shape whose scratch
    # exceeds the static array is refused before any HIP call, with both sizes
    assert L.ssd_round_noalloc(ctypes.byref(s), BAD, BAD, None, good_F, 8, 0.5, ssd.ssd_rng(0, 0), 0,
                               ctypes.byref(out), None, None) == ssd.SSD_ERR_ARG
    assert L.ssd_round_noalloc(ctypes.byref(s), BAD, BAD, BAD, good_F, 8, 0.5, ssd.ssd_rng(0, 0), 9,
                               ctypes.byref(out), None, None) == ssd.SSD_ERR_ARG
    huge = _shape(ssd, B=1024, K=8, V=128256, dtype=ssd.SSD_BF16)
    hF = _F([20, 14, 10, 7, 5, 3, 2, 2, 1])
    need = L.ssd_workspace_bytes(ctypes.byref(huge), 64)
    assert need > ssd.SSD_NOALLOC_SCRATCH_BYTES
    assert L.ssd_round_noalloc(ctypes.byref(huge), BAD, BAD, BAD, hF, 64, 0.5, ssd.ssd_rng(0, 0), 0,
                               ctypes.byref(out), None, None) == ssd.SSD_ERR_WORKSPACE
    msg = L.ssd_last_error().decode()
    assert str(need) in msg and str(ssd.SSD_NOALLOC_SCRATCH_BYTES) in msg, msg
    m = re.search(r"#define SSD_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << 20\)", open(HEADER).read())
    assert m and int(m.group(1)) << 20 == ssd.SSD_NOALLOC_SCRATCH_BYTES
    # device-side round counter: required
    assert L.ssd_round_devrng(ctypes.byref(s), BAD, BAD, BAD, good_F, 8, 0.5, 1, None, 0, ctypes.byref(out), None,
                              ws, 1 << 30, None) == ssd.SSD_ERR_ARG
    # fused round: a next draft with Bf > 0 needs the value store
    out.next_draft = 0x3000
    assert L.ssd_round(ctypes.byref(s), BAD, BAD, BAD, good_F, 8, 0.5, ssd.ssd_rng(0, 0), 0, ctypes.byref(out), None,
                       ws, 1 << 30, None) == ssd.SSD_ERR_ARG
    # gather: bad sizes, missing buffers, too many tokens for one launch
    for B, K, Bf, vals, nd in ((0, 4, 3, BAD, BAD), (2, 0, 3, BAD, BAD), (2, 17, 3, BAD, BAD), (2, 4, -1, BAD, BAD),
                               (2, 4, 3, None, BAD), (2, 4, 3, BAD, None)):
        assert L.ssd_cache_gather(B, K, Bf, vals, BAD, BAD, BAD, nd, None, None) == ssd.SSD_ERR_ARG
    assert L.ssd_cache_gather(1 << 28, 16, 3, BAD, BAD, BAD, BAD, BAD, None, None) == ssd.SSD_ERR_UNSUPPORTED
    # bonus rank: missing inputs, no output, R out of range, small workspace
    for q, acc, bon, R, ro, rh in ((None, BAD, BAD, 8, BAD, BAD), (BAD, None, BAD, 8, BAD, BAD),
                                   (BAD, BAD, None, 8, BAD, BAD), (BAD, BAD, BAD, 8, None, None),
                                   (BAD, BAD, BAD, 0, BAD, BAD), (BAD, BAD, BAD, 65, BAD, BAD)):
        assert L.ssd_bonus_rank(ctypes.byref(s), q, acc, bon, R, ro, rh, ws, 1 << 30, None) == ssd.SSD_ERR_ARG
    assert L.ssd_bonus_rank(ctypes.byref(s), BAD, BAD, BAD, 8, BAD, None, ws, 8, None) == ssd.SSD_ERR_WORKSPACE



def test_stream_read_validation(ssd):
    L = ssd.lib()
    for buf, nb, sink in ((None, 64, BAD), (BAD, 64, None), (BAD, 0, BAD), (BAD, 40, BAD),
                          (ctypes.c_void_p(0x1008), 64, BAD)):
        assert L.ssd_stream_read(buf, nb, sink, None) == ssd.SSD_ERR_ARG


def test_ngram_validation(ssd):
    """n-gram fallback: sizes, n-gram range and required pointers are checked on the
    host; a missing history is allowed only for ld_hist = 0."""
    L = ssd.lib()
    rng = ssd.ssd_rng(0, 0)

    def call(B=2, K=4, V=100, hist=BAD, ld=8, hl=BAD, dr=BAD, acc=BAD, bon=BAD, nmin=1, nmax=3, out=BAD):
        return L.ssd_ngram_fallback(B, K, V, hist, ld, hl, dr, acc, bon, None, nmin, nmax, rng, out, None, None,
                                    None, None, None)

    for kw in (dict(B=0), dict(K=0), dict(K=17), dict(V=1), dict(ld=-1), dict(hist=None), dict(hl=None),
               dict(dr=None), dict(acc=None), dict(bon=None), dict(out=None), dict(nmin=0), dict(nmin=4, nmax=3),
               dict(nmax=17)):
        assert call(**kw) == ssd.SSD_ERR_ARG, kw
    assert call(ld=(1 << 31) - 10) == ssd.SSD_ERR_UNSUPPORTED

def test_binding_refuses_host_tensors(ssd):
    import torch
    z = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        ssd.ssd_softmax(ssd.shape_of(z, 1.0), z, torch.zeros(2), torch.zeros(2))
    with pytest.raises(TypeError):
        ssd.shape_of(torch.zeros(1, 2, 8, dtype=torch.float16), 1.0)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and says why,
    before importing torch or touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
