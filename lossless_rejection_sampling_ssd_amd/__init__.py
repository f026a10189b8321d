"""MI355X (gfx950) verify-and-pre-speculate round of Speculative Speculative Decoding
(Saguaro): a thin ctypes binding of the C ABI in ``include/ssd.h``.

Every function here has the name of the C entry point it marshals to and only
turns torch tensors into pointers; every step of the round runs in the HIP kernels
of ``liblrs_ssd.so``.  PyTorch provides device memory and streams.  There is no
CPU fallback: importing the package fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch  # the process's HIP runtime must be torch's before the library loads

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblrs_ssd.so")

SSD_OK, SSD_ERR_ARG, SSD_ERR_UNSUPPORTED, SSD_ERR_HIP, SSD_ERR_WORKSPACE = 0, 1, 2, 3, 4
SSD_F32, SSD_BF16 = 0, 1
SSD_FALLBACK_NONE, SSD_FALLBACK_UNIFORM = 0, 1
SSD_DEVERR_TOKEN_RANGE, SSD_DEVERR_QPRIME_ZERO, SSD_DEVERR_LEN_RANGE, SSD_DEVERR_SLOT_RANGE = 1, 2, 4, 8
SSD_DEVERR_HIST_RANGE = 16
SSD_MAX_K, SSD_MAX_F, SSD_MAX_NGRAM = 16, 64, 16
SSD_NOALLOC_SCRATCH_BYTES = 96 << 20

EXPORTED = ("ssd_fanout", "ssd_workspace_bytes", "ssd_softmax", "ssd_build_cache", "ssd_saguaro_reweight",
            "ssd_verify", "ssd_residual_sample", "ssd_cache_lookup", "ssd_cache_gather", "ssd_ngram_fallback",
            "ssd_round", "ssd_round_devrng", "ssd_round_noalloc", "ssd_bonus_rank", "ssd_fanout_optimize", "ssd_fallback_choose",
            "ssd_fallback_critical_batch", "ssd_stream_read", "ssd_status_string", "ssd_last_error")


class SSDError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        super().__init__("%s failed: %s%s" % (where, _status_text(status), (" (" + detail + ")") if detail else ""))


class ssd_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("ld", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("T", ctypes.c_float)]


class ssd_rng(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("round", ctypes.c_uint64)]


_P = ctypes.c_void_p


class ssd_round_out(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("p_max", "p_sum", "p_argmax", "q_max", "q_sum", "q_argmax", "cache_ids",
                                  "cache_mass", "Z", "accept_len", "accept_prob", "bonus", "resid_mass", "hit",
                                  "slot", "fallback_tokens", "dev_err", "cache_values", "next_draft")]


class ssd_fallback_model(ctypes.Structure):
    _fields_ = [(n, ctypes.c_double) for n in ("t_verify", "t_primary", "t_random", "n_hit", "n_primary",
                                               "n_random")]


class ssd_round_events(ctypes.Structure):
    _fields_ = [("pass1_start", _P), ("pass1_stop", _P), ("pass2_start", _P), ("pass2_stop", _P)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("liblrs_ssd.so is not built (run __graft_entry__.build() or "
                          "python lossless_rejection_sampling_ssd_amd/build.py); there is no CPU fallback")
    L = ctypes.CDLL(LIB_PATH)
    i32, u64, f32, f64, sz = ctypes.c_int32, ctypes.c_uint64, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
    S = ctypes.POINTER(ssd_shape)
    L.ssd_fanout.argtypes = [i32, i32, f64, _P]
    L.ssd_workspace_bytes.argtypes = [S, i32]
    L.ssd_workspace_bytes.restype = sz
    L.ssd_softmax.argtypes = [S, _P, _P, _P, _P, _P, _P, sz, _P]
    L.ssd_build_cache.argtypes = [S, _P, _P, _P, _P, i32, _P, _P, _P, sz, _P]
    L.ssd_saguaro_reweight.argtypes = [S, _P, f32, _P, _P, _P, _P, _P, _P, i32, _P, _P, ssd_rng, _P, _P, sz, _P]
    L.ssd_verify.argtypes = [S, _P, _P, _P, _P, _P, _P, _P, _P, _P, i32, _P, _P, f32, ssd_rng, _P, _P, _P, _P]
    L.ssd_residual_sample.argtypes = [S, _P, _P, _P, _P, _P, _P, _P, _P, i32, _P, _P, f32, _P, ssd_rng, _P, _P, _P,
                                      _P, sz, _P]
    L.ssd_cache_gather.argtypes = [i32, i32, i32, _P, _P, _P, _P, _P, _P, _P]
    L.ssd_ngram_fallback.argtypes = [i32, i32, i32, _P, ctypes.c_int64, _P, _P, _P, _P, _P, i32, i32, ssd_rng,
                                     _P, _P, _P, _P, _P, _P]
    L.ssd_cache_lookup.argtypes = [i32, i32, i32, _P, i32, _P, _P, _P, i32, ssd_rng, _P, _P, _P, _P, _P]
    L.ssd_round.argtypes = [S, _P, _P, _P, _P, i32, f32, ssd_rng, i32, ctypes.POINTER(ssd_round_out),
                            ctypes.POINTER(ssd_round_events), _P, sz, _P]
    L.ssd_round_devrng.argtypes = [S, _P, _P, _P, _P, i32, f32, u64, _P, i32, ctypes.POINTER(ssd_round_out),
                                   ctypes.POINTER(ssd_round_events), _P, sz, _P]
    L.ssd_round_noalloc.argtypes = [S, _P, _P, _P, _P, i32, f32, ssd_rng, i32, ctypes.POINTER(ssd_round_out),
                                    ctypes.POINTER(ssd_round_events), _P]
    L.ssd_bonus_rank.argtypes = [S, _P, _P, _P, i32, _P, _P, _P, sz, _P]
    L.ssd_fanout_optimize.argtypes = [i32, i32, i32, i32, _P, _P, _P, _P]
    FM = ctypes.POINTER(ssd_fallback_model)
    L.ssd_fallback_choose.argtypes = [FM, i32, _P, _P, _P, _P]
    L.ssd_fallback_critical_batch.argtypes = [FM, f64, i32, _P]
    L.ssd_stream_read.argtypes = [_P, sz, _P, _P]
    L.ssd_status_string.argtypes = [i32]
    L.ssd_status_string.restype = ctypes.c_char_p
    L.ssd_last_error.argtypes = []
    L.ssd_last_error.restype = ctypes.c_char_p
    for name in ("ssd_fanout", "ssd_softmax", "ssd_build_cache", "ssd_saguaro_reweight", "ssd_verify",
                 "ssd_residual_sample", "ssd_cache_lookup", "ssd_cache_gather", "ssd_ngram_fallback", "ssd_round",
                 "ssd_round_devrng", "ssd_round_noalloc", "ssd_bonus_rank", "ssd_fanout_optimize", "ssd_fallback_choose", "ssd_fallback_critical_batch",
                 "ssd_stream_read"):
        getattr(L, name).restype = i32
    return L


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def _status_text(st: int) -> str:
    return _lib.ssd_status_string(st).decode()


def _check(st: int, where: str):
    if st != SSD_OK:
        raise SSDError(st, where, _lib.ssd_last_error().decode() if st == SSD_ERR_HIP else "")


# ---------------------------------------------------------------------------- marshalling
def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if dtype is not None and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _host_F(F: Sequence[int]):
    arr = (ctypes.c_int32 * len(F))(*[int(x) for x in F])
    return arr


def shape_of(logits: torch.Tensor, T: float) -> ssd_shape:
    """The ssd_shape of a [B, K+1, V] logit tensor (rows unit-stride, uniform row
    stride ld >= V) at temperature T."""
    if logits.dim() != 3:
        raise ValueError("logits must be [B, K+1, V]")
    if logits.dtype == torch.float32:
        dt = SSD_F32
    elif logits.dtype == torch.bfloat16:
        dt = SSD_BF16
    else:
        raise TypeError("logits must be float32 or bfloat16")
    B, K1, V = logits.shape
    if logits.stride(2) != 1 or logits.stride(0) != logits.stride(1) * K1:
        raise ValueError("logits rows must be unit-stride with one uniform row stride")
    return ssd_shape(B, K1 - 1, V, logits.stride(1), dt, float(T))


def _logit_ptr(t: torch.Tensor, name: str):
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    return ctypes.c_void_p(t.data_ptr())


class Workspace:
    """Caller-owned, zero-initialised device workspace (torch memory) for the calls
    that need one.  Grows on demand.  Calls that overlap in time must not share one:
    use one per stream (the calls without ``ws`` do, keyed by device and stream)."""

    def __init__(self, device=None):
        self.device = device
        self.buf: Optional[torch.Tensor] = None
        self._stream = None  # stream the buffer was allocated on

    def get(self, nbytes: int, stream=None):
        s = torch.cuda.current_stream() if stream is None else stream
        if self.buf is None or self.buf.numel() < nbytes:
            old = self.buf
            if old is not None and self._stream is not None and s != self._stream:
                # kernels queued on the stream that last used it may still read the old
                # block: the allocator must not hand it out before they finish
                old.record_stream(s)
            with torch.cuda.stream(s):
                self.buf = torch.zeros(max(nbytes, 1) + 256, dtype=torch.uint8,
                                       device=self.device if self.device is not None else s.device)
            self._stream = s
        elif self._stream is not None and s != self._stream:
            self.buf.record_stream(s)  # used on another stream than it was allocated on
        base = self.buf.data_ptr()
        off = (-base) % 256
        return ctypes.c_void_p(base + off), self.buf.numel() - off


def _ws(ws: Optional[Workspace], shape: ssd_shape, Bf: int, stream=None):
    need = _lib.ssd_workspace_bytes(ctypes.byref(shape), int(Bf))
    if need == 0:
        raise SSDError(SSD_ERR_ARG, "ssd_workspace_bytes")
    if ws is None:
        ws = _default_ws(stream)
    return ws.get(need, stream)


_default = {}


def _default_ws(stream=None) -> Workspace:
    """The workspace of the calls given no ``ws``: one per (device, stream), so that
    calls on different streams never share scratch."""
    s = torch.cuda.current_stream() if stream is None else stream
    key = (s.device.index, s.cuda_stream)
    if key not in _default:
        _default[key] = Workspace(s.device)
    return _default[key]


# ---------------------------------------------------------------------------- entry points
def ssd_fanout(K: int, Bf: int, r: float):
    F = (ctypes.c_int32 * (K + 1))()
    _check(_lib.ssd_fanout(int(K), int(Bf), float(r), F), "ssd_fanout")
    return list(F)


def ssd_workspace_bytes(shape: ssd_shape, Bf: int) -> int:
    return int(_lib.ssd_workspace_bytes(ctypes.byref(shape), int(Bf)))


def ssd_softmax(shape, logits, row_max, row_sum, row_argmax=None, probs=None, ws=None, stream=None):
    args = (_logit_ptr(logits, "logits"), _ptr(row_max, torch.float32, "row_max"),
            _ptr(row_sum, torch.float64, "row_sum"), _ptr(row_argmax, torch.int32, "row_argmax"),
            _ptr(probs, torch.float32, "probs"))
    w, nb = _ws(ws, shape, 1, stream)
    _check(_lib.ssd_softmax(ctypes.byref(shape), *args, w, nb, _stream(stream)), "ssd_softmax")


def ssd_build_cache(shape, q_logits, q_max, q_sum, F, cache_ids, cache_mass, ws=None, stream=None):
    Bf = int(sum(F))
    w, nb = _ws(ws, shape, Bf, stream)
    _check(_lib.ssd_build_cache(ctypes.byref(shape), _logit_ptr(q_logits, "q_logits"), _ptr(q_max, torch.float32),
                                _ptr(q_sum, torch.float64), _host_F(F), Bf, _ptr(cache_ids, torch.int32, "cache_ids"),
                                _ptr(cache_mass, torch.float64, "cache_mass"), w, nb, _stream(stream)),
           "ssd_build_cache")


def ssd_saguaro_reweight(shape, cache_mass, C, Z, q_logits=None, q_max=None, q_sum=None, q_argmax=None, F=None,
                         cache_ids=None, q_prime=None, seed=0, round_=0, draft=None, ws=None, stream=None):
    Bf = int(sum(F)) if F is not None else 0
    w, nb = (None, 0)
    if draft is not None:
        w, nb = _ws(ws, shape, Bf, stream)
    _check(_lib.ssd_saguaro_reweight(ctypes.byref(shape), _ptr(cache_mass, torch.float64), float(C),
                                     _ptr(Z, torch.float64, "Z"),
                                     _logit_ptr(q_logits, "q_logits") if q_logits is not None else None,
                                     _ptr(q_max, torch.float32), _ptr(q_sum, torch.float64),
                                     _ptr(q_argmax, torch.int32), _host_F(F) if F is not None else None, Bf,
                                     _ptr(cache_ids, torch.int32), _ptr(q_prime, torch.float32, "q_prime"),
                                     ssd_rng(seed, round_), _ptr(draft, torch.int32, "draft"), w, nb,
                                     _stream(stream)), "ssd_saguaro_reweight")


def ssd_verify(shape, p_logits, q_logits, draft, p_max, p_sum, p_argmax, q_max, q_sum, F, cache_ids, Z, C, seed,
               round_, accept_len, accept_prob=None, dev_err=None, stream=None):
    Bf = int(sum(F))
    _check(_lib.ssd_verify(ctypes.byref(shape), _logit_ptr(p_logits, "p_logits"), _logit_ptr(q_logits, "q_logits"),
                           _ptr(draft, torch.int32, "draft"), _ptr(p_max, torch.float32), _ptr(p_sum, torch.float64),
                           _ptr(p_argmax, torch.int32), _ptr(q_max, torch.float32), _ptr(q_sum, torch.float64),
                           _host_F(F), Bf, _ptr(cache_ids, torch.int32), _ptr(Z, torch.float64), float(C),
                           ssd_rng(seed, round_), _ptr(accept_len, torch.int32, "accept_len"),
                           _ptr(accept_prob, torch.float32, "accept_prob"), _ptr(dev_err, torch.int32, "dev_err"),
                           _stream(stream)), "ssd_verify")


def ssd_residual_sample(shape, p_logits, q_logits, p_max, p_sum, p_argmax, q_max, q_sum, F, cache_ids, Z, C,
                        accept_len, seed, round_, bonus, resid_mass=None, dev_err=None, ws=None, stream=None):
    Bf = int(sum(F))
    w, nb = _ws(ws, shape, Bf, stream)
    _check(_lib.ssd_residual_sample(ctypes.byref(shape), _logit_ptr(p_logits, "p_logits"),
                                    _logit_ptr(q_logits, "q_logits"), _ptr(p_max, torch.float32),
                                    _ptr(p_sum, torch.float64), _ptr(p_argmax, torch.int32),
                                    _ptr(q_max, torch.float32), _ptr(q_sum, torch.float64), _host_F(F), Bf,
                                    _ptr(cache_ids, torch.int32), _ptr(Z, torch.float64), float(C),
                                    _ptr(accept_len, torch.int32, "accept_len"), ssd_rng(seed, round_),
                                    _ptr(bonus, torch.int32, "bonus"), _ptr(resid_mass, torch.float64),
                                    _ptr(dev_err, torch.int32), w, nb, _stream(stream)), "ssd_residual_sample")


def ssd_cache_lookup(B, K, V, F, cache_ids, accept_len, bonus, fallback, seed, round_, hit, slot, fallback_tokens,
                     dev_err=None, stream=None):
    Bf = int(sum(F))
    _check(_lib.ssd_cache_lookup(int(B), int(K), int(V), _host_F(F), Bf, _ptr(cache_ids, torch.int32),
                                 _ptr(accept_len, torch.int32), _ptr(bonus, torch.int32), int(fallback),
                                 ssd_rng(seed, round_), _ptr(hit, torch.uint8, "hit"), _ptr(slot, torch.int32, "slot"),
                                 _ptr(fallback_tokens, torch.int32, "fallback_tokens"), _ptr(dev_err, torch.int32),
                                 _stream(stream)), "ssd_cache_lookup")


def ssd_cache_gather(values, hit, slot, fallback_tokens, next_draft, dev_err=None, stream=None):
    """values [B, Bf, K] int32 -> next_draft [B, K] (device tensors)."""
    B, Bf, K = (int(x) for x in values.shape)
    _check(_lib.ssd_cache_gather(B, K, Bf, _ptr(values, torch.int32), _ptr(hit, torch.uint8, "hit"),
                                 _ptr(slot, torch.int32, "slot"), _ptr(fallback_tokens, torch.int32, "fallback_tokens"),
                                 _ptr(next_draft, torch.int32, "next_draft"), _ptr(dev_err, torch.int32),
                                 _stream(stream)), "ssd_cache_gather")


def ssd_ngram_fallback(V, hist, hist_len, draft, accept_len, bonus, n_min, n_max, seed, round_, fallback_tokens,
                       hit=None, next_draft=None, match_n=None, match_end=None, dev_err=None, stream=None):
    """n-gram fallback draft [B, K] for the sequences that missed (all when hit is
    None) from hist [B, ld_hist] (contiguous int32, row b valid up to hist_len[b])
    and the round's accepted tokens and bonus."""
    B, K = (int(x) for x in draft.shape)
    ld = int(hist.shape[1])
    _check(_lib.ssd_ngram_fallback(B, K, int(V), _ptr(hist, torch.int32, "hist") if ld > 0 else None, ld,
                                   _ptr(hist_len, torch.int32, "hist_len"),
                                   _ptr(draft, torch.int32, "draft"), _ptr(accept_len, torch.int32, "accept_len"),
                                   _ptr(bonus, torch.int32, "bonus"), _ptr(hit, torch.uint8, "hit"), int(n_min),
                                   int(n_max), ssd_rng(seed, round_),
                                   _ptr(fallback_tokens, torch.int32, "fallback_tokens"),
                                   _ptr(next_draft, torch.int32, "next_draft"), _ptr(match_n, torch.int32, "match_n"),
                                   _ptr(match_end, torch.int32, "match_end"), _ptr(dev_err, torch.int32),
                                   _stream(stream)), "ssd_ngram_fallback")


def ssd_bonus_rank(shape, q_logits, accept_len, bonus, R, rank_out=None, rank_hist=None, ws=None, stream=None):
    """Rank of each bonus within draft row accept_len (rank_out [B] int32) and the
    coverage histogram rank_hist [K+1, R+1] (int32 tensor holding uint32 counts,
    accumulated)."""
    _check(_lib.ssd_bonus_rank(ctypes.byref(shape), _logit_ptr(q_logits, "q_logits"),
                               _ptr(accept_len, torch.int32, "accept_len"), _ptr(bonus, torch.int32, "bonus"),
                               int(R), _ptr(rank_out, torch.int32, "rank_out"),
                               _ptr(rank_hist, torch.int32, "rank_hist"), *_ws(ws, shape, 1, stream), _stream(stream)),
           "ssd_bonus_rank")


def ssd_fanout_optimize(K: int, Bf: int, Fmax: int, hist):
    """Host: the fan-out [K+1] maximising the hits predicted by hist [K+1, R+1]
    (any integer array-like); returns (F, hits, total)."""
    import numpy as np
    h = np.ascontiguousarray(np.asarray(hist), dtype=np.uint32)
    if h.ndim != 2 or h.shape[0] != K + 1:
        raise ValueError("hist must be [K+1, R+1]")
    F = (ctypes.c_int32 * (K + 1))()
    hits, total = ctypes.c_uint64(), ctypes.c_uint64()
    _check(_lib.ssd_fanout_optimize(int(K), int(Bf), int(Fmax), h.shape[1] - 1, h.ctypes.data_as(_P), F,
                                    ctypes.byref(hits), ctypes.byref(total)), "ssd_fanout_optimize")
    return list(F), int(hits.value), int(total.value)


def ssd_fallback_choose(model: "ssd_fallback_model", h):
    """Host: SSD_FALLBACK_NONE or SSD_FALLBACK_UNIFORM for hit probabilities h [B];
    returns (choice, tokens/time with the primary speculator, with random tokens)."""
    import numpy as np
    hv = np.ascontiguousarray(np.asarray(h, dtype=np.float64).reshape(-1))
    choice = ctypes.c_int32()
    tp, tr = ctypes.c_double(), ctypes.c_double()
    _check(_lib.ssd_fallback_choose(ctypes.byref(model), hv.size, hv.ctypes.data_as(_P), ctypes.byref(choice),
                                    ctypes.byref(tp), ctypes.byref(tr)), "ssd_fallback_choose")
    return int(choice.value), tp.value, tr.value


def ssd_fallback_critical_batch(model: "ssd_fallback_model", h: float, b_max: int) -> int:
    """Host: the smallest batch size at which random tokens beat the primary
    speculator (0: none up to b_max)."""
    b = ctypes.c_int32()
    _check(_lib.ssd_fallback_critical_batch(ctypes.byref(model), float(h), int(b_max), ctypes.byref(b)),
           "ssd_fallback_critical_batch")
    return int(b.value)


def ssd_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Measurement: one read-only pass over the bytes of the contiguous device tensor
    buf in the vocabulary pass's access shape (sink: a one-element int32 device
    tensor the kernel almost never writes)."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.ssd_stream_read(_logit_ptr(buf, "buf"), nbytes - nbytes % 16, _ptr(sink, torch.int32, "sink"),
                                _stream(stream)), "ssd_stream_read")


_ROUND_DTYPES = {"p_max": torch.float32, "p_sum": torch.float64, "p_argmax": torch.int32, "q_max": torch.float32,
                 "q_sum": torch.float64, "q_argmax": torch.int32, "cache_ids": torch.int32,
                 "cache_mass": torch.float64, "Z": torch.float64, "accept_len": torch.int32,
                 "accept_prob": torch.float32, "bonus": torch.int32, "resid_mass": torch.float64,
                 "hit": torch.uint8, "slot": torch.int32, "fallback_tokens": torch.int32, "dev_err": torch.int32,
                 "cache_values": torch.int32, "next_draft": torch.int32}


def make_round_out(**tensors) -> ssd_round_out:
    """An ssd_round_out from named device tensors (missing names stay NULL)."""
    out = ssd_round_out()
    for name, t in tensors.items():
        if name not in _ROUND_DTYPES:
            raise KeyError(name)
        if t is not None:
            setattr(out, name, _ptr(t, _ROUND_DTYPES[name], name).value)
    return out


def ssd_round(shape, p_logits, q_logits, draft, F, C, seed, round_, fallback, out: ssd_round_out,
              events: Optional[ssd_round_events] = None, ws=None, stream=None):
    Bf = int(sum(F))
    w, nb = _ws(ws, shape, Bf, stream)
    _check(_lib.ssd_round(ctypes.byref(shape), _logit_ptr(p_logits, "p_logits"), _logit_ptr(q_logits, "q_logits"),
                          _ptr(draft, torch.int32, "draft"), _host_F(F), Bf, float(C), ssd_rng(seed, round_),
                          int(fallback), ctypes.byref(out), ctypes.byref(events) if events is not None else None,
                          w, nb, _stream(stream)), "ssd_round")


def ssd_round_devrng(shape, p_logits, q_logits, draft, F, C, seed, round_dev, fallback, out: ssd_round_out,
                     events: Optional[ssd_round_events] = None, ws=None, stream=None):
    """ssd_round with the round counter read from round_dev (a one-element int64
    device tensor holding the uint64 round) when the kernels run."""
    if round_dev.numel() != 1:
        raise ValueError("round_dev must hold one counter")
    Bf = int(sum(F))
    w, nb = _ws(ws, shape, Bf, stream)
    _check(_lib.ssd_round_devrng(ctypes.byref(shape), _logit_ptr(p_logits, "p_logits"),
                                 _logit_ptr(q_logits, "q_logits"), _ptr(draft, torch.int32, "draft"), _host_F(F), Bf,
                                 float(C), int(seed), _ptr(round_dev, torch.int64, "round_dev"), int(fallback),
                                 ctypes.byref(out), ctypes.byref(events) if events is not None else None, w, nb,
                                 _stream(stream)), "ssd_round_devrng")


def ssd_round_noalloc(shape, p_logits, q_logits, draft, F, C, seed, round_, fallback, out: ssd_round_out,
                      events: Optional[ssd_round_events] = None, stream=None):
    """ssd_round with its scratch in the library's static per-GPU array (no workspace,
    nothing allocated); calls that overlap in time on one GPU race."""
    st = _lib.ssd_round_noalloc(ctypes.byref(shape), _logit_ptr(p_logits, "p_logits"),
                                _logit_ptr(q_logits, "q_logits"), _ptr(draft, torch.int32, "draft"), _host_F(F),
                                int(sum(F)), float(C), ssd_rng(seed, round_), int(fallback), ctypes.byref(out),
                                ctypes.byref(events) if events is not None else None, _stream(stream))
    if st == SSD_ERR_WORKSPACE:
        raise SSDError(st, "ssd_round_noalloc", _lib.ssd_last_error().decode())
    _check(st, "ssd_round_noalloc")


# ---------------------------------------------------------------------------- convenience
class RoundBuffers:
    """Device output tensors of one fused round (all outputs materialised)."""

    def __init__(self, B: int, K: int, Bf: int, device=None, with_stats: bool = True, cache_values=None):
        dev = device or torch.cuda.current_device()
        R = B * (K + 1)
        f32, f64, i32 = torch.float32, torch.float64, torch.int32
        z = lambda n, dt: torch.zeros(n, dtype=dt, device=dev)  # noqa: E731
        self.t = {"cache_ids": z((B, max(Bf, 1)), i32), "accept_len": z(B, i32), "bonus": z(B, i32),
                  "hit": z(B, torch.uint8), "slot": z(B, i32), "fallback_tokens": z((B, K), i32),
                  "dev_err": z(B, i32), "accept_prob": z((B, K), f32), "resid_mass": z(B, f64),
                  "cache_mass": z(R, f64), "Z": z(R, f64)}
        if with_stats:
            self.t.update({"p_max": z(R, f32), "p_sum": z(R, f64), "p_argmax": z(R, i32), "q_max": z(R, f32),
                           "q_sum": z(R, f64), "q_argmax": z(R, i32)})
        if cache_values is not None:  # value store [B, Bf, K]: the round also writes the next draft
            self.t["next_draft"] = z((B, K), i32)
            self.values = cache_values
            self.out = make_round_out(cache_values=cache_values if Bf > 0 else None, **self.t)
        else:
            self.out = make_round_out(**self.t)

    def __getitem__(self, k):
        return self.t[k]
