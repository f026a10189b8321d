"""The no-allocation round: ssd_round_noalloc, whose scratch is the library's static
per-GPU array, gives exactly the outputs of ssd_round with a caller workspace, on
two calls in a row, the second with a smaller input (then the first shape again, over
the scratch the smaller call left, then a larger batch whose bonus pass takes two tiles
per wave), and allocates nothing through torch."""
import pytest
import torch

import lossless_rejection_sampling_ssd_amd as ssd
from lossless_rejection_sampling_ssd_amd.workloads import WORKLOADS, make_logits, scaled

pytestmark = pytest.mark.gpu


def _inputs(w, buffer):
    zq, zp = make_logits(w, buffer=buffer, device="cuda")
    # drafts: the draft model's argmax per position (accepts often at T = 1), the last
    # sequence's drafts out of range to exercise the error bits
    draft = zq[:, :w.K].float().argmax(-1).to(torch.int32).contiguous()
    draft[-1, 0] = w.V + 3
    Fv = [int(x) for x in ssd.ssd_fanout(w.K, w.Bf, w.r)]
    g = torch.Generator(device="cuda")
    g.manual_seed(buffer + 5)
    values = torch.randint(0, w.V, (w.B, max(sum(Fv), 1), w.K), generator=g, device="cuda", dtype=torch.int32)
    return zq, zp, draft, Fv, values


def _run(w, T, zq, zp, draft, Fv, values, noalloc):
    buf = ssd.RoundBuffers(w.B, w.K, sum(Fv), cache_values=values)
    shape = ssd.shape_of(zp, T)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    if noalloc:
        ssd.ssd_round_noalloc(shape, zp, zq, draft, Fv, w.Cs[0], w.seed, 11, int(w.fallback_uniform), buf.out)
    else:
        ssd.ssd_round(shape, zp, zq, draft, Fv, w.Cs[0], w.seed, 11, int(w.fallback_uniform), buf.out)
    torch.cuda.synchronize()
    after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    return buf.t, after - before


def test_noalloc_matches_round():
    big = WORKLOADS["c3"]                                  # B=64 K=8 V=128256 bf16
    small = scaled(WORKLOADS["c2"], B=8, V=32001)          # fp32, odd vocabulary, 2 fewer positions
    large = WORKLOADS["c4"]                                # B=256 K=6: the two-tile bonus pass
    for w in (big, large):
        need = ssd.ssd_workspace_bytes(ssd.ssd_shape(w.B, w.K, w.V, w.V, ssd.SSD_BF16, 1.0), w.Bf)
        assert need <= ssd.SSD_NOALLOC_SCRATCH_BYTES
    for step, (w, T) in enumerate(((big, 1.0), (small, 0.7), (big, 1.0), (large, 1.2))):
        print("no-alloc step %d: %s B=%d K=%d V=%d %s T=%g" % (step, w.name, w.B, w.K, w.V, w.dtype, T), flush=True)
        zq, zp, draft, Fv, values = _inputs(w, step)
        ref, _ = _run(w, T, zq, zp, draft, Fv, values, noalloc=False)
        got, grew = _run(w, T, zq, zp, draft, Fv, values, noalloc=True)
        assert grew == 0, "ssd_round_noalloc allocated through torch"
        for k in ref:
            assert torch.equal(got[k], ref[k]), (step, k)
        acc = got["accept_len"]
        assert int(acc.min()) >= 0 and int(acc.max()) <= w.K
        assert int(got["dev_err"][-1]) & ssd.SSD_DEVERR_TOKEN_RANGE
        assert int((acc > 0).sum()) > 0, "no sequence accepted anything"
