"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI, run
the fp64 oracle on the same bits, and compare under the parity rules:
 - integer outputs bit-exact, except on sequences the oracle flags with its own fp64
   values: E1 (|u - p/q'| < 1e-5 at a tested position) and E5 (a tested p or q'
   below 1e-30 from a finite logit) exclude everything from the accepted length on;
   E2 (a uniform of a draw within its per-draw band of a CDF step around its pick, at
   the block or the id level) and
   E3 (residual mass below 1e-5) exclude the bonus, hit, slot and fallback tokens;
 - probabilities within 1e-5 absolute; row sums within 1e-5 relative; row maxima
   exact (they are input values)."""
import numpy as np
import torch

import oracle
import lossless_rejection_sampling_ssd_amd as ssd
from parity_cases import oracle_draft  # noqa: F401  (the harness's draft sampler)

PROB_ATOL = 1e-5
SUM_RTOL = 1e-5


def dev(t):
    return t.to("cuda")


def gpu_round(zp, zq, T, F, C, draft, seed, rnd, fallback, ws=None, values=None):
    """One fused round; values (numpy [B, Bf, K] int32) also asks for the next draft."""
    shape = ssd.shape_of(zp, T)
    B, K = shape.B, shape.K
    vals = None if values is None else torch.as_tensor(np.ascontiguousarray(values), device="cuda")
    buf = ssd.RoundBuffers(B, K, int(sum(F)), cache_values=vals)
    d = torch.as_tensor(np.ascontiguousarray(draft), dtype=torch.int32, device="cuda")
    ssd.ssd_round(shape, zp, zq, d, list(F), C, seed, rnd, fallback, buf.out, ws=ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in buf.t.items()}


def compare_round(g, o, K, Bf, check_stats=True, label="", values=None):
    """Asserts parity of a GPU fused round g (dict of numpy) with an oracle round o
    (oracle.RoundResult); with the value store values [B, Bf, K] also the next draft.
    Returns the number of flagged sequences."""
    B = o.accept_len.shape[0]
    R = B * (K + 1)
    if check_stats:
        assert np.array_equal(g["p_max"], o.p_max.reshape(R).astype(np.float32)), label
        assert np.array_equal(g["q_max"], o.q_max.reshape(R).astype(np.float32)), label
        np.testing.assert_allclose(g["p_sum"], o.p_sum.reshape(R), rtol=SUM_RTOL, err_msg=label)
        np.testing.assert_allclose(g["q_sum"], o.q_sum.reshape(R), rtol=SUM_RTOL, err_msg=label)
        assert np.array_equal(g["p_argmax"], o.p_arg.reshape(R)), label
        assert np.array_equal(g["q_argmax"], o.q_arg.reshape(R)), label
    if Bf > 0:
        assert np.array_equal(g["cache_ids"][:, :Bf], o.cache_ids), label
    np.testing.assert_allclose(g["cache_mass"], o.cache_mass.reshape(R), atol=PROB_ATOL, rtol=0, err_msg=label)
    np.testing.assert_allclose(g["Z"], o.Z.reshape(R), atol=PROB_ATOL, rtol=0, err_msg=label)
    np.testing.assert_allclose(g["accept_prob"], o.accept_prob, atol=PROB_ATOL, rtol=0, err_msg=label)
    assert np.array_equal(g["dev_err"], o.err), label
    e_len = (o.exc & (oracle.E1_ACCEPT_TIE | oracle.E5_TINY_PROB)) != 0
    e_any = o.exc != 0
    ok = ~e_len
    assert np.array_equal(g["accept_len"][ok], o.accept_len[ok]), (label, np.nonzero(g["accept_len"] != o.accept_len))
    same_k = g["accept_len"] == o.accept_len
    # E3: a residual mass below 1e-5 is decided by rounding (exactly 0 in the oracle's
    # fp64 selects the target law instead), so its value is not compared
    cmp_z = same_k & ((o.exc & oracle.E3_DEGENERATE_RESIDUAL) == 0)
    np.testing.assert_allclose(g["resid_mass"][cmp_z], o.resid_mass[cmp_z], atol=PROB_ATOL, rtol=0, err_msg=label)
    ok2 = ~e_any
    bad = np.nonzero((g["bonus"] != o.bonus) & ok2)[0]
    assert bad.size == 0, (label, "bonus", bad[:10], g["bonus"][bad[:10]], o.bonus[bad[:10]])
    assert np.array_equal(g["hit"][ok2], o.hit[ok2]), label
    assert np.array_equal(g["slot"][ok2], o.slot[ok2]), label
    assert np.array_equal(g["fallback_tokens"][ok2], o.fallback_tokens[ok2]), label
    if values is not None:
        nd, nerr = oracle.cache_gather(values, o.hit, o.slot, o.fallback_tokens)
        assert not nerr.any(), label
        assert np.array_equal(g["next_draft"][ok2], nd[ok2]), (label, "next_draft")
        # flagged sequences: the next draft still follows the GPU's own hit / slot
        nd_g, _ = oracle.cache_gather(values, g["hit"], g["slot"], g["fallback_tokens"])
        assert np.array_equal(g["next_draft"], nd_g), (label, "next_draft self")
    return int(e_any.sum())
