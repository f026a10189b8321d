"""Seeded synthetic workloads for the verify-and-pre-speculate round.

This module only draws random logits; it holds none of the method's arithmetic (no
softmax, sampling, verification or cache logic), so both the HIP path and the
fp64 oracle can be fed from it.

The pages measure the method on real models (Llama-3.1-70B and Qwen-3-32B targets
with a Llama-3.2-1B draft, on math, code and chat data).  No model or dataset is
used here: the logits below are seeded Gaussian stand-ins with the shapes of those
model families' vocabularies (32000, 128256, 151936) and a draft/target
correlation that sets the acceptance regime of each workload.

Each workload gives draft logits ``zq`` and target logits ``zp`` of shape
``[B, K+1, V]`` (row i < K is position i of the draft block, row K is the position
after the last draft token).  bf16 workloads are drawn in fp32 and rounded to
nearest-even bf16 once; the oracle then receives the same bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence, Tuple

import torch

SEED_BASE = 0x55D0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    K: int
    V: int
    dtype: str                 # "f32" or "bf16"
    temps: Tuple[float, ...]   # temperatures the workload is run at
    Bf: int                    # cache budget
    r: float                   # geometric fan-out ratio
    Cs: Tuple[float, ...]      # Saguaro factors
    draft_sigma: float
    target_scale: float        # zp = target_scale * zq + N(0, target_sigma^2)
    target_sigmas: Tuple[float, ...]
    head_frac: float = 0.0     # fraction of ids boosted in the draft (Zipf-like head)
    head_boost: float = 0.0
    fallback_uniform: bool = False
    rounds: int = 1
    index: int = 0
    note: str = ""

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def label(self) -> str:
        return "B=%d K=%d V=%d %s" % (self.B, self.K, self.V, self.dtype)


WORKLOADS = {
    # 1 sequence, K=4, V=32000, fp32; draft N(0, 2^2), target = draft + N(0, 0.7^2);
    # T=1, r=0.7, Bf=16, C=0.5; 1000 rounds, each with its own logits and counter.
    "c1": Workload("c1", 1, 4, 32000, "f32", (1.0,), 16, 0.7, (0.5,), 2.0, 1.0, (0.7,),
                   rounds=1000, index=1, note="single sequence"),
    # B=16, K=5, V=32000, fp32; draft N(0, 2.5^2), target = 0.9 draft + N(0, 0.8^2);
    # T in {0 (greedy), 0.7, 1.0}; Bf=32, r=0.6, C=0.3.
    "c2": Workload("c2", 16, 5, 32000, "f32", (0.0, 0.7, 1.0), 32, 0.6, (0.3,), 2.5, 0.9, (0.8,),
                   index=2, note="temperature sweep incl. greedy"),
    # Headline: B=64, K=8, V=128256, bf16; draft N(0, 3^2) with 5% of ids boosted by +6,
    # target = draft + N(0, 1); T=1, Bf=64, r=0.7, C=0.5.
    "c3": Workload("c3", 64, 8, 128256, "bf16", (1.0,), 64, 0.7, (0.5,), 3.0, 1.0, (1.0,),
                   head_frac=0.05, head_boost=6.0, index=3, note="headline"),
    # B=256, K=6, V=128256, bf16; draft as c3; target noise swept for mean
    # sum(min(p, q)) of about {0.5, 0.7, 0.9} at T=1.2; Bf=96, r=0.8, C in {0.2, 0.5, 0.8}.
    "c4": Workload("c4", 256, 6, 128256, "bf16", (1.2,), 96, 0.8, (0.2, 0.5, 0.8), 3.0, 1.0,
                   (1.65, 0.97, 0.3), head_frac=0.05, head_boost=6.0, index=4,
                   note="high-temperature hit-rate regime"),
    # B=512, K=4, V=151936, bf16; draft N(0, 2^2), target = draft + N(0, 1.5^2);
    # T=1, Bf=32, r=0.5, C=0.5; uniform random fallback on a miss.
    "c5": Workload("c5", 512, 4, 151936, "bf16", (1.0,), 32, 0.5, (0.5,), 2.0, 1.0, (1.5,),
                   fallback_uniform=True, index=5, note="large batch, miss-heavy"),
}


def scaled(w: Workload, B: Optional[int] = None, V: Optional[int] = None, K: Optional[int] = None) -> Workload:
    """The same recipe at a smaller size (for tests the oracle finishes quickly)."""
    from dataclasses import replace
    return replace(w, B=B or w.B, V=V or w.V, K=K or w.K)


def make_logits(w: Workload, buffer: int = 0, target_sigma: Optional[float] = None,
                device="cpu", ld: Optional[int] = None, B: Optional[int] = None):
    """Draft and target logits ``(zq, zp)`` as torch tensors ``[B, K+1, V]`` of the
    workload's dtype on ``device``.  ``buffer`` selects an independent draw (for
    rotating distinct buffers); ``ld`` > V pads each row (the pad holds NaN so that a
    read past V would show).  Deterministic for a given (workload, buffer, device
    type)."""
    B = B or w.B
    K1, V = w.K + 1, w.V
    sig_t = w.target_sigmas[0] if target_sigma is None else target_sigma
    g = torch.Generator(device=device)
    g.manual_seed((w.seed << 20) ^ (buffer * 7919 + 17))
    zq = torch.randn((B, K1, V), generator=g, device=device, dtype=torch.float32) * w.draft_sigma
    if w.head_frac > 0.0:
        gh = torch.Generator(device="cpu")
        gh.manual_seed(w.seed)
        n_head = int(w.head_frac * V)
        head = torch.randperm(V, generator=gh)[:n_head].to(device)
        zq[:, :, head] += w.head_boost
    zp = w.target_scale * zq + torch.randn((B, K1, V), generator=g, device=device,
                                           dtype=torch.float32) * sig_t
    zq = zq.to(w.torch_dtype)
    zp = zp.to(w.torch_dtype)
    if ld is not None and ld > V:
        def pad(z):
            out = torch.full((B, K1, ld), float("nan"), dtype=z.dtype, device=device)
            out[:, :, :V] = z
            return out[:, :, :V]
        zq, zp = pad(zq), pad(zp)
    return zq, zp


def to_oracle_array(z: torch.Tensor):
    """The exact bits of a CPU logit tensor as the oracle takes them: float32 for
    fp32, the raw 16-bit patterns (uint16) for bf16.  Row-strided views keep their
    stride."""
    import numpy as np
    z = z.detach()
    if z.device.type != "cpu":
        z = z.cpu()
    if z.dtype == torch.float32:
        return z.numpy()
    if z.dtype == torch.bfloat16:
        return z.view(torch.int16).numpy().view(np.uint16)
    raise TypeError("unsupported logit dtype %s" % z.dtype)


def make_histories(B: int, L: int, V: int, seed: int, min_frac: float = 0.5, p_copy: float = 0.4,
                   span=(4, 32), zipf_a: float = 1.2):
    """Token histories for the n-gram fallback speculator: int32 ``hist [B, L]`` and
    ragged lengths ``[B]`` in ``[min_frac L, L]`` (entries past a length are -1).
    Each history is a run of spans of ``span`` tokens: with probability ``p_copy`` a
    copy of an earlier span of the same history (the repeats that code, math and chat
    text have), otherwise fresh tokens of Zipf-distributed rank mapped through a fixed
    random permutation of the vocabulary.  numpy generator, deterministic per seed."""
    import numpy as np
    rng = np.random.default_rng(seed)
    perm = rng.permutation(V).astype(np.int32)
    hist = np.full((B, L), -1, dtype=np.int32)
    lens = rng.integers(int(min_frac * L), L + 1, B).astype(np.int32)
    for b in range(B):
        n = int(lens[b])
        row = hist[b]
        cur = 0
        while cur < n:
            w = min(int(rng.integers(span[0], span[1] + 1)), n - cur)
            if cur >= span[0] and rng.random() < p_copy:
                w = min(w, cur)
                s = int(rng.integers(0, cur - w + 1))
                row[cur:cur + w] = row[s:s + w]
            else:
                row[cur:cur + w] = perm[(rng.zipf(zipf_a, w) - 1) % V]
            cur += w
    return hist, lens


def plant_contexts(hist, lens, draft, accept_len, bonus, n: int, rows):
    """A copy of the histories in which each sequence b of ``rows`` holds, at position
    lens[b] // 2, the last ``n`` tokens of its context (history, the k = accept_len[b]
    accepted draft tokens, the bonus), so that the n-gram fallback finds a match of
    length n there.  Host numpy arrays; the histories must be at least 2n + 2 long."""
    import numpy as np
    out = hist.copy()
    for b in rows:
        k = int(accept_len[b])
        tail = np.concatenate([hist[b, :lens[b]][-n:], draft[b, :k], [bonus[b]]]).astype(np.int32)[-n:]
        p = int(lens[b]) // 2
        out[b, p:p + len(tail)] = tail
    return out
