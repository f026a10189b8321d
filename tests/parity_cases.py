"""Inputs of the GPU parity runs whose oracle exception counts are stored
(tests/golden/flag_counts.json, written by tests/golden/make_flag_counts.py): every
workload at its full size (c4 at three of its (target spread, C) points, c3 also with
an odd vocabulary), c2 on its own recipe at each of its temperatures, the c1 rounds,
the edge cases, the masked vocabularies and the seeded random configurations.
Logits are generated on the CPU (seeded torch generators), drafts are sampled by the
oracle from its own q' (a step of the harness, not of the round), value-store
contents are seeded integers.  No GPU code here."""
import numpy as np
import torch

import oracle
from lossless_rejection_sampling_ssd_amd.workloads import WORKLOADS, make_logits, scaled, to_oracle_array


def rand_logits(B, K, V, dtype, seed, scale=2.0, noise=0.8, ld=None):
    """Draft logits N(0, scale^2), target = draft + N(0, noise^2); with ld > V the
    rows are views into NaN-padded rows of stride ld."""
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


def oracle_draft(zp_np, zq_np, T, F, C, seed, rnd, b_base=0):
    """Draft tokens sampled by the oracle from its own q' (harness step)."""
    F = np.asarray(F, np.int32)
    ids, mass = oracle.build_cache(zq_np, T, F)
    Z, _ = oracle.saguaro(zq_np, T, F, ids, mass, C)
    d, flags = oracle.draft_sample(zq_np, T, F, ids, Z, C, seed, rnd, b_base)
    return d, flags


def exception_counts(o):
    """Flagged sequences and per-bit counts E1..E5 of an oracle round."""
    bits = {"E1": oracle.E1_ACCEPT_TIE, "E2": oracle.E2_CDF_TIE, "E3": oracle.E3_DEGENERATE_RESIDUAL,
            "E4": oracle.E4_FANOUT_TIE, "E5": oracle.E5_TINY_PROB}
    out = {k: int(((o.exc & v) != 0).sum()) for k, v in bits.items()}
    out["flagged"] = int((o.exc != 0).sum())
    return out


class RoundCase:
    """One round's inputs: torch CPU logits (zq, zp), their oracle arrays, the fan-out
    F (list), T, C, drafts, (seed, round), the fallback mode and the value store
    ([B, Bf, K] int32, or None)."""

    def __init__(self, label, zq, zp, T, F, C, seed, rnd, fallback, draft=None, values=None, gap=None):
        self.label, self.zq, self.zp, self.T, self.C = label, zq, zp, T, C
        self.F = [int(x) for x in F]
        self.seed, self.rnd, self.fallback, self.gap = seed, rnd, int(fallback), gap
        self.B, self.K, self.V = zq.shape[0], zq.shape[1] - 1, zq.shape[2]
        self.zp_np, self.zq_np = to_oracle_array(zp), to_oracle_array(zq)
        if draft is None:
            draft, _ = oracle_draft(self.zp_np, self.zq_np, T, self.F, C, seed, rnd)
        self.draft = draft
        self.values = values

    def oracle_round(self):
        return oracle.round_(self.zp_np, self.zq_np, self.T, np.array(self.F, np.int32), self.C, self.draft,
                             self.seed, self.rnd, self.fallback, self.gap)


# ----------------------------------------------------------------------------- workloads
# (label, workload, temperature, C, target spread (None: the recipe's), vocabulary override)
FULL_CASES = [
    ("c3", "c3", 1.0, 0.5, None, None),
    ("c3 odd V", "c3", 1.0, 0.5, None, 128257),
    ("c4 s1.65 C0.2", "c4", 1.2, 0.2, 1.65, None),
    ("c4 s0.97 C0.5", "c4", 1.2, 0.5, 0.97, None),
    ("c4 s0.3 C0.8", "c4", 1.2, 0.8, 0.3, None),
    ("c5", "c5", 1.0, 0.5, None, None),
    ("c2 T0", "c2", 0.0, 0.3, None, None),
    ("c2 T0.7", "c2", 0.7, 0.3, None, None),
    ("c2 T1", "c2", 1.0, 0.3, None, None),
]
C1_ROUNDS = 1000


def full_case(label):
    """A workload's whole batch at its full size, at round counter 1."""
    _, name, T, C, sig, V = next(c for c in FULL_CASES if c[0] == label)
    w = WORKLOADS[name] if V is None else scaled(WORKLOADS[name], V=V)
    zq, zp = make_logits(w, target_sigma=sig, device="cpu")
    F, gap = oracle.fanout(w.K, w.Bf, w.r)
    rng = np.random.default_rng(sum(map(ord, label)))
    values = rng.integers(0, w.V, size=(w.B, w.Bf, w.K)).astype(np.int32)
    c = RoundCase(label, zq, zp, T, F, C, w.seed, 1, w.fallback_uniform, values=values, gap=gap)
    c.w = w
    return c


def c1_case(rnd):
    """Round rnd of the single-sequence workload, with its own logits."""
    w = WORKLOADS["c1"]
    zq, zp = make_logits(w, buffer=rnd, device="cpu")
    F, gap = oracle.fanout(w.K, w.Bf, w.r)
    c = RoundCase("c1 round %d" % rnd, zq, zp, w.temps[0], F, w.Cs[0], w.seed, rnd, 0, gap=gap)
    c.w = w
    return c


# ----------------------------------------------------------------------------- edges
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
    # more than 1024 (sequence, position) pairs with more than 64 tiles per row: the
    # one-wave finalisation (large rounds) on its general path
    ("1025 pairs V=140k f32", "f32", 205, 4, 140001, 1.0, [8, 4, 2, 1, 1], 0.5, 2.0, 0.5, 0.0),
    # bonus passes of more than 8192 tiles on 16-byte aligned rows (two tiles per wave):
    # the row's last wave with a whole and a ragged tile (bf16, 64 tiles of 2048), or
    # with a ragged tile alone (fp32, 117 tiles of 1024)
    ("paired tiles bf16", "bf16", 130, 1, 130072, 1.0, [8, 4], 0.5, 2.0, 0.5, 0.0),
    ("paired tiles f32", "f32", 72, 3, 119000, 1.0, [8, 4, 2, 1], 0.5, 2.0, 0.5, 0.0),
]


def edge_case(label):
    """Drafts sampled from q', then the first token forced to id 0 and the last to
    V - 1."""
    _, dtype, B, K, V, T, F, C, scale, noise, quantum = next(c for c in EDGE_CASES if c[0] == label)
    g = torch.Generator().manual_seed(sum(map(ord, label)))
    zq = torch.randn((B, K + 1, V), generator=g) * scale
    if quantum > 0:
        zq = torch.round(zq / quantum) * quantum
    zp = zq + torch.randn((B, K + 1, V), generator=g) * noise
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    zq, zp = zq.to(dt), zp.to(dt)
    seed, rnd = 0xED6E + B, 5
    d, _ = oracle_draft(to_oracle_array(zp), to_oracle_array(zq), T, F, C, seed, rnd)
    d[0, 0] = 0
    d[-1, -1] = V - 1
    return RoundCase(label, zq, zp, T, F, C, seed, rnd, 1, draft=d)


# ----------------------------------------------------------------------------- masks
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


def mask_case(label):
    """-inf logits: shared masks, target-only masks, a draft row with fewer finite ids
    than its cache share; every row keeps one finite id in both models."""
    _, dtype, B, K, V, T, F, C, f_shared, f_target, n_fin = next(c for c in MASK_CASES if c[0] == label)
    g = torch.Generator().manual_seed(sum(map(ord, label)))
    zq = torch.randn((B, K + 1, V), generator=g) * 2.0
    zp = zq + torch.randn((B, K + 1, V), generator=g) * 0.7
    shared = torch.rand((B, K + 1, V), generator=g) < f_shared
    target = torch.rand((B, K + 1, V), generator=g) < f_target
    zq[shared] = float("-inf")
    zp[shared | target] = float("-inf")
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
    values = np.random.default_rng(B).integers(0, V, (B, sum(F), K)).astype(np.int32)
    return RoundCase(label, zq, zp, T, F, C, 0x3A5C + B, 2, 1, values=values)


# ----------------------------------------------------------------------------- random configurations
N_RANDOM = 96


def random_round_config(i):
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


def random_case(i):
    dtype, B, K, V, pad, T, F, C, fb, scale, noise, mask = random_round_config(i)
    label = "random %d: %s B=%d K=%d V=%d pad=%d T=%g F=%s C=%.3f fb=%d mask=%.2f" % (
        i, dtype, B, K, V, pad, T, F, C, fb, mask)
    zq, zp = rand_logits(B, K, V, dtype, 0xAB00 + i, scale, noise, ld=V + pad if pad else None)
    if mask > 0:
        g = torch.Generator().manual_seed(0xAB00 + i)
        m = torch.rand((B, K + 1, V), generator=g) < mask
        m[:, :, 0] = False  # every row keeps a finite id
        zq[m] = float("-inf")
        zp[m] = float("-inf")
    Bf = sum(F)
    values = np.random.default_rng(i).integers(0, V, (B, max(Bf, 1), K)).astype(np.int32)[:, :Bf]
    return RoundCase(label, zq, zp, T, F, C, 0x5EED + i, 100 + i, fb, values=values if Bf > 0 else None)
