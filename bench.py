#!/usr/bin/env python3
"""Throughput of the fused verify-and-pre-speculate round (SSD / Saguaro) on one
MI355X: rounds per second and achieved HBM bandwidth of the vocabulary pass.

One step is one whole round over one batch: softmax statistics of both models,
top-F speculation cache with geometric fan-out, Saguaro reweighting, lossless
verification, residual bonus sampling, cache lookup and the next draft gathered
from a synthetic value store (one ssd_round call: two streaming HIP kernels, each
followed by a small one).  Outside the timed rounds it also measures the coverage
statistics pass (bonus rank within the draft row), reports the fan-out the
optimiser picks from them, and times the n-gram fallback speculator on the misses.  Inputs (seeded synthetic
logits, draft tokens from the library's own Saguaro sampler) are resident in HBM
before timing; the timed loop rotates over distinct logit buffers totalling more
than the 256 MB last-level cache so that rows come from HBM.

The roofline figure is for pass 1 (the vocabulary pass over all 2 B (K+1) rows),
timed live with HIP events recorded on the launch stream.  Its HBM traffic comes
from the rocprofv3 byte counters summarised under profiles/, and is reported only
while the kernel sources are the ones those counters were taken from.

Prints one JSON line on stdout.  With --gpus above 1 it exits: this build measures
one GPU.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pass1_kernel_c3_traffic.md")
KERNEL_SOURCES = ["ssd_kernels.hip", "ssd_device.h", "ssd_kernels.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="c3", help="c1..c5 (default: the headline B=64 K=8 V=128256 bf16)")
    ap.add_argument("--buffers", type=int, default=0, help="distinct logit buffers to rotate (0: >= 1 GB)")
    ap.add_argument("--T", type=float, default=None, help="temperature (default: the workload's last)")
    ap.add_argument("--C", type=float, default=None)
    ap.add_argument("--target-sigma", type=float, default=None)
    ap.add_argument("--r", type=float, default=None, help="fan-out ratio r (default: the workload's)")
    ap.add_argument("--Bf", type=int, default=None, help="cache budget B_f (default: the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-every", type=int, default=0,
                    help="time the vocabulary pass with HIP events on every N-th timed round "
                         "(0: max(1, steps // 16), so that at least 16 launches are timed)")
    ap.add_argument("--stream-passes", type=int, default=32,
                    help="read-only passes over the rotating buffers for the same-run read ceiling")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calib", action="store_true",
                    help="3 copies of 1 GiB instead of 5 (the count the byte-counter calibration expects)")
    return ap.parse_args()


class HipEvents:
    """HIP events created with hipEventDisableSystemFence: recording one writes a
    timestamp without the system-scope cache writeback and invalidation a default
    event performs, so timing a kernel between two of them barely disturbs the
    kernels around it.  Loaded from the HIP runtime torch has already loaded."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self):
        e = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)
        self.made.append(e)
        return e

    def record(self, e, stream):
        rc = self.hip.hipEventRecord(e, stream)
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def ms(self, a, b):
        out = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(out), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(out.value)

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(e)
        self.made = []


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the round of this library runs on a single MI355X "
              "(sequences would shard across GPUs with no exchange; only the one-GPU path is built); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import lossless_rejection_sampling_ssd_amd as ssd
    from lossless_rejection_sampling_ssd_amd.workloads import WORKLOADS, make_histories, make_logits, plant_contexts

    w = WORKLOADS[args.workload]
    if args.r is not None or args.Bf is not None:
        import dataclasses
        w = dataclasses.replace(w, r=w.r if args.r is None else args.r, Bf=w.Bf if args.Bf is None else args.Bf)
    T = w.temps[-1] if args.T is None else args.T
    C = args.C if args.C is not None else w.Cs[len(w.Cs) // 2]
    sig = args.target_sigma
    esize = 2 if w.dtype == "bf16" else 4
    F = ssd.ssd_fanout(w.K, w.Bf, w.r)
    B, K, V = w.B, w.K, w.V
    K1 = K + 1
    pass1_bytes = 2 * B * K1 * V * esize
    nbuf = args.buffers or max(1, -(-(1 << 30) // pass1_bytes))
    torch.cuda.set_device(0)
    dev = "cuda"

    # ---- inputs resident in HBM (untimed): logits and draft tokens sampled from q'
    bufs = []
    ws = ssd.Workspace()
    for i in range(nbuf):
        zq, zp = make_logits(w, buffer=i, target_sigma=sig, device=dev)
        shape = ssd.shape_of(zq, T)
        R = B * K1
        qm = torch.zeros(R, device=dev)
        qs = torch.zeros(R, dtype=torch.float64, device=dev)
        qa = torch.zeros(R, dtype=torch.int32, device=dev)
        ssd.ssd_softmax(shape, zq, qm, qs, qa, ws=ws)
        ids = torch.zeros((B, w.Bf), dtype=torch.int32, device=dev)
        mass = torch.zeros(R, dtype=torch.float64, device=dev)
        ssd.ssd_build_cache(shape, zq, qm, qs, F, ids, mass, ws=ws)
        Z = torch.zeros(R, dtype=torch.float64, device=dev)
        d = torch.zeros((B, K), dtype=torch.int32, device=dev)
        ssd.ssd_saguaro_reweight(shape, mass, C, Z, zq, qm, qs, qa, F, ids, None, w.seed, 10_000 + i, d, ws=ws)
        bufs.append((zp, zq, d))
    torch.cuda.synchronize()
    shape = ssd.shape_of(bufs[0][0], T)
    fallback = ssd.SSD_FALLBACK_UNIFORM if w.fallback_uniform else ssd.SSD_FALLBACK_NONE
    # value store [B, B_f, K]: synthetic continuations (real ones come from draft forward
    # passes); each round also gathers the next draft from it
    values = torch.randint(0, V, (B, w.Bf, K), dtype=torch.int32, device=dev,
                           generator=torch.Generator(device=dev).manual_seed(w.seed))
    outb = ssd.RoundBuffers(B, K, w.Bf, with_stats=False, cache_values=values)

    def step(i, events=None):
        zp, zq, d = bufs[i % nbuf]
        ssd.ssd_round(shape, zp, zq, d, F, C, w.seed, i, fallback, outb.out, events=events, ws=ws)

    hev = HipEvents()
    cur = torch.cuda.current_stream()
    st = cur.cuda_stream

    # ---- the same-run read ceiling: read-only passes over the same rotating buffers,
    # in pass 1's access shape, each pass the 2 B (K+1) V s bytes of one round
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    ns = max(1, args.stream_passes)
    s0, s1 = hev.create(), hev.create()
    for j in range(2):  # untimed: first touch
        ssd.ssd_stream_read(bufs[j % nbuf][0], sink)
        ssd.ssd_stream_read(bufs[j % nbuf][1], sink)
    hev.record(s0, st)
    for j in range(ns):
        zp_j, zq_j, _ = bufs[j % nbuf]
        ssd.ssd_stream_read(zp_j, sink)
        ssd.ssd_stream_read(zq_j, sink)
    hev.record(s1, st)
    torch.cuda.synchronize()
    stream_us = hev.ms(s0, s1) * 1e3 / ns
    stream_gbps = pass1_bytes / (stream_us * 1e-6) / 1e9
    log("read ceiling: %d passes of %d bytes, %.2f us each, %.1f GB/s" % (ns, pass1_bytes, stream_us, stream_gbps))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: K rounds back to back; HIP events (no system fence) around the
    # vocabulary pass of every --event-every-th round, at least 16 launches in all
    n = args.steps
    every = args.event_every if args.event_every > 0 else max(1, n // 16)
    sampled = list(range(0, n, every))
    ev = [(hev.create(), hev.create()) for _ in sampled]
    evs = [None] * n
    for j, (a, b) in zip(sampled, ev):
        evs[j] = ssd.ssd_round_events(a.value, b.value, None, None)
    # events at 5 chunk boundaries give the spread between repeats
    nrep = 5 if n >= 5 else 1
    bounds = [n * j // nrep for j in range(nrep + 1)]
    marks = [hev.create() for _ in range(nrep + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    hev.record(marks[0], st)
    for j in range(nrep):
        for i in range(bounds[j], bounds[j + 1]):
            step(args.warmup + i, evs[i])
        hev.record(marks[j + 1], st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = hev.ms(marks[0], marks[-1])
    rep_us = [hev.ms(marks[j], marks[j + 1]) * 1e3 / (bounds[j + 1] - bounds[j]) for j in range(nrep)]
    pass1_ms = [hev.ms(a, b) for a, b in ev]
    pass1_avg_ms = float(np.mean(pass1_ms))
    ms_per_step = total_ms / n
    rounds_per_s = 1000.0 / ms_per_step

    # ---- algorithmic bytes of the same rounds (deterministic replay, untimed)
    # with the coverage histogram of the same rounds (bonus rank within draft row k)
    RB = 64
    hist = torch.zeros((K1, RB + 1), dtype=torch.int32, device=dev)
    rank = torch.zeros(B, dtype=torch.int32, device=dev)
    ks, hits, aprob = [], [], []
    for i in range(min(n, 64)):
        step(args.warmup + i)
        zq_i = bufs[(args.warmup + i) % nbuf][1]
        ssd.ssd_bonus_rank(shape, zq_i, outb["accept_len"], outb["bonus"], RB, rank, hist, ws=ws)
        ks.append(outb["accept_len"].cpu().numpy().copy())
        hits.append(outb["hit"].cpu().numpy().copy())
        aprob.append(float(outb["accept_prob"].double().mean().item()))
    ks = np.stack(ks)
    hits = np.stack(hits)
    h_np = hist.cpu().numpy()
    covered = sum(int(h_np[k, :F[k]].sum()) for k in range(K1))
    F_opt, hits_opt, total = ssd.ssd_fanout_optimize(K, w.Bf, RB, h_np)

    # the coverage pass alone: one draft row per sequence (B V s bytes per call)
    nr = 200
    r0 = torch.cuda.Event(enable_timing=True)
    r1 = torch.cuda.Event(enable_timing=True)
    r0.record()
    for i in range(nr):
        ssd.ssd_bonus_rank(shape, bufs[i % nbuf][1], outb["accept_len"], outb["bonus"], RB, rank, hist, ws=ws)
    r1.record()
    torch.cuda.synchronize()
    rank_us = r0.elapsed_time(r1) * 1e3 / nr
    rank_bytes = B * V * esize
    # the n-gram fallback speculator on the misses of the last round, over synthetic
    # 4096-token histories (spans repeated within each history)
    NG_L, NG_MIN, NG_MAX = 4096, 2, 5
    h_np_tok, h_len = make_histories(B, NG_L, V, seed=w.seed)
    ng_hist = torch.as_tensor(h_np_tok, device=dev)
    ng_len = torch.as_tensor(h_len, device=dev)
    ng_tok = torch.zeros((B, K), dtype=torch.int32, device=dev)
    ng_n = torch.zeros(B, dtype=torch.int32, device=dev)
    d_last = bufs[(args.warmup + min(n, 64) - 1) % nbuf][2]

    def ngram():
        ssd.ssd_ngram_fallback(V, ng_hist, ng_len, d_last, outb["accept_len"], outb["bonus"], NG_MIN, NG_MAX,
                               w.seed, 0, ng_tok, hit=outb["hit"], match_n=ng_n)

    ngram()
    torch.cuda.synchronize()
    served = outb["hit"].cpu().numpy() == 0
    ng_match = float((ng_n.cpu().numpy()[served] > 0).mean()) if served.any() else 0.0
    r0.record()
    for i in range(nr):
        ngram()
    r1.record()
    torch.cuda.synchronize()
    ngram_us = r0.elapsed_time(r1) * 1e3 / nr
    # the same calls with every other served sequence's context planted mid-history,
    # so that about half of them find a match (the histories above match none)
    plant = np.nonzero(served)[0][::2]
    h_pl = plant_contexts(h_np_tok, h_len, d_last.cpu().numpy(), outb["accept_len"].cpu().numpy(),
                          outb["bonus"].cpu().numpy(), NG_MAX, plant)
    ng_hist = torch.as_tensor(h_pl, device=dev)
    ngram()
    torch.cuda.synchronize()
    ng_match_pl = float((ng_n.cpu().numpy()[served] > 0).mean()) if served.any() else 0.0
    r0.record()
    for i in range(nr):
        ngram()
    r1.record()
    torch.cuda.synchronize()
    ngram_pl_us = r0.elapsed_time(r1) * 1e3 / nr
    rows2 = np.where(ks < K, 2, 1).sum(axis=1).mean() if T > 0 else 0.0
    pass2_bytes = rows2 * V * esize
    round_bytes = pass1_bytes + pass2_bytes
    round_gbps = round_bytes / (ms_per_step * 1e-3) / 1e9
    pass1_gbps = pass1_bytes / (pass1_avg_ms * 1e-3) / 1e9

    # a plain device copy of 1 GiB in the same run: reference for the HBM byte counters
    # (rocprofv3 --pmc) and for the achievable streaming rate on this machine
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    ncopy = 3 if args.copy_calib else 5
    torch.cuda.synchronize()
    c0.record()
    for _ in range(ncopy):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 4 * ncopy / (c0.elapsed_time(c1) * 1e-3) / 1e9
    log("device copy: %d x %d bytes, %.1f GB/s (read + write)" % (ncopy, src.numel() * 4, copy_gbps))
    del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, bufs[0], T, C, F, args.cpu_seconds)

    traffic = measured_traffic()
    label = "%s: B=%d K=%d V=%d %s logits, T=%g, B_f=%d, r=%g, C=%g" % (
        args.workload, B, K, V, w.dtype, T, w.Bf, w.r, C)
    if sig is not None:
        label += ", target sigma=%g" % sig
    rec = {
        "metric": "verify+cache rounds/sec and achieved HBM GB/s (% of peak), B=64 V=128256 K=8",
        "value": round(rounds_per_s, 2),
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",  # arithmetic: fp32 terms, fp64 sums; the logits themselves are config.logits
        "data": "synthetic",
        "config": {
            "workload": label,
            "logits": w.dtype,
            "arithmetic": "fp32 per-element terms, fp64 normalisers and running sums",
            "fan_out": F,
            "next_draft_gather": True,
            "buffers": nbuf,
            "round_bytes": int(round_bytes),
            "round_GBps": round(round_gbps, 1),
            "round_frac_of_peak": round(round_gbps / PEAK_HBM_GBPS, 4),
            "pass1_us": round(pass1_avg_ms * 1e3, 2),
            "pass1_timed_launches": "%d of the %d timed rounds (one in %d)" % (len(sampled), n, every),
            "us_per_round_median_of_%d_repeats" % nrep: round(float(np.median(rep_us)), 2),
            "us_per_round_repeats": [round(x, 2) for x in rep_us],
            "copy_GBps_read_plus_write": round(copy_gbps, 1),
            "pass1_frac_of_copy": round(pass1_gbps / copy_gbps, 4),
            "stream_read_us": round(stream_us, 2),
            "stream_read_GBps": round(stream_gbps, 1),
            "stream_read_frac_of_peak": round(stream_gbps / PEAK_HBM_GBPS, 4),
            "pass1_frac_of_stream": round(pass1_gbps / stream_gbps, 4),
            "pass1_us_min": round(min(pass1_ms) * 1e3, 2),
            "pass1_us_median": round(float(np.median(pass1_ms)) * 1e3, 2),
            "pass2_and_gaps_us": round((ms_per_step - pass1_avg_ms) * 1e3, 2),
            "mean_accept_len": round(float(ks.mean()), 3),
            "mean_sum_min_p_qprime": round(float(np.mean(aprob)), 4),
            "hit_rate": round(float(hits.mean()), 4),
            # P(some sequence of the batch misses in a round): measured over the replayed
            # rounds, and 1 - prod_b h_b from each sequence's own hit rate over them
            "p_any_miss_measured": round(float((hits == 0).any(axis=1).mean()), 4),
            "p_any_miss_from_h": round(float(1.0 - np.prod(hits.mean(axis=0))), 6),
            "hit_rate_from_rank_hist": round(covered / max(total, 1), 4),
            "fanout_optimized": F_opt,
            "predicted_hit_rate_optimized": round(hits_opt / max(total, 1), 4),
            "pass1_counter_GBps": (round(traffic / (pass1_avg_ms * 1e-3) / 1e9, 1) if traffic else None),
            "bonus_rank_us": round(rank_us, 2),
            "bonus_rank_GBps": round(rank_bytes / (rank_us * 1e-6) / 1e9, 1),
            "ngram_fallback_us": round(ngram_us, 2),
            "ngram_history": "%d-token synthetic histories, n = %d..%d, misses of the last round (%d of %d)" % (
                NG_L, NG_MIN, NG_MAX, int(served.sum()), B),
            "ngram_match_rate": round(ng_match, 4),
            "ngram_fallback_planted_us": round(ngram_pl_us, 2),
            "ngram_planted_match_rate": round(ng_match_pl, 4),
            "wall_s": round(wall, 3),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(pass1_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(pass1_gbps / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
            "kernel": "pass1_kernel (vocabulary pass over all 2*B*(K+1) rows); the whole round's fraction is "
                      "config.round_frac_of_peak",
            "bytes_per_launch": int(pass1_bytes),
        },
        "cpu_baseline": cpu,
    }
    hev.close()
    print(json.dumps(rec), flush=True)


def kernel_digest():
    """sha256 over the device sources of the kernels."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "lossless_rejection_sampling_ssd_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per pass-1 launch from the committed counter summary, or None when
    it is missing or was taken from other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        line = line.strip().strip("`-* ")
        if ":" in line:
            k, _, v = line.partition(":")
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, buf, T, C, F, seconds):
    """The fp64 oracle, as it stands, on whole rounds of the same workload (first
    logit buffer), on this host's cores, for about `seconds` of CPU work."""
    import numpy as np
    import oracle
    from lossless_rejection_sampling_ssd_amd.workloads import to_oracle_array

    zp, zq, _ = buf
    zp_np, zq_np = to_oracle_array(zp.cpu()), to_oracle_array(zq.cpu())
    Fa = np.asarray(F, np.int32)
    ids, mass = oracle.build_cache(zq_np, T, Fa)
    Z, _ = oracle.saguaro(zq_np, T, Fa, ids, mass, C)
    draft, _ = oracle.draft_sample(zq_np, T, Fa, ids, Z, C, w.seed, 0)
    _, gap = oracle.fanout(w.K, w.Bf, w.r)
    threads = oracle.num_threads()
    rounds = 0
    exc = {name: 0 for name in ("E1", "E2", "E3", "E4", "E5")}
    bits = {"E1": oracle.E1_ACCEPT_TIE, "E2": oracle.E2_CDF_TIE, "E3": oracle.E3_DEGENERATE_RESIDUAL,
            "E4": oracle.E4_FANOUT_TIE, "E5": oracle.E5_TINY_PROB}
    t0 = time.perf_counter()
    while True:
        o = oracle.round_(zp_np, zq_np, T, Fa, C, draft, w.seed, rounds, w.fallback_uniform, gap)
        for name, bit in bits.items():
            exc[name] += int(((o.exc & bit) != 0).sum())
        rounds += 1
        el = time.perf_counter() - t0
        if el >= seconds or rounds >= 50:
            break
    log("cpu baseline: %d oracle rounds in %.2f s on %d threads" % (rounds, el, threads))
    # one thread, on the first 4 sequences of the batch, scaled to whole rounds
    nb = min(4, w.B)
    oracle.set_num_threads(1)
    try:
        t1 = time.perf_counter()
        oracle.round_(zp_np[:nb], zq_np[:nb], T, Fa, C, draft[:nb], w.seed, 0, w.fallback_uniform)
        el1 = time.perf_counter() - t1
    finally:
        oracle.set_num_threads(threads)
    one = nb / w.B / el1
    log("cpu baseline, 1 thread: %d sequences in %.2f s" % (nb, el1))
    return {"value": round(rounds / el, 4), "unit": "rounds/s", "cores": threads, "kind": "oracle",
            "sample": "%d whole rounds (B=%d sequences each) of the timed workload's first logit buffer" % (
                rounds, w.B),
            "cpu_model": cpu_model(),
            "value_1_thread": round(one, 5),
            "sample_1_thread": "one round of the first %d sequences, scaled to B=%d" % (nb, w.B),
            "oracle_exception_rows": dict(exc, rows=rounds * w.B)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.partition(":")[2].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
