#!/usr/bin/env python3
"""Benchmark of the batched lossless verify-and-resample step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic logits:
draft sampling with Saguaro sigma_{F,C} (which also writes the speculation-
cache keys: each draft row's top-F_k list under the truncated-geometric
fan-out) and verification (acceptance, accepted prefix, bonus, the cache
lookup of (k*, bonus), misses filled with random tokens).  The headline runs
the steps as SSD does, through ssd_round: step i's verification shares its
launches with step i+1's sampling (every step still samples and verifies its
own batch in full; results are checked equal to the separate calls, which
are timed as well).  Default workload: B=64, K=7, V=151936 (Qwen-3
vocabulary), bf16 logits, T=1, F=4, C=0.5; cache budget 64 with fan-out
ratio 0.6.  Inputs rotate over > 1 GiB of distinct sets so the 256 MB
Infinity Cache cannot serve them.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--config N] [--no-cache] [--no-cpu-baseline] [--no-early]
  python bench.py --copy-gib G   (plain device copy of G GiB, for counter calibration)
  python bench.py --read-gib G   (the library's streaming-read probe over G GiB: the read ceiling)
  python bench.py --phases       (phase timings of the epilogues; needs the instrumented libssd_phases.so)

Timing: the headline steps run once eagerly (checked equal to the separate
calls; ms_per_step_eager) and are then captured in a HIP graph and replayed
three times, every replay checked again (ms_per_step_graph); ms_per_step is
the faster of the two: the eager run where the host keeps ahead of the GPU,
the replay (free of the Python binding's host path) where it does not.
After that each entry point runs over the same steps back to back
(sampling, verification, verification with early exit unless --no-early),
with the library's kernel timer on, which stamps the streaming launches with
HIP events recorded by the launch itself on the call's stream; each of those
loops is then timed eagerly and as a HIP graph replay (every replay checked
against the eager results), and ms_sample, ms_verify and ms_verify_early
take the faster of the two; the headline schedule runs once more with the
timer for the shared launch (separate passes, because the event work slows
the step).

Roofline: the dominant kernel of the headline schedule, the longer of its two
HBM-bound launches: the shared launch k_round_mid (sampling's streaming pass
beside the verification of each sequence) or the verification's streaming
pass.  Algorithmic bytes: B (K+1) V element bytes read + one 16-byte partial
per 2048-token block written (+ for the shared launch the verification's
reads of the target partials; + for the verification stream the drafted
tokens and captured logits); the few blocks of row k* that the lazy block
race reads again are not counted.  `traffic` comes from the rocprofv3
FETCH_SIZE / WRITE_SIZE summary committed under profiles/ for that kernel,
and is null when the kernel sources changed since it was taken.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD specification
# ssd_round's schedule: while B (K+1) <= this, two launches (both streaming
# passes, then the verification beside the sampling epilogue), else three
ARITH_DTYPE = "f32"  # every input type is decoded to fp32 for the streaming arithmetic
ROUND_TWO_LAUNCH_ROWS = 256
EARLY_J = 2            # positions streamed for every sequence by ssd_verify_early


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--cache-budget", type=int, default=64)
    ap.add_argument("--cache-ratio", type=float, default=0.6)
    ap.add_argument("--no-cache", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--min-input-gib", type=float, default=1.1)
    ap.add_argument("--copy-gib", type=float, default=0.0)
    ap.add_argument("--read-gib", type=float, default=0.0)
    ap.add_argument("--read-variants", default="all")
    ap.add_argument("--read-chunk-mb", type=float, default=0.0)
    ap.add_argument("--phases", action="store_true")
    # skip the early-exit verification (its first pass is the same kernel as
    # the full verification stream: a clean counter profile of the latter)
    ap.add_argument("--no-early", action="store_true")
    return ap.parse_args()


def source_hash():
    """sha256 (16 hex digits) of the kernel sources."""
    h = hashlib.sha256()
    for f in ("device.hpp", "kernels.hpp", "ssd.hip"):
        with open(os.path.join(ROOT, "lossless_verify_sample_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from its committed
    counter summary (profiles/*.md line 'traffic: kernel=... workload=...
    source=... fetch_bytes=... write_bytes=...'), if it was taken on the
    current sources."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    for f in sorted(os.listdir(pdir)):
        if not f.endswith(".md"):
            continue
        for line in open(os.path.join(pdir, f)):
            if not line.startswith("traffic:"):
                continue
            kv = dict(x.split("=", 1) for x in line.split()[1:])
            if kv.get("kernel") == kernel and kv.get("workload") == workload and kv.get("source") == source_hash():
                return float(kv["fetch_bytes"]) + float(kv["write_bytes"])
    return None


def copy_calibration(gib):
    """A plain device-to-device copy of `gib` GiB, timed: the reference for
    scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = int(gib * 2 ** 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dst.copy_(src)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "seconds": el,
                      "gbs": round(2 * n * 4 / el / 1e9, 1)}), flush=True)


def read_ceiling(gib, variants, chunk_mb):
    """The library's streaming-read probe (ssd_read_probe) over a buffer of
    `gib` GiB, larger than the 256 MB Infinity Cache: each launch layout read
    3 times untimed, then 10 times timed with HIP events on the probe's
    stream.  With chunk_mb > 0 every launch reads one chunk of that many MB
    (10^6 bytes), the chunks taken in turn, so launches of a streaming pass's
    size are timed with their ramp-up and drain.  Prints one JSON line per
    layout and one with the best."""
    import torch

    import lossless_verify_sample_amd as ssd
    n = int(gib * 2 ** 30) // 16 * 16
    buf = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
    cw = int(chunk_mb * 1e6) // 16 * 4 if chunk_mb > 0 else n // 4  # int32 words per launch
    chunks = [buf[i:i + cw] for i in range(0, n // 4 - cw + 1, cw)]
    out = None
    best = None
    for v in (range(12) if variants == "all" else [int(x) for x in variants.split(",")]):
        for i in range(3):
            out = ssd.read_probe(chunks[i % len(chunks)], v, out)
        torch.cuda.synchronize()
        reps = max(10, 2 * len(chunks))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            ssd.read_probe(chunks[i % len(chunks)], v, out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nb = cw * 4
        gbs = nb / (ms * 1e-3) / 1e9
        line = {"read_probe_variant": v, "bytes_per_launch": nb, "launches": reps, "buffer_bytes": n,
                "ms": round(ms, 5), "gbs": round(gbs, 1), "frac_of_8000": round(gbs / HBM_PEAK_GBS, 4)}
        print(json.dumps(line), flush=True)
        if best is None or gbs > best["gbs"]:
            best = line
    print(json.dumps({"read_ceiling": best}), flush=True)


def phases(a):
    """Phase timings of the latency-bound kernels from the instrumented
    library (libssd_phases.so, built by `python -m
    lossless_verify_sample_amd.build --phases`): the workload's sampling and
    verification as separate calls, with the cache step, a few times; then
    per phase the median, 90th percentile and maximum over the items of the
    last call (rows for the sampling epilogue, sequences with a residual for
    the verification kernel), in microseconds, the spread from the first
    item's start to the last item's end, and the number of blocks the lazy
    block race evaluated.  Prints one JSON line.""" 
    import numpy as np
    import torch

    import lossless_verify_sample_amd as ssd
    from lossless_verify_sample_amd import workloads as W
    ssd.use_library(os.path.join(ROOT, "lossless_verify_sample_amd", "libssd_phases.so"))
    dev = torch.device("cuda:0")
    cfg = W.CONFIGS[a.config]
    B, K, V = cfg.B, cfg.K, cfg.V
    T = W.temperatures(cfg, dev)
    Fk = ssd.fanout(a.cache_budget, K, a.cache_ratio, V)
    for it in range(4):
        t, d = W.logits(cfg, it, dev)
        cache = ssd.Cache(Fk, B, K, dev, payload=W.payload(cfg, a.cache_budget, it, dev), miss_fill=True)
        s = ssd.saguaro_sample(d, T, cfg.F, cfg.C, W.seed(cfg, it), F_out=cfg.fout, cache=cache)
        v = ssd.verify(t, d, T, cfg.F, cfg.C, W.seed(cfg, it), s["tokens"], s["q"], s["stats"], s["topf_idx"],
                       cache=cache)
    torch.cuda.synchronize()
    acc = v["accept_len"].cpu().numpy()
    names = {0: ["partials loaded, row maximum", "block weights summed", "top-F list",
                 "sigma normaliser and outputs", "block drawn", "chosen block re-read, token drawn"],
             1: ["K+1 rows' statistics", "acceptance decisions", "lazy block race", "bonus token", "cache lookup"]}
    items = {0: B * (K + 1), 1: B}
    Tb = T.cpu().numpy()
    keep = {0: (np.arange(B * (K + 1)) % (K + 1) < K) & (np.repeat(Tb, K + 1) > 0),  # sampled rows
            1: (acc < K) & (Tb > 0)}                                  # sequences with a residual
    out = {"metric": "phase timings of the latency-bound kernels", "unit": "us", "config": cfg.name,
           "B": B, "K": K, "V": V, "cache_fanout": Fk}
    for kind in (0, 1):
        st = ssd.phase_read(kind, items[kind])[keep[kind]]
        n = len(names[kind])
        ph = {}
        for k in range(n):
            dd = (st[:, k + 1] - st[:, k]) * 0.01
            ph[names[kind][k]] = {"median": round(float(np.median(dd)), 3), "p90": round(float(np.percentile(dd, 90)), 3),
                                  "max": round(float(dd.max()), 3)}
        tot = (st[:, n] - st[:, 0]) * 0.01
        rec = {"items": int(len(st)), "phases": ph,
               "item_total": {"median": round(float(np.median(tot)), 3), "max": round(float(tot.max()), 3)},
               "first_start_to_last_end": round(float((st[:, n].max() - st[:, 0].min()) * 0.01), 3)}
        if kind == 1:
            # slot 7: blocks the lazy race evaluated per sequence
            ev = st[:, 7]
            rec["blocks_evaluated"] = {"mean": round(float(ev.mean()), 3), "p90": float(np.percentile(ev, 90)),
                                       "max": int(ev.max()), "row_blocks": int((V + 2047) // 2048)}
        out[["sampling_epilogue", "verification"][kind]] = rec
    print(json.dumps(out), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the multi-GPU sharding is a design "
                                   "note, not an implementation", "n_gpus": a.gpus}), flush=True)
        sys.exit(2)
    if a.copy_gib > 0:
        copy_calibration(a.copy_gib)
        return
    if a.read_gib > 0:
        read_ceiling(a.read_gib, a.read_variants, a.read_chunk_mb)
        return
    if a.phases:
        phases(a)
        return
    import torch

    import lossless_verify_sample_amd as ssd
    from lossless_verify_sample_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.CONFIGS[a.config]
    B, K, V = cfg.B, cfg.K, cfg.V
    esz = torch.tensor([], dtype=cfg.dtype).element_size()
    set_bytes = 2 * cfg.rows * V * esz
    nsets = max(2, math.ceil(a.min_input_gib * 2 ** 30 / set_bytes))
    sets = [W.logits(cfg, i, dev) for i in range(nsets)]
    T = W.temperatures(cfg, dev)
    use_cache = not a.no_cache
    Fo = cfg.fout
    if use_cache:
        Fk = ssd.fanout(a.cache_budget, K, a.cache_ratio, V)
        # misses take the random fallback tokens (the back-off rule's choice at
        # this batch size and hit rate, reported below)
        caches = [ssd.Cache(Fk, B, K, dev, payload=W.payload(cfg, a.cache_budget, i, dev), miss_fill=True)
                  for i in range(nsets)]
    else:
        Fk, caches = None, None
    total = a.warmup + a.steps
    acc_buf = torch.zeros((total, B), dtype=torch.int32, device=dev)
    hit_buf = torch.zeros((total, B), dtype=torch.int32, device=dev)
    # every step's bonus, p_j(x_j) and gathered cache tokens are kept, so the
    # timed schedules' outputs are checked against the separate calls' in full
    bonus_buf = torch.zeros((total, B), dtype=torch.int32, device=dev)
    p_buf = torch.zeros((total, B, K), dtype=torch.float32, device=dev)
    tok_buf = torch.zeros((total, B, K), dtype=torch.int32, device=dev)
    def smp_buffers():
        return dict(tokens=torch.empty((B, K), dtype=torch.int32, device=dev),
                    q=torch.empty((B, K), dtype=torch.float32, device=dev),
                    stats=torch.empty((cfg.rows, 2), dtype=torch.float64, device=dev),
                    topf_idx=torch.empty((B, K + 1, Fo), dtype=torch.int32, device=dev),
                    topf_val=torch.empty((B, K + 1, Fo), dtype=torch.float32, device=dev))

    smp_bufs = [smp_buffers(), smp_buffers()]  # the sampling of step i + 1 beside step i's verification
    smp_out = smp_bufs[0]
    def step(i):
        t, d = sets[i % nsets]
        seed = W.seed(cfg, i)
        cache = caches[i % nsets] if use_cache else None
        if cache is not None:
            cache.hit = hit_buf[i]
            cache.tokens = tok_buf[i]
        ssd.saguaro_sample(d, T, cfg.F, cfg.C, seed, F_out=Fo, out=smp_out, cache=cache)
        ver_out = dict(accept_len=acc_buf[i], bonus=bonus_buf[i], p=p_buf[i], stats=None)
        ssd.verify(t, d, T, cfg.F, cfg.C, seed, smp_out["tokens"], smp_out["q"], smp_out["stats"],
                   smp_out["topf_idx"], out=ver_out, cache=cache)

    # Headline schedule (ssd_round): step i's verification shares launches
    # with step i + 1's sampling, as the draft speculates the next round
    # while the target verifies in SSD; every step still does one full
    # sampling and one full verification of its own inputs.
    def sample_args(i):
        return dict(draft=sets[i % nsets][1], temperature=T, F=cfg.F, C=cfg.C, seed=W.seed(cfg, i), F_out=Fo,
                    out=smp_bufs[i % 2], cache=caches[i % nsets] if use_cache else None)

    def verify_args(i):
        t, d = sets[i % nsets]
        smp = smp_bufs[i % 2]
        cache = caches[i % nsets] if use_cache else None
        if cache is not None:
            cache.hit = hit_buf[i]
            cache.tokens = tok_buf[i]
        return dict(target=t, draft=d, temperature=T, F=cfg.F, C=cfg.C, seed=W.seed(cfg, i), tokens=smp["tokens"],
                    draft_q=smp["q"], draft_stats=smp["stats"], draft_topf_idx=smp["topf_idx"],
                    out=dict(accept_len=acc_buf[i], bonus=bonus_buf[i], p=p_buf[i], stats=None), cache=cache)

    def run_rounds(lo, hi, early_J=None):
        ssd.round_step(None, sample_args(lo))
        for i in range(lo, hi):
            ssd.round_step(verify_args(i), sample_args(i + 1) if i + 1 < hi else None, early_J=early_J)

    # the same steps with separate calls (sample, then verify)
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for i in range(a.warmup, total):
        step(i)
    s1.record()
    torch.cuda.synchronize()
    acc_sep = acc_buf[a.warmup:].clone()
    hit_sep = hit_buf[a.warmup:].clone()
    outs_sep = [x[a.warmup:].clone() for x in (bonus_buf, p_buf, tok_buf)]

    def same_outputs():
        # accepted lengths, bonus, p_j(x_j), hits and gathered tokens of every
        # timed step equal to the separate calls' (bit for bit)
        ok = (torch.equal(acc_sep, acc_buf[a.warmup:]) and torch.equal(outs_sep[0], bonus_buf[a.warmup:])
              and torch.equal(outs_sep[1], p_buf[a.warmup:]))
        if use_cache:
            ok = ok and torch.equal(hit_sep, hit_buf[a.warmup:]) and torch.equal(outs_sep[2], tok_buf[a.warmup:])
        return ok

    def clear_outputs():
        for x in (acc_buf, bonus_buf) + ((hit_buf, tok_buf) if use_cache else ()):
            x[a.warmup:].fill_(-1)
        p_buf[a.warmup:].fill_(-1.0)
    run_rounds(0, a.warmup)
    torch.cuda.synchronize()
    clear_outputs()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    run_rounds(a.warmup, total)
    stop.record()
    torch.cuda.synchronize()
    if not same_outputs():
        raise SystemExit("ssd_round gave other outputs than the separate calls")
    ms_eager = start.elapsed_time(stop) / a.steps
    # the headline steps captured once in a HIP graph and replayed: the GPU's
    # time per step, free of the binding's host path (slower than the GPU at
    # small batches); every replay is checked against the separate calls
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # the binding's workspaces for this stream, before capture
        run_rounds(a.warmup, total)
    side.synchronize()
    g_round = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_round, stream=side):
        run_rounds(a.warmup, total)
    side.synchronize()
    step_ms = []
    for rep_ in range(3):
        clear_outputs()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):
            e0.record()
            g_round.replay()
            e1.record()
        side.synchronize()
        step_ms.append(e0.elapsed_time(e1) / a.steps)
        if not same_outputs():
            raise SystemExit(f"ssd_round graph replay {rep_} gave other outputs than the separate calls")
    # per-call pass: each entry point over all the timed steps back to back
    # (the host enqueues ahead, so the times are the GPU's), with per-step
    # sampling outputs and cache keys, and the streaming launches stamped by
    # the library's kernel timer (kept out of the headline pass, whose step
    # time the event work would inflate); then the same verifications with
    # early exit, whose accepted lengths must be the same
    timed = range(a.warmup, total)
    smp_all = [smp_buffers() for _ in timed]
    caches_t = ([ssd.Cache(Fk, B, K, dev, payload=caches[i % nsets].payload, miss_fill=True) for i in timed]
                if use_cache else [None] * a.steps)
    acc_early = torch.zeros((a.steps, B), dtype=torch.int32, device=dev)
    bonus_early = torch.zeros((a.steps, B), dtype=torch.int32, device=dev)
    p_early = torch.empty((B, K), dtype=torch.float32, device=dev)  # (NaN past k*: not compared)
    def loop_sample():
        for n, i in enumerate(timed):
            ssd.saguaro_sample(sets[i % nsets][1], T, cfg.F, cfg.C, W.seed(cfg, i), F_out=Fo, out=smp_all[n],
                               cache=caches_t[n])

    def loop_verify():
        for n, i in enumerate(timed):
            t, d = sets[i % nsets]
            sm = smp_all[n]
            if caches_t[n] is not None:
                caches_t[n].hit = hit_buf[i]
                caches_t[n].tokens = tok_buf[i]
            ssd.verify(t, d, T, cfg.F, cfg.C, W.seed(cfg, i), sm["tokens"], sm["q"], sm["stats"], sm["topf_idx"],
                       out=dict(accept_len=acc_buf[i], bonus=bonus_buf[i], p=p_buf[i], stats=None), cache=caches_t[n])

    def loop_early():
        for n, i in enumerate(timed):
            t, d = sets[i % nsets]
            sm = smp_all[n]
            ssd.verify_early(t, d, T, cfg.F, cfg.C, W.seed(cfg, i), sm["tokens"], sm["q"], sm["stats"],
                             sm["topf_idx"], J=EARLY_J,
                             out=dict(accept_len=acc_early[n], bonus=bonus_early[n], p=p_early, stats=None))

    def results_match():
        return same_outputs() and (a.no_early or (torch.equal(acc_early, acc_sep)
                                                  and torch.equal(bonus_early, outs_sep[0])))
    loops = (loop_sample, loop_verify) if a.no_early else (loop_sample, loop_verify, loop_early)

    ssd.timer_enable(a.steps)
    for fn in loops:
        fn()
    torch.cuda.synchronize()
    k_launch = {op: ssd.timer_read(op) for op in (ssd.OP_SAMPLE, ssd.OP_VERIFY)}
    ssd.timer_enable(0)
    if not results_match():
        raise SystemExit("the per-call pass or ssd_verify_early gave other outputs than the separate calls")
    # per-call times on the GPU: each loop captured once in a HIP graph (at
    # small batches the binding's host path is slower than the GPU) and
    # replayed several times, every replay checked against the eager results
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # the binding's workspaces for this stream, before capture
        for fn in loops:
            fn()
    side.synchronize()
    graphs = []
    for fn in loops:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            fn()
        graphs.append(g)
    side.synchronize()
    # each loop timed eagerly as well (no timer): where the host keeps ahead
    # of the GPU this avoids the graph's own per-node cost
    eager_ms = [[] for _ in loops]
    for rep_ in range(3):
        for k, fn in enumerate(loops):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            eager_ms[k].append(e0.elapsed_time(e1) / a.steps)
    call_ms = [[] for _ in loops]
    for rep_ in range(3):
        clear_outputs()
        acc_early.fill_(-1)
        bonus_early.fill_(-1)
        torch.cuda.synchronize()
        for k, g in enumerate(graphs):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(side):
                e0.record()
                g.replay()
                e1.record()
            side.synchronize()
            call_ms[k].append(e0.elapsed_time(e1) / a.steps)
        if not results_match():
            raise SystemExit(f"graph replay {rep_} gave other outputs than the separate calls")
    # the same steps with early-exit verification (ssd_round_early): timed
    # eagerly (median of three), accepted lengths, bonus, hits and gathered
    # tokens checked against the separate calls (p is NaN past k* there)
    ms_early = None
    if not a.no_early:
        ems = []
        for rep_ in range(3):
            clear_outputs()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run_rounds(a.warmup, total, early_J=EARLY_J)
            e1.record()
            torch.cuda.synchronize()
            ems.append(e0.elapsed_time(e1) / a.steps)
            ok = torch.equal(acc_sep, acc_buf[a.warmup:]) and torch.equal(outs_sep[0], bonus_buf[a.warmup:])
            if use_cache:
                ok = ok and torch.equal(hit_sep, hit_buf[a.warmup:]) and torch.equal(outs_sep[2], tok_buf[a.warmup:])
            if not ok:
                raise SystemExit("ssd_round_early gave other outputs than the separate calls")
        ms_early = sorted(ems)[1]
    # and the headline schedule once more with the timer: there the sampling
    # op is the shared launch (sampling stream + verification of each sequence)
    ssd.timer_enable(a.steps + 1)
    run_rounds(a.warmup, total)
    torch.cuda.synchronize()
    r_launch = {op: ssd.timer_read(op) for op in (ssd.OP_SAMPLE, ssd.OP_VERIFY)}
    ssd.timer_enable(0)
    # per step and per call: the faster of the graph replays and the eager
    # runs (eager where the host keeps ahead of the GPU, the graph where not)
    fin = lambda x: round(x, 5) if math.isfinite(x) else None  # (a launch the schedule does not time)
    med = lambda x: sorted(x)[len(x) // 2]  # (the median of three repeats drops a stray one)
    ms_graph = med(step_ms)
    ms = min(ms_graph, ms_eager)
    ms_sep = s0.elapsed_time(s1) / a.steps
    per_call = [min(med(g), med(e)) for g, e in zip(call_ms, eager_ms)]
    t_s, t_v = per_call[:2]
    t_ve = per_call[2] if len(per_call) > 2 else None
    acc = acc_buf[a.warmup:].to(torch.int64)
    tokens = int((acc + 1).sum().item())
    # sequences drawing their bonus from a residual per step: T > 0, k* < K
    rej = int(((acc < K) & (T > 0).unsqueeze(0)).sum().item()) / a.steps
    row_bytes = V * esz
    # bytes each call must read: every draft row, every target row; the
    # residual's blocks that the lazy block race re-reads (a few per sequence,
    # under 2% of the call) are not counted
    b_sample = cfg.rows * row_bytes
    b_verify = cfg.rows * row_bytes
    rows_per_s = cfg.rows / (ms * 1e-3)
    gbs_sample = b_sample / (t_s * 1e-3) / 1e9
    gbs_verify = b_verify / (t_v * 1e-3) / 1e9
    # per-launch times: streaming passes of the separate calls, and in the
    # headline schedule the shared launch and the verification's stream
    k_ms = {op: (t / n if n else float("nan")) for op, (n, t) in k_launch.items()}
    r_ms = {op: (t / n if n else float("nan")) for op, (n, t) in r_launch.items()}
    NB = -(-V // 2048)
    s_bytes = cfg.rows * row_bytes + cfg.rows * NB * 16
    v_bytes = cfg.rows * row_bytes + cfg.rows * NB * 16 + 2 * B * K * 4 + B * K * 4
    # shared launch: sampling's stream + the verification role's reads of the
    # target partials (its lazy race's block re-reads not counted)
    m_bytes = s_bytes + cfg.rows * NB * 16
    dtn = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[cfg.dtype]
    al = "aligned" if (V * esz) % 16 == 0 else "unaligned"
    # the dominant kernel of the headline schedule: the longer of its two
    # HBM-bound launches
    two = cfg.rows <= ROUND_TWO_LAUNCH_ROWS
    if two:
        # both streaming passes share one launch (timed as the sampling op)
        kname, k_alg, k_t, k_n = (f"k_round_streams<{dtn},{al}>", s_bytes + v_bytes, r_ms[ssd.OP_SAMPLE],
                                  r_launch[ssd.OP_SAMPLE][0])
    elif r_ms[ssd.OP_SAMPLE] >= r_ms[ssd.OP_VERIFY]:
        kname, k_alg, k_t, k_n = f"k_round_mid<{dtn},{al}>", m_bytes, r_ms[ssd.OP_SAMPLE], r_launch[ssd.OP_SAMPLE][0]
    else:
        kname, k_alg, k_t, k_n = f"k_stream<{dtn},{al},verify>", v_bytes, r_ms[ssd.OP_VERIFY], r_launch[ssd.OP_VERIFY][0]
    achieved = k_alg / (k_t * 1e-3) / 1e9
    traffic = recorded_traffic(kname, cfg.name)
    backoff = None
    if use_cache:
        # back-off rule on the measured per-sequence hit rates: a round costs
        # the measured step; the accurate backup is taken to cost about one
        # more round (a synchronous speculation), random tokens nothing; an
        # accurate speculation yields the measured tokens per sequence, random
        # tokens about one (the bonus)
        p_hit = (hit_buf[a.warmup:].float().mean(dim=0)).cpu().tolist()
        e_acc = tokens / (a.steps * B)
        use_fast, gain = ssd.backoff(p_hit, ms, ms, 0.0, e_acc, 1.0)
        p_mean = sum(p_hit) / B
        crit = None
        if 0.0 < p_mean < 1.0:
            e_mix = p_mean * e_acc + (1 - p_mean) * 1.0
            q = (e_acc - e_mix) / (e_mix - 0.0)  # t_round = t_slow, t_fast = 0
            crit = round(math.log1p(-q) / math.log(p_mean), 2) if 0.0 < q < 1.0 else None
        backoff = {"use_fast": use_fast, "gain": round(gain, 4), "p_hit_mean": round(p_mean, 4),
                   "critical_batch": crit, "assumed": "t_slow = one step, t_fast = 0, e_fast = 1"}
    out = {
        "metric": "verified logit rows/s",
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic of the path: fp32 streaming sums and races over the
        # decoded logits (fp64 row normalisers and acceptance tests)
        "dtype": ARITH_DTYPE,
        "input_dtype": dtn,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: B={B} K={K} V={V} {str(cfg.dtype).split('.')[-1]} logits, "
                               f"T={cfg.T} F={cfg.F} C={cfg.C}"
                               + (f", cache budget {a.cache_budget} ratio {a.cache_ratio} fan-out {Fk}, misses filled with random tokens"
                                  if use_cache else ""),
                   "B": B, "K": K, "V": V, "input_sets": nsets, "input_gib": round(nsets * set_bytes / 2 ** 30, 2)},
        "tokens_per_s": round(tokens / (a.steps * ms * 1e-3), 1),
        "schedule": ("ssd_round: step i's verification shares launches with step i+1's sampling: "
                     + ("both streaming passes, then the verification beside the sampling epilogue" if two else
                        "the verification stream, then the verification beside the sampling stream, then the "
                        "sampling epilogue")),
        "ms_per_step_separate_calls": round(ms_sep, 5),
        "ms_per_step_eager": round(ms_eager, 5),
        "ms_per_step_graph": round(ms_graph, 5),
        "ms_per_step_early_exit": round(ms_early, 5) if ms_early is not None else None,
        "ms_per_call_graph": [round(med(g), 5) for g in call_ms],
        "ms_per_call_eager": [round(med(e), 5) for e in eager_ms],
        "mean_accepted": round(float(acc.float().mean().item()), 4),
        "ms_sample": round(t_s, 5),
        "ms_verify": round(t_v, 5),
        "ms_verify_early": round(t_ve, 5) if t_ve is not None else None,
        "early_exit_J": EARLY_J,
        "gbs_sample": round(gbs_sample, 1),
        "gbs_verify": round(gbs_verify, 1),
        "cache_hit_rate": round(float(hit_buf[a.warmup:].sum().item()) / (a.steps * B), 4) if use_cache else None,
        "backoff": backoff,
        "roofline": {
            "kernel": kname,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes": int(k_alg),
            "launches": k_n,
            "ms_per_launch": round(k_t, 5),
            "source": source_hash(),
        },
        "ms_round_mid": fin(r_ms[ssd.OP_SAMPLE]),
        "ms_round_verify_stream": fin(r_ms[ssd.OP_VERIFY]),
        "residual_sequences_per_step": round(rej, 2),
        "ms_stream_sample": round(k_ms[ssd.OP_SAMPLE], 5),
        "ms_stream_verify": round(k_ms[ssd.OP_VERIFY], 5),
        "gbs_stream_sample": round(s_bytes / (k_ms[ssd.OP_SAMPLE] * 1e-3) / 1e9, 1),
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, sets, T, Fo)
    print(json.dumps(out), flush=True)


def cpu_baseline(cfg, sets, T, Fo, min_seconds=10.0, max_steps=64):
    """The oracle (unchanged) on whole steps of the workload on the host
    cores: sample + verify of every row, repeated over the input sets until
    about min_seconds have passed."""
    import numpy as np
    import torch

    from oracle import pool as OP

    def raw(x):
        return x.view(torch.int16).cpu().numpy().view(np.uint16) if x.dtype != torch.float32 else x.cpu().numpy()

    dt = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[cfg.dtype]
    Th = T.cpu().numpy().astype(np.float64)
    host = [(raw(t), raw(d)) for t, d in sets]
    workers = OP.default_workers()
    t0 = time.perf_counter()
    n = 0
    while n < max_steps and (n == 0 or time.perf_counter() - t0 < min_seconds):
        rt, rd = host[n % len(host)]
        OP.run(rd, dt, Th, cfg.F, cfg.C, n, F_out=Fo, target_raw=rt, workers=workers)
        n += 1
    el = time.perf_counter() - t0
    return {"value": round(n * cfg.rows / el, 2), "unit": "rows/s", "cores": workers, "kind": "oracle",
            "sample": f"{n} full steps ({cfg.B} sequences, {cfg.rows} rows each: sample + verify) "
                      f"in {el:.1f} s wall"}


if __name__ == "__main__":
    main()
