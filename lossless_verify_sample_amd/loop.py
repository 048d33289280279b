"""Synthetic multi-round SSD loop on one GPU, served from the speculation
cache.

Round r of a batch: the target verifies the drafted tokens x_r (ssd_verify);
meanwhile the draft has pre-speculated round r+1 for every outcome it keeps
in the cache ([SSD-B] core-mechanism section: the draft fills a speculation
cache while verification runs and one lookup follows; [SSD-A]: on a hit the
prepared tokens go to the verifier at once).  The cache of round r is keyed
by (k, y) = (accepted length, bonus token) with the top-F_k tokens of draft
row k as the guesses y ([SSD-B] part 1), and slot s holds a real
pre-speculation: K tokens drawn with Saguaro sigma_{F,C} from round r+1's
draft rows under a seed of the slot's own (ssd_saguaro_sample), with their
sigma_j(x_j).  The lookup of (k*_r, bonus_r) then decides round r+1's drafted
tokens:
  hit  -> the slot's tokens and their q;
  miss -> policy "fresh": a fresh sigma draw from the same draft rows (the
          accurate backup speculator, one more draft pass);
          policy "random": K uniform random tokens (the near-zero-latency
          backup of [SSD-B] part 3), verified against the uniform draft
          distribution (q = 1/V, residual max(0, p - 1/V)) in a verification
          call of their own, so every round stays lossless.
Every choice above depends only on round r's outcome, never on the slot's own
randomness, so the selected tokens are exact sigma (or uniform) samples.

Synthetic stand-in: round r+1's draft rows are one set of K+1 rows per
sequence, the same for every slot (a draft model would condition each
branch on its (k, y)); logits come from workloads.logits with fresh steps.
Measured per setting: tokens per round (k* + 1) of sequences served by a hit
and by the backup, hit rate, and the chance that a whole batch hits.

  python -m lossless_verify_sample_amd.loop [--config 3] [--rounds 24] [--B 4,16,64] [--policy fresh,random]
"""
import argparse
import json
import math

import torch

import lossless_verify_sample_amd as ssd
from lossless_verify_sample_amd import workloads as W

SLOT_SEED = 1 << 20  # per-slot seeds of the pre-speculation: (base << 32) | (SLOT_SEED * (s + 1) + round)


def slot_seed(cfg, r, s):
    return (cfg.base_seed << 32) | (SLOT_SEED * (s + 1) + r)


def _sample(cfg, d, T, seed, cache=None):
    return ssd.saguaro_sample(d, T, cfg.F, cfg.C, seed, F_out=cfg.fout, cache=cache)


def run_loop(cfg, rounds, budget, ratio, policy, dev, step0=0, keep=False):
    """Runs `rounds` verification rounds; returns (per-round records,
    summary).  With keep=True every round's inputs and outputs are kept (as
    device tensors) for checking against the oracle."""
    assert policy in ("fresh", "random")
    B, K, V = cfg.B, cfg.K, cfg.V
    T = W.temperatures(cfg, dev)
    Fk = ssd.fanout(budget, K, ratio, V)
    Bgt = sum(Fk)
    ar = torch.arange(B, device=dev)
    # round 0: its draft rows sampled once (no earlier round served it)
    t, d = W.logits(cfg, step0, dev)
    cache = ssd.Cache(Fk, B, K, dev)
    main = _sample(cfg, d, T, W.seed(cfg, step0), cache)
    x, q = main["tokens"], main["q"]
    served_hit = torch.zeros(B, dtype=torch.bool, device=dev)  # round 0: drafted directly
    recs, tok_hit, tok_miss, n_hit, n_miss, whole = [], 0, 0, 0, 0, 0
    for r in range(rounds):
        step = step0 + r
        # the draft pre-speculates round r+1 while round r verifies: its rows'
        # main draw (statistics, top-F lists, keys of round r+1's cache, the
        # fresh-draw backup) and one sigma draw per cache slot
        t1, d1 = W.logits(cfg, step + 1, dev)
        cache1 = ssd.Cache(Fk, B, K, dev)
        main1 = _sample(cfg, d1, T, W.seed(cfg, step + 1), cache1)
        pay = torch.empty((B, Bgt, K), dtype=torch.int32, device=dev)
        payq = torch.empty((B, Bgt, K), dtype=torch.float32, device=dev)
        for s in range(Bgt):
            o = ssd.saguaro_sample(d1, T, cfg.F, cfg.C, slot_seed(cfg, step + 1, s), F_out=cfg.fout)
            pay[:, s] = o["tokens"]
            payq[:, s] = o["q"]
        cache.payload = pay
        cache.miss_fill = policy == "random"
        seed = W.seed(cfg, step)
        # sequences whose drafted tokens are the random backup's
        uni = (~served_hit) if (policy == "random" and r > 0) else torch.zeros(B, dtype=torch.bool, device=dev)
        # verification of round r: sequences drafted by sigma (hits, fresh
        # draws, round 0) against the draft rows; random backup tokens
        # against the uniform draft distribution
        acc = torch.empty(B, dtype=torch.int32, device=dev)
        bonus = torch.empty(B, dtype=torch.int32, device=dev)
        p = torch.empty((B, K), dtype=torch.float32, device=dev)
        idx_s = (~uni).nonzero().flatten()
        idx_u = uni.nonzero().flatten()
        if idx_s.numel() == B:
            v = ssd.verify(t, d, T, cfg.F, cfg.C, seed, x, q, main["stats"], main["topf_idx"])
            acc, bonus, p = v["accept_len"], v["bonus"], v["p"]
        else:
            for idx, uniform in ((idx_s, False), (idx_u, True)):
                if idx.numel() == 0:
                    continue
                ts = t.index_select(0, idx).contiguous()
                if uniform:
                    # all-zero draft rows: softmax is uniform (F = 0, C = 1);
                    # a seed of its own for this call's acceptance draws
                    Tu = T.index_select(0, idx).contiguous()
                    v = ssd.verify(ts, torch.zeros_like(ts), Tu, 0, 1.0, uniform_seed(seed),
                                   x.index_select(0, idx).contiguous(), q.index_select(0, idx).contiguous(),
                                   uniform_stats(idx.numel(), K, V, Tu), None)
                else:
                    ds = d.index_select(0, idx).contiguous()
                    v = ssd.verify(ts, ds, T.index_select(0, idx).contiguous(), cfg.F, cfg.C, seed,
                                   x.index_select(0, idx).contiguous(), q.index_select(0, idx).contiguous(),
                                   main["stats"].view(B, K + 1, 2).index_select(0, idx).reshape(-1, 2).contiguous(),
                                   main["topf_idx"].index_select(0, idx).contiguous())
                acc[idx], bonus[idx], p[idx] = v["accept_len"], v["bonus"], v["p"]
        hit, slot, ctok = ssd.cache_lookup(cache.keys, cache.depth_off, pay, acc, bonus,
                                           miss_fill=policy == "random", V=V, seed=seed)
        got = (acc + 1).to(torch.int64)
        if r > 0:
            tok_hit += int(got[served_hit].sum())
            tok_miss += int(got[~served_hit].sum())
            n_hit += int(served_hit.sum())
            n_miss += int((~served_hit).sum())
            whole += int(bool(served_hit.all()))
        # round r+1's drafted tokens
        hb = hit.bool()
        sl = slot.clamp_min(0).long()
        q_hit = payq[ar, sl]
        if policy == "fresh":
            x1 = torch.where(hb.unsqueeze(1), ctok, main1["tokens"])
            q1 = torch.where(hb.unsqueeze(1), q_hit, main1["q"])
        else:
            x1 = ctok
            q1 = torch.where(hb.unsqueeze(1), q_hit, torch.full_like(q_hit, 1.0 / V))
        if keep:
            recs.append(dict(t=t, d=d, x=x, q=q, main=main, keys=cache.keys.clone(), fanout=Fk, pay=pay, payq=payq,
                             uni=uni.clone(), seed=seed, acc=acc.clone(), bonus=bonus.clone(), p=p.clone(),
                             hit=hit, slot=slot, ctok=ctok, x1=x1.clone(), q1=q1.clone(), main1=main1, d1=d1,
                             step=step))
        t, d, main, cache = t1, d1, main1, cache1
        x, q = x1.contiguous(), q1.contiguous()
        served_hit = hb
    summary = dict(policy=policy, B=B, rounds=rounds, budget=budget, fanout=Fk,
                   hit_rate=round(n_hit / max(1, n_hit + n_miss), 4),
                   tokens_per_round_hit=round(tok_hit / max(1, n_hit), 4),
                   tokens_per_round_backup=round(tok_miss / max(1, n_miss), 4),
                   tokens_per_round=round((tok_hit + tok_miss) / max(1, n_hit + n_miss), 4),
                   whole_batch_hit=round(whole / max(1, rounds - 1), 4))
    return recs, summary


def uniform_seed(seed):
    """Seed of the verification call over random backup tokens (its Philox
    streams differ from the main call's, whose sequence indices it reuses)."""
    return seed ^ (1 << 31)


def uniform_stats(n, K, V, T):
    """ssd_row_stats of n sequences' K+1 all-zero draft rows: max 0, argmax 0,
    lse ln V (greedy rows 0)."""
    st = torch.zeros((n * (K + 1), 2), dtype=torch.float64, device=T.device)
    lse = torch.where(T > 0, torch.full_like(T, math.log(V)), torch.zeros_like(T)).double()
    st[:, 0] = lse.repeat_interleave(K + 1)
    return st


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--rounds", type=int, default=24)
    ap.add_argument("--B", default="4,16,64")
    ap.add_argument("--policy", default="fresh,random")
    ap.add_argument("--budget", type=int, default=64)
    ap.add_argument("--ratio", type=float, default=0.6)
    a = ap.parse_args()
    dev = torch.device("cuda:0")
    base = W.CONFIGS[a.config]
    for B in [int(x) for x in a.B.split(",")]:
        cfg = W.custom(B, base.K, base.V, base.dtype, T=base.T, F=base.F, C=base.C, kind=base.kind,
                       draft_sd=base.draft_sd, target_sd=base.target_sd, F_out=base.F_out, base_seed=base.base_seed,
                       greedy_half=base.greedy_half)
        res = {}
        for pol in a.policy.split(","):
            _, s = run_loop(cfg, a.rounds, a.budget, a.ratio, pol, dev, step0=10_000)
            s["workload"] = f"{base.name} recipe at B={B}"
            res[pol] = s
            print(json.dumps(s), flush=True)
        if "fresh" in res and "random" in res:
            # back-off rule on the measurements: accurate backup = a fresh
            # draw costing one more round, fast backup = random tokens at no
            # cost; tokens per sequence and round as measured
            f, rnd = res["fresh"], res["random"]
            p = (f["hit_rate"] + rnd["hit_rate"]) / 2
            use_fast, gain = ssd.backoff([p] * B, 1.0, 1.0, 0.0, f["tokens_per_round"], rnd["tokens_per_round_backup"])
            print(json.dumps({"B": B, "backoff_use_fast": use_fast, "gain_fast_over_accurate": round(gain, 4),
                              "assumed": "t_round = t_slow = 1, t_fast = 0"}), flush=True)


if __name__ == "__main__":
    main()
