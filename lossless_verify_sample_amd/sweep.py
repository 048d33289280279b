"""Synthetic multi-round SSD loop on one GPU: acceptance against bonus
predictability as C and F vary, cache hit rate against batch size, and the
fan-out allocated from measured statistics.

Every round samples the draft rows with Saguaro sigma_{F,C} (ssd_saguaro_sample,
writing the speculation-cache keys under the truncated-geometric fan-out),
verifies them (ssd_verify with the cache lookup) and records the accepted
lengths, the bonus tokens and the bonus's rank in the draft row's top-64 list
([SSD-B] part 2: lowering C moves residual mass, and with it the bonus,
into the draft's top-F set, at some cost in acceptance; part 1: the budget
goes where acceptance stops).  From those records: P(k* = k), the hit curves
h_k(F) = P(bonus among the top F of draft row k | k* = k), the fan-out that
ssd_fanout_greedy allocates from them, and its hit rate on fresh rounds
beside the geometric fan-out's.  The logits are synthetic (the workload's
recipe with fresh seeds per round); nothing here feeds tokens back into a
model.

  python -m lossless_verify_sample_amd.sweep [--config 3] [--rounds 32] [--C 1,0.5,0.25] [--F 0,4,16]
"""
import argparse
import json

import torch

import lossless_verify_sample_amd as ssd
from lossless_verify_sample_amd import workloads as W

FMAX = 64


def run(cfg, C, F, fanout, rounds, seed0, dev):
    B, K, V = cfg.B, cfg.K, cfg.V
    T = W.temperatures(cfg, dev)
    rec = dict(acc=[], hit=[], rank=[])
    for r in range(rounds):
        step = seed0 + r
        t, d = W.logits(cfg, step, dev)
        cache = ssd.Cache(fanout, B, K, dev, payload=W.payload(cfg, sum(fanout), step, dev))
        s = ssd.saguaro_sample(d, T, F, C, W.seed(cfg, step), F_out=FMAX, cache=cache)
        v = ssd.verify(t, d, T, F, C, W.seed(cfg, step), s["tokens"], s["q"], s["stats"], s["topf_idx"],
                       cache=cache)
        k = v["accept_len"].long()
        lists = s["topf_idx"][torch.arange(B, device=dev), k]            # [B, FMAX]: draft row k*'s top list
        match = lists == v["bonus"].unsqueeze(1)
        rank = torch.where(match.any(1), match.int().argmax(1), torch.full_like(k, FMAX))
        rec["acc"].append(k)
        rec["hit"].append(cache.hit.clone())
        rec["rank"].append(rank)
    return {n: torch.stack(x).cpu() for n, x in rec.items()}


def stats(rec, K):
    acc, rank = rec["acc"].flatten(), rec["rank"].flatten()
    n = acc.numel()
    a = [float((acc == k).sum()) / n for k in range(K + 1)]
    h = []
    for k in range(K + 1):
        rk = rank[acc == k]
        h.append([float((rk < f).sum()) / max(1, rk.numel()) for f in range(FMAX + 1)])
    return a, h


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--rounds", type=int, default=32)
    ap.add_argument("--C", default="1,0.5,0.25")
    ap.add_argument("--F", default="0,4,16")
    ap.add_argument("--budget", type=int, default=64)
    ap.add_argument("--ratio", type=float, default=0.6)
    a = ap.parse_args()
    dev = torch.device("cuda:0")
    cfg = W.CONFIGS[a.config]
    K, V = cfg.K, cfg.V
    geo = ssd.fanout(a.budget, K, a.ratio, V)
    out = []
    for C in [float(x) for x in a.C.split(",")]:
        for F in [int(x) for x in a.F.split(",")]:
            if (F == 0) != (C == 1.0):
                continue  # F = 0 or C = 1 both give sigma = q: one run covers them
            rec = run(cfg, C, F, geo, a.rounds, 10_000, dev)
            pa, h = stats(rec, K)
            opt = ssd.fanout_greedy(pa, h, a.budget)
            fresh_geo = run(cfg, C, F, geo, a.rounds, 20_000, dev)
            fresh_opt = run(cfg, C, F, opt, a.rounds, 20_000, dev)
            hit = fresh_geo["hit"].float()
            whole = {B: float(hit[:, :B].prod(1).mean()) for B in (1, 4, 16, cfg.B)}
            out.append({"C": C, "F": F,
                        "mean_accepted": round(float(rec["acc"].float().mean()), 3),
                        "tokens_per_round": round(float(rec["acc"].float().mean()) + 1.0, 3),
                        "bonus_in_top1": round(float((rec["rank"] < 1).float().mean()), 3),
                        "bonus_in_top8": round(float((rec["rank"] < 8).float().mean()), 3),
                        "hit_rate_geometric": round(float(hit.mean()), 4),
                        "hit_rate_measured_fanout": round(float(fresh_opt["hit"].float().mean()), 4),
                        "fanout_geometric": geo, "fanout_measured": opt,
                        "whole_batch_hit": {str(B): round(p, 4) for B, p in whole.items()}})
            print(json.dumps(out[-1]), flush=True)
    print("| C | F | mean k* | bonus in top-1 | top-8 | hit (geometric) | hit (measured fan-out) | fan-out from measurements | whole batch hits B=1/4/16/" + str(cfg.B) + " |")
    print("|---|---|---|---|---|---|---|---|---|")
    for r in out:
        wb = "/".join(f"{v:.3f}" for v in r["whole_batch_hit"].values())
        print(f"| {r['C']} | {r['F']} | {r['mean_accepted']} | {r['bonus_in_top1']} | {r['bonus_in_top8']} | "
              f"{r['hit_rate_geometric']} | {r['hit_rate_measured_fanout']} | {r['fanout_measured']} | {wb} |")


if __name__ == "__main__":
    main()
