"""GPU-versus-oracle parity checks.

Rules: drafted tokens, accepted lengths, bonus tokens, top-F lists, argmax,
row maxima and cache results are bit-exact, except units whose deciding
margin (the oracle's |u - rho| or top-2 Gumbel score gap) is below 1e-5;
those are counted, and after a near-tie acceptance the sequence's later
fields are exempt.  Probabilities agree within 1e-5 relative (+1e-30
absolute for underflow), log-normalisers within 1e-5 * max(1, |L|).
"""
import math
from dataclasses import dataclass, field

import numpy as np
import torch

import lossless_verify_sample_amd as ssd
from oracle import pool as OP
from oracle import ssd as O

NEAR = 1e-5
RTOL = 1e-5
ATOL = 1e-30

DTNAME = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}


def raw_host(x):
    """Stored logits as numpy: float32, or the uint16 bit patterns of bf16/fp16."""
    if x.dtype == torch.float32:
        return x.detach().cpu().numpy()
    return x.detach().view(torch.int16).cpu().numpy().view(np.uint16)


@dataclass
class Report:
    units: int = 0
    near: int = 0
    hits: int = 0
    fails: list = field(default_factory=list)

    def fail(self, msg):
        if len(self.fails) < 50:
            self.fails.append(msg)

    def add(self, other):
        self.units += other.units
        self.near += other.near
        self.fails += other.fails[: max(0, 50 - len(self.fails))]

    def ok(self):
        return not self.fails


def _close(g, o):
    return abs(g - o) <= RTOL * abs(o) + ATOL


def stats_np(st, B, K1):
    lse, mx, am = ssd.stats_fields(st)
    return (lse.cpu().numpy().reshape(B, K1), mx.cpu().numpy().reshape(B, K1).astype(np.float64),
            am.cpu().numpy().reshape(B, K1))


def compare_stats(rep, tag, g, o_max, o_lse, o_am, greedy):
    lse, mx, am = g
    B, K1 = mx.shape
    for b in range(B):
        for j in range(K1):
            if mx[b, j] != o_max[b, j]:
                rep.fail(f"{tag} max b={b} j={j}: {mx[b, j]} vs {o_max[b, j]}")
            if am[b, j] != o_am[b, j]:
                rep.fail(f"{tag} argmax b={b} j={j}: {am[b, j]} vs {o_am[b, j]}")
            ol = 0.0 if greedy[b] else o_lse[b, j]
            if abs(lse[b, j] - ol) > 1e-5 * max(1.0, abs(ol)):
                rep.fail(f"{tag} lse b={b} j={j}: {lse[b, j]} vs {ol}")


def compare_draft(rep, g, o, T):
    """g: GPU sample outputs (numpy), o: oracle draft_sample output."""
    B, K = o["tokens"].shape
    greedy = [O.is_greedy(t) for t in T]
    for b in range(B):
        for j in range(K):
            rep.units += 1
            near = o["margin"][b, j] < NEAR
            rep.near += int(near)
            if g["tokens"][b, j] != o["tokens"][b, j]:
                if not near:
                    rep.fail(f"draft token b={b} j={j}: {g['tokens'][b, j]} vs {o['tokens'][b, j]} "
                             f"(margin {o['margin'][b, j]:.3g})")
                continue
            if not _close(g["q"][b, j], o["q"][b, j]):
                rep.fail(f"q b={b} j={j}: {g['q'][b, j]!r} vs {o['q'][b, j]!r}")
    compare_stats(rep, "draft", g["stats"], o["max"], o["lse"], o["argmax"], greedy)
    fo = o["topf_idx"].shape[2]
    if fo:
        if not np.array_equal(g["topf_idx"][:, :, :fo], o["topf_idx"]):
            bad = np.argwhere(g["topf_idx"][:, :, :fo] != o["topf_idx"])[:3]
            rep.fail(f"topf idx differs at {bad.tolist()}")
        if not np.array_equal(g["topf_val"][:, :, :fo].astype(np.float64), o["topf_val"]):
            rep.fail("topf values differ")


def compare_verify(rep, g, o, T):
    B, K = o["p"].shape
    greedy = [O.is_greedy(t) for t in T]
    for b in range(B):
        ko = int(o["accept_len"][b])
        exempt = False
        for j in range(min(ko, K - 1) + 1 if K > 0 else 0):
            rep.units += 1
            if o["acc_margin"][b, j] < NEAR:
                rep.near += 1
                exempt = True
        rep.units += 1
        bn = o["bonus_margin"][b] < NEAR
        rep.near += int(bn)
        if not exempt and g["accept_len"][b] != ko:
            rep.fail(f"accept_len b={b}: {g['accept_len'][b]} vs {ko}")
        elif not exempt and not bn and g["bonus"][b] != o["bonus"][b]:
            rep.fail(f"bonus b={b}: {g['bonus'][b]} vs {o['bonus'][b]} (margin {o['bonus_margin'][b]:.3g})")
        for j in range(K):
            if not _close(g["p"][b, j], o["p"][b, j]):
                rep.fail(f"p b={b} j={j}: {g['p'][b, j]!r} vs {o['p'][b, j]!r}")
    if g.get("stats") is not None:
        compare_stats(rep, "target", g["stats"], o["max"], o["lse"], o["argmax"], greedy)


def gpu_round(target, draft, T, F, C, seed, F_out=None, cache=None):
    """One sample + verify on the GPU (with a speculation cache when given:
    sampling writes its keys, verification looks the outcome up); numpy
    copies of every output."""
    B, K1, V = draft.shape
    smp = ssd.saguaro_sample(draft, T, F, C, seed, F_out=F_out, cache=cache)
    ver = ssd.verify(target, draft, T, F, C, seed, smp["tokens"], smp["q"], smp["stats"], smp["topf_idx"],
                     want_stats=True, cache=cache)
    torch.cuda.synchronize()
    g_s = dict(tokens=smp["tokens"].cpu().numpy(), q=smp["q"].cpu().numpy().astype(np.float64),
               stats=stats_np(smp["stats"], B, K1), topf_idx=smp["topf_idx"].cpu().numpy(),
               topf_val=smp["topf_val"].cpu().numpy())
    g_v = dict(accept_len=ver["accept_len"].cpu().numpy(), bonus=ver["bonus"].cpu().numpy(),
               p=ver["p"].cpu().numpy().astype(np.float64), stats=stats_np(ver["stats"], B, K1))
    return g_s, g_v, smp, ver


def check_round(target, draft, T, F, C, seed, F_out=None, workers=None, pool=None, cache=None):
    """GPU sample + verify against the oracle on the same inputs.  The oracle
    verifies the GPU's drafted tokens so later units stay comparable.  With a
    cache, the keys sampling wrote are checked against the oracle's top
    lists and the lookup against the oracle's lookup of the GPU's (k*,
    bonus), which are themselves checked against the oracle's."""
    g_s, g_v, smp, ver = gpu_round(target, draft, T, F, C, seed, F_out, cache)
    Th = T.cpu().numpy().astype(np.float64)
    dt = DTNAME[draft.dtype]
    fo = F_out if F_out is not None else F
    fl = max(fo, max(cache.fanout)) if cache is not None else fo
    o = OP.run(raw_host(draft), dt, Th, F, C, seed, F_out=fl, target_raw=raw_host(target),
               tokens=g_s["tokens"].astype(np.int64), workers=workers, pool=pool)
    rep = Report()
    od = dict(o["draft"], topf_idx=o["draft"]["topf_idx"][:, :, :fo], topf_val=o["draft"]["topf_val"][:, :, :fo])
    compare_draft(rep, g_s, od, Th)
    compare_verify(rep, g_v, o["verify"], Th)
    if cache is not None:
        compare_cache(rep, cache, o["draft"]["topf_idx"], g_v, seed, draft.shape[2])
    return rep, g_s, g_v, smp, ver, o


def compare_cache(rep, cache, o_lists, g_v, seed, V):
    """Keys [B, Bgt] against the first F_k entries of the oracle's top lists
    of each draft row; hit, slot and gathered (or filled) tokens against the
    oracle's lookup of the GPU's accepted lengths and bonus tokens."""
    keys_o, off = O.build_keys(o_lists, cache.fanout)
    keys = cache.keys.cpu().numpy()
    if not np.array_equal(keys, keys_o):
        bad = np.argwhere(keys != keys_o)[:3]
        rep.fail(f"cache keys differ at {bad.tolist()}")
    pay = cache.payload.cpu().numpy() if cache.payload is not None else np.zeros((keys.shape[0], cache.Bgt, 0))
    oh, osl, ot = O.cache_lookup(keys_o, off, pay, g_v["accept_len"], g_v["bonus"], seed=seed, V=V,
                                 miss_fill=cache.miss_fill)
    for name, g, o in (("hit", cache.hit, oh), ("slot", cache.slot, osl), ("tokens", cache.tokens, ot)):
        if not np.array_equal(g.cpu().numpy(), o):
            rep.fail(f"cache {name} differs")
    rep.hits = int(oh.sum())
