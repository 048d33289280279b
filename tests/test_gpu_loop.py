"""The cache-served multi-round loop (lossless_verify_sample_amd.loop) on a
small shape, round by round against the oracle: each round's main draft draw
(tokens, q, statistics, top-F lists) and cache keys; every slot's
pre-speculation (a sigma_{F,C} draw of the next round's draft rows under the
slot's seed); the verification of the drafted tokens the previous round's
lookup selected (against sigma, or against the uniform draft for random
backup tokens); the lookup; and the selection of the next round's drafted
tokens and their q (the slot's payload on a hit, the backup on a miss)."""
import numpy as np
import pytest
import torch

from lossless_verify_sample_amd import loop as LP
from lossless_verify_sample_amd import workloads as W
from oracle import ssd as O
from parity import NEAR, Report, compare_draft, compare_verify, raw_host, stats_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np(x):
    return x.cpu().numpy()


@pytest.mark.parametrize("policy", ["fresh", "random"])
def test_loop_against_oracle(policy):
    cfg = W.custom(6, 3, 5000, torch.bfloat16, T=0.9, F=2, C=0.5, kind="zipf", draft_sd=0.4, F_out=2,
                   greedy_half=True)
    B, K, V = cfg.B, cfg.K, cfg.V
    recs, summary = LP.run_loop(cfg, 6, 12, 0.6, policy, DEV, keep=True)
    torch.cuda.synchronize()
    print(summary, flush=True)
    Th = W.temperatures(cfg, DEV).cpu().numpy().astype(np.float64)
    rep = Report()
    for r, R in enumerate(recs):
        Fk = R["fanout"]
        zt, zd = O.decode(raw_host(R["t"]), "bf16"), O.decode(raw_host(R["d"]), "bf16")
        # the round's main draw and its cache keys
        od = O.draft_sample(zd, Th, cfg.F, cfg.C, W.seed(cfg, R["step"]), F_out=max(max(Fk), cfg.fout))
        m = R["main"]
        g_s = dict(tokens=_np(m["tokens"]), q=_np(m["q"]).astype(np.float64), stats=stats_np(m["stats"], B, K + 1),
                   topf_idx=_np(m["topf_idx"]), topf_val=_np(m["topf_val"]))
        compare_draft(rep, g_s, dict(od, topf_idx=od["topf_idx"][:, :, :cfg.fout],
                                     topf_val=od["topf_val"][:, :, :cfg.fout]), Th)
        keys_o, off = O.build_keys(od["topf_idx"], Fk)
        assert np.array_equal(_np(R["keys"]), keys_o), r
        # every slot's pre-speculation of the next round
        zd1 = O.decode(raw_host(R["d1"]), "bf16")
        pay, payq = _np(R["pay"]), _np(R["payq"])
        for s in range(sum(Fk)):
            os_ = O.draft_sample(zd1, Th, cfg.F, cfg.C, LP.slot_seed(cfg, R["step"] + 1, s))
            for b in range(B):
                for j in range(K):
                    rep.units += 1
                    if os_["margin"][b, j] < NEAR:
                        rep.near += 1
                        continue
                    assert pay[b, s, j] == os_["tokens"][b, j], (r, s, b, j)
                    assert abs(payq[b, s, j] - os_["q"][b, j]) <= 1e-5 * os_["q"][b, j], (r, s, b, j)
        # verification of the drafted tokens (sigma, or uniform for random backup tokens)
        x = _np(R["x"]).astype(np.int64)
        uni = _np(R["uni"]).astype(bool)
        g_v = dict(accept_len=_np(R["acc"]), bonus=_np(R["bonus"]), p=_np(R["p"]).astype(np.float64))
        idx_s, idx_u = np.nonzero(~uni)[0], np.nonzero(uni)[0]
        for idx, uniform in ((idx_s, False), (idx_u, True)):
            if idx.size == 0:
                continue
            sub = {k: v[idx] for k, v in g_v.items()}
            if uniform:
                ov = O.verify(zt[idx], np.zeros_like(zd[idx]), Th[idx], 0, 1.0, LP.uniform_seed(R["seed"]), x[idx])
            else:
                ov = O.verify(zt[idx], zd[idx], Th[idx], cfg.F, cfg.C, R["seed"], x[idx])
            compare_verify(rep, sub, ov, Th[idx])
        # the lookup of the GPU's outcome, and the next round's drafted tokens
        oh, osl, ot = O.cache_lookup(keys_o, off, pay, g_v["accept_len"], g_v["bonus"], seed=R["seed"], V=V,
                                     miss_fill=policy == "random")
        assert np.array_equal(_np(R["hit"]), oh) and np.array_equal(_np(R["slot"]), osl), r
        assert np.array_equal(_np(R["ctok"]), ot), r
        x1, q1 = _np(R["x1"]), _np(R["q1"])
        m1 = R["main1"]
        for b in range(B):
            if oh[b]:
                assert np.array_equal(x1[b], pay[b, osl[b]]) and np.array_equal(q1[b], payq[b, osl[b]])
            elif policy == "fresh":
                assert np.array_equal(x1[b], _np(m1["tokens"])[b]) and np.array_equal(q1[b], _np(m1["q"])[b])
            else:
                assert np.array_equal(x1[b], ot[b]) and np.all(q1[b] == np.float32(1.0 / V))
        print(f"{policy} round {r}: accepted {g_v['accept_len'].tolist()} hits {oh.tolist()} "
              f"random-backup rows {idx_u.tolist()}", flush=True)
    assert rep.ok(), rep.fails
    print(f"{policy}: units {rep.units} near ties {rep.near}", flush=True)
    assert summary["hit_rate"] > 0.0  # some rounds were served from the cache
