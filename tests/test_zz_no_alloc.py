"""ssd_round_noalloc, the round step on the library's own static scratch for
callers that cannot allocate device memory, against ssd_round with a caller
workspace: every output identical (verification, sampling, cache keys and
lookup) on two calls in a row, the second with a smaller input, plus the
calls with only one half of the step."""
import pytest
import torch

import lossless_verify_sample_amd as ssd
from lossless_verify_sample_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    # B, K, V, dtype, T, budget: the benchmark's shape, then a smaller fp16 one
    (64, 7, 151936, torch.bfloat16, 1.0, 64),
    (6, 3, 20000, torch.float16, 0.8, 16),
]


def _inputs(case):
    B, K, V, dt, T, budget = case
    cfg = W.custom(B, K, V, dt, T=T, F=4, C=0.5, kind="zipf", draft_sd=1.0, F_out=4)
    t, d = W.logits(cfg, 0, DEV)
    _, d1 = W.logits(cfg, 1, DEV)
    temp = torch.full((B,), T, device=DEV)
    temp[: max(1, B // 8)] = 0.0  # greedy sequences
    Fk = ssd.fanout(budget, K, 0.6, V)
    pay = W.payload(cfg, budget, 0, DEV)
    c0 = ssd.Cache(Fk, B, K, DEV, payload=pay, miss_fill=True)
    s0 = ssd.saguaro_sample(d, temp, 4, 0.5, 21, F_out=4, cache=c0)
    torch.cuda.synchronize()
    return dict(case=case, t=t, d=d, d1=d1, T=temp, Fk=Fk, pay=pay, c0=c0, s0=s0)


def _run(x, noalloc, halves=("v", "s")):
    """One step: verification of round 0 and sampling of round 1, every
    output in fresh buffers; returns clones of all of them."""
    B, K, V, *_ = x["case"]
    c0 = ssd.Cache(x["Fk"], B, K, DEV, payload=x["pay"], keys=x["c0"].keys, miss_fill=True)
    c1 = ssd.Cache(x["Fk"], B, K, DEV, payload=x["pay"])
    s0 = x["s0"]
    va = dict(target=x["t"], draft=x["d"], temperature=x["T"], F=4, C=0.5, seed=21, tokens=s0["tokens"],
              draft_q=s0["q"], draft_stats=s0["stats"], draft_topf_idx=s0["topf_idx"], cache=c0)
    sa = dict(draft=x["d1"], temperature=x["T"], F=4, C=0.5, seed=22, F_out=4, cache=c1)
    v, s = ssd.round_step(va if "v" in halves else None, sa if "s" in halves else None, noalloc=noalloc)
    out = {}
    if v is not None:
        out.update({"v_" + k: y.clone() for k, y in v.items() if y is not None})
        out.update(hit=c0.hit.clone(), slot=c0.slot.clone(), tokens=c0.tokens.clone())
    if s is not None:
        out.update({"s_" + k: y.clone() for k, y in s.items()})
        out["keys1"] = c1.keys.clone()
    return out


def _same(got, ref):
    assert got.keys() == ref.keys()
    for k in ref:
        assert torch.equal(got[k], ref[k]), k


def test_noalloc_matches_round_on_two_calls_second_smaller():
    xs = [_inputs(c) for c in CASES]
    refs = [_run(x, False) for x in xs]
    torch.cuda.synchronize()
    gots = [_run(x, True) for x in xs]  # two calls in a row on the scratch, the second smaller
    torch.cuda.synchronize()
    for x, g, r in zip(xs, gots, refs):
        print(f"noalloc {x['case'][:4]}: accepted {r['v_accept_len'][:8].tolist()} hits {int(r['hit'].sum())}",
              flush=True)
        _same(g, r)


def test_noalloc_single_halves():
    x = _inputs(CASES[1])
    for halves in (("v",), ("s",)):
        ref = _run(x, False, halves)
        got = _run(x, True, halves)
        torch.cuda.synchronize()
        _same(got, ref)


def test_noalloc_rejects_requests_beyond_the_scratch():
    """A verification needing more than the scratch half is refused with
    SSD_ERR_SCRATCH_LIMIT before any launch (B = 130 sequences of K = 7 at
    V = 2^20: 1040 rows of 512 blocks, 8.3 MiB of partials)."""
    B, K, V = 130, 7, 1 << 20
    assert ssd.workspace_bytes(ssd.OP_VERIFY, B, K, V) > (8 << 20)
    t = torch.empty((B, K + 1, V), dtype=torch.bfloat16, device=DEV)
    temp = torch.ones(B, device=DEV)
    tok = torch.zeros((B, K), dtype=torch.int32, device=DEV)
    q = torch.ones((B, K), device=DEV)
    st = torch.zeros((B * (K + 1), 2), dtype=torch.float64, device=DEV)
    tf = torch.zeros((B, K + 1, 4), dtype=torch.int32, device=DEV)
    va = dict(target=t, draft=t, temperature=temp, F=4, C=0.5, seed=1, tokens=tok, draft_q=q, draft_stats=st,
              draft_topf_idx=tf)
    with pytest.raises(ssd.SSDError, match="SCRATCH_LIMIT"):
        ssd.round_step(va, None, noalloc=True)
    del t
