"""Token-tree verification (ssd_verify_tree) against the oracle's
verify_tree on the same inputs: the node where the walk stops (hence the
accepted path and its length) and the bonus token bit-exact outside near
ties; a path-shaped tree equal to ssd_verify bit for bit.  The drafted
children of node n are independent sigma_{F,C} draws of draft row n: child
rank i takes the token that ssd_saguaro_sample draws at row n under seed
base + i."""
import numpy as np
import pytest
import torch

import lossless_verify_sample_amd as ssd
from lossless_verify_sample_amd import workloads as W
from oracle import ssd as O
from parity import DTNAME, NEAR, raw_host

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16, F16, F32 = torch.bfloat16, torch.float16, torch.float32

TREES = {
    "wide": [-1, 0, 0, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4],
    "deep": [-1, 0, 0, 1, 1, 3, 3, 5, 5],
    "root-only": [-1],
    "binary-63": [-1] + [(m - 1) // 2 for m in range(1, 63)],
}


def _sample_rows(draft, T, F, C, seed, F_out):
    """sigma draws, q, statistics and top-F lists of every row of draft [B, N1, V]
    (ssd_saguaro_sample takes at most 33 rows per sequence and draws at all
    but its last row, so the calls cover rows in overlapping windows); the
    last row is never drawn (the last node of a tree is a leaf)."""
    B, N1, V = draft.shape
    tok = torch.zeros((B, N1), dtype=torch.int32, device=DEV)
    q = torch.ones((B, N1), dtype=torch.float32, device=DEV)
    st = torch.empty((B, N1, 2), dtype=torch.float64, device=DEV)
    tf = torch.empty((B, N1, F_out), dtype=torch.int32, device=DEV)
    lo = 0
    while lo < N1:
        hi = min(N1, lo + 33)
        o = ssd.saguaro_sample(draft[:, lo:hi].contiguous(), T, F, C, seed, F_out=F_out)
        tok[:, lo:hi - 1] = o["tokens"]
        q[:, lo:hi - 1] = o["q"]
        st[:, lo:hi] = o["stats"].view(B, hi - lo, 2)
        tf[:, lo:hi] = o["topf_idx"]
        if hi == N1:
            break
        lo = hi - 1
    return tok, q, st.view(B * N1, 2), tf


def _draft_tree(draft, T, F, C, seed, parent, F_out):
    """Node tokens [B, N+1] and their sigma_{parent} [B, N+1]: child rank i of
    node n is the token drawn at row n by the sampling of seed + i."""
    B, N1, V = draft.shape
    ranks = [0] * N1
    seen = {}
    for m in range(1, N1):
        ranks[m] = seen.get(parent[m], 0)
        seen[parent[m]] = ranks[m] + 1
    draws = [_sample_rows(draft, T, F, C, seed + i, F_out) for i in range(max(seen.values(), default=1))]
    tok = torch.zeros((B, N1), dtype=torch.int32, device=DEV)
    q = torch.ones((B, N1), dtype=torch.float32, device=DEV)
    for m in range(1, N1):
        tok[:, m] = draws[ranks[m]][0][:, parent[m]]
        q[:, m] = draws[ranks[m]][1][:, parent[m]]
    return tok, q, draws[0][2], draws[0][3]


def _check(tree, B, V, dt, T, F, C, kind, gh, steps=6):
    parent = TREES[tree]
    N = len(parent) - 1
    cfg = W.custom(B, N, V, dt, T=T, F=F, C=C, kind=kind, draft_sd=0.6, F_out=max(F, 1), greedy_half=gh)
    temp = W.temperatures(cfg, DEV)
    Th = temp.cpu().numpy().astype(np.float64)
    units = near = 0
    for step in range(steps):
        t, d = W.logits(cfg, step, DEV)
        seed = W.seed(cfg, step)
        tok, q, st, tf = _draft_tree(d, temp, F, C, seed, parent, max(F, 1))
        g = ssd.verify_tree(t, d, temp, F, C, seed, parent, tok, q, st, tf)
        torch.cuda.synchronize()
        zt, zd = O.decode(raw_host(t), DTNAME[dt]), O.decode(raw_host(d), DTNAME[dt])
        o = O.verify_tree(zt, zd, Th, F, C, seed, parent, tok.cpu().numpy().astype(np.int64))
        last, acc, bon = (g[k].cpu().numpy() for k in ("last", "accept_len", "bonus"))
        for b in range(B):
            ev = o["acc_margin"][b][np.isfinite(o["acc_margin"][b])]
            units += ev.size + 1
            tie = bool(np.any(ev < NEAR))
            near += int(tie) + int(o["bonus_margin"][b] < NEAR)
            if tie:
                continue
            assert last[b] == o["last"][b] and acc[b] == o["accept_len"][b], (tree, step, b, last[b], o["last"][b])
            if o["bonus_margin"][b] >= NEAR:
                assert bon[b] == o["bonus"][b], (tree, step, b, bon[b], o["bonus"][b])
        print(f"tree {tree} V={V} {DTNAME[dt]} step {step}: last {last.tolist()} bonus {bon.tolist()}", flush=True)
    print(f"tree {tree}: units {units} near ties {near}", flush=True)


CASES = [
    # tree, B, V, dtype, T, F, C, kind, greedy_half
    ("wide", 4, 5000, BF16, 1.0, 2, 0.5, "zipf", False),
    ("wide", 6, 20000, F16, 0.8, 4, 0.3, "peaks", True),
    ("deep", 4, 5001, F32, 1.2, 3, 0.6, "normal", False),   # unaligned rows
    ("deep", 3, 300000, BF16, 1.0, 4, 0.5, "zipf", False),  # more than 128 blocks
    ("root-only", 5, 40000, BF16, 1.0, 4, 0.5, "zipf", True),
    ("binary-63", 2, 8000, BF16, 1.0, 0, 1.0, "normal", False),  # 63 nodes, F = 0
    ("wide", 8, 151936, BF16, 1.0, 4, 0.5, "zipf", False),  # the Qwen-3 vocabulary
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-B{c[1]}V{c[2]}{DTNAME[c[3]]}")
def test_tree_against_oracle(case):
    _check(*case)


def test_path_tree_equals_verify():
    """parent[m] = m - 1: the walk, the bonus and the accepted length are
    ssd_verify's, bit for bit."""
    B, K, V = 16, 5, 60000
    cfg = W.custom(B, K, V, BF16, T=0.9, F=4, C=0.5, kind="zipf", draft_sd=0.7, greedy_half=True)
    temp = W.temperatures(cfg, DEV)
    for step in range(4):
        t, d = W.logits(cfg, step, DEV)
        seed = W.seed(cfg, step)
        s = ssd.saguaro_sample(d, temp, 4, 0.5, seed)
        v = ssd.verify(t, d, temp, 4, 0.5, seed, s["tokens"], s["q"], s["stats"], s["topf_idx"])
        tok = torch.cat([torch.zeros((B, 1), dtype=torch.int32, device=DEV), s["tokens"]], dim=1).contiguous()
        q = torch.cat([torch.ones((B, 1), device=DEV), s["q"]], dim=1).contiguous()
        g = ssd.verify_tree(t, d, temp, 4, 0.5, seed, [-1] + list(range(K)), tok, q, s["stats"], s["topf_idx"])
        torch.cuda.synchronize()
        assert torch.equal(g["accept_len"], v["accept_len"]) and torch.equal(g["last"], v["accept_len"])
        assert torch.equal(g["bonus"], v["bonus"])


def test_leaf_after_rejected_sibling():
    """Regression: the walk rejects a sibling (leaving residual mass), accepts
    the next one and stops at a leaf; the bonus is drawn from that leaf's
    p, not from the parent's residual.  Tree root -> 1 -> {2, 3}; row 0 of
    draft and target are equal (node 1 accepted), node 2's token is outside
    [0, V) (rejected), node 3's token is where target row 1 puts almost all
    its mass and the draft almost none (accepted)."""
    B, V, T = 4, 5000, 1.0
    parent = [-1, 0, 1, 1]
    cfg = W.custom(B, 3, V, F32, T=T, F=0, C=1.0, kind="normal", draft_sd=0.5)
    t, d = W.logits(cfg, 0, DEV)
    t[:, 0] = d[:, 0]
    t[:, 1, 0] = 12.0
    d[:, 1, 0] = -8.0
    temp = torch.full((B,), T, device=DEV)

    def sig(row, x):  # softmax probability of token x (F = 0, C = 1: sigma = q)
        z = row.double()
        return float(torch.exp(z[x] - torch.logsumexp(z, 0)))

    tok = torch.zeros((B, 4), dtype=torch.int32, device=DEV)
    q = torch.ones((B, 4), dtype=torch.float32, device=DEV)
    for b in range(B):
        tok[b, 1], q[b, 1] = 7, sig(d[b, 0], 7)
        tok[b, 2], q[b, 2] = V, 0.5
        tok[b, 3], q[b, 3] = 0, sig(d[b, 1], 0)
    st = ssd.saguaro_sample(d, temp, 0, 1.0, 1, F_out=1)
    zt, zd = O.decode(raw_host(t), "f32"), O.decode(raw_host(d), "f32")
    for seed in range(8):
        g = ssd.verify_tree(t, d, temp, 0, 1.0, seed, parent, tok, q, st["stats"], st["topf_idx"])
        torch.cuda.synchronize()
        o = O.verify_tree(zt, zd, [T] * B, 0, 1.0, seed, parent, tok.cpu().numpy().astype(np.int64))
        assert (o["last"] == 3).all()
        assert g["last"].tolist() == o["last"].tolist()
        for b in range(B):
            if o["bonus_margin"][b] >= NEAR:
                assert int(g["bonus"][b]) == o["bonus"][b], (seed, b)
