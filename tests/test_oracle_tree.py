"""Pins of token-tree verification (oracle.ssd.verify_tree).

Reading: recursive rejection sampling over the children of each node, the
residual renormalised after each rejected sibling (the textbook multi-
candidate rule; the pages name token-tree speculation only as a direction
SSD combines with).  Pinned by
- losslessness by exact enumeration: every token assignment of small trees
  (V <= 5, up to 3 levels, contexts whose target and draft rows depend on the
  token path), weighted by the draft law; at every reached context the
  emitted token follows the target row of that context;
- the seeded oracle against the exact law of (stopping node, bonus) for
  fixed drafted tokens (chi-square over seeds);
- reduction to the chain: a tree with one child per node gives verify()'s
  accepted length and bonus;
- greedy and degenerate cases."""
import itertools
import math

import numpy as np
import pytest
from scipy import stats

from oracle import ssd as O

TREES = {
    "two-branch": [-1, 0, 0, 1, 2],
    "three-wide": [-1, 0, 0, 0, 1, 1],
    "three-level": [-1, 0, 0, 1, 1, 3],
    "chain": [-1, 0, 1, 2],
}


def _ctx_rows(V, seed):
    cache = {}

    def rows(path):
        if path not in cache:
            rng = np.random.default_rng([seed, len(path)] + [x + 1 for x in path])
            zt = rng.standard_normal(V) * 1.5
            cache[path] = (zt, zt + rng.standard_normal(V) * 0.8)
        return cache[path]
    return rows


def _rrs(r, s, toks):
    """Exact recursive rejection sampling at one node: probability that each
    child is accepted, and the law of the bonus drawn when all are rejected
    (times the chance of getting there)."""
    acc, rem = [], 1.0
    for x in toks:
        if not 0 <= x < len(r):
            a = 0.0
        elif s[x] > 0:
            a = min(1.0, r[x] / s[x])
        else:
            a = 1.0 if r[x] > 0 else 0.0
        acc.append(rem * a)
        rem *= 1.0 - a
        nr = np.maximum(0.0, r - s)
        if nr.sum() > 0:
            r = nr / nr.sum()
    return acc, rem * r


@pytest.mark.parametrize("name", sorted(TREES))
@pytest.mark.parametrize("V,T,F,C", [(4, 1.0, 1, 0.5), (3, 0.7, 2, 0.3), (4, 1.0, 0, 1.0), (4, 0.0, 1, 0.5)])
def test_tree_losslessness_by_enumeration(name, V, T, F, C):
    parent = TREES[name]
    if name == "three-level" and V > 3:
        V = 3
    kids = O.tree_children(parent)
    N1 = len(parent)
    rows = _ctx_rows(V, 5)
    reach, emit = {}, {}
    for xs in itertools.product(range(V), repeat=N1 - 1):
        tok = (None,) + xs
        path = [()] * N1
        for m in range(1, N1):
            path[m] = path[parent[m]] + (tok[m],)
        w = 1.0
        for m in range(1, N1):
            w *= O.sigma(rows(path[parent[m]])[1], T, F, C)["sigma"][tok[m]]
        if w == 0:
            continue
        pr = {0: w}
        for n in range(N1):  # parents come before children
            if pr.get(n, 0.0) == 0.0:
                continue
            zt, zd = rows(path[n])
            p = O.softmax_t(zt, T)["p"]
            e = np.zeros(V)
            if O.is_greedy(T):
                a = int(np.argmax(zt))
                hit = next((m for m in kids[n] if tok[m] == a), None)
                if hit is not None:
                    pr[hit] = pr[n]
                e[a] = 1.0
            else:
                acc, bon = _rrs(p, O.sigma(zd, T, F, C)["sigma"], [tok[m] for m in kids[n]])
                for m, a in zip(kids[n], acc):
                    pr[m] = pr[n] * a
                    e[tok[m]] += a
                e += bon
            reach[path[n]] = reach.get(path[n], 0.0) + pr[n]
            emit[path[n]] = emit.get(path[n], np.zeros(V)) + pr[n] * e
    assert reach
    for ctx, rp in reach.items():
        p = O.softmax_t(rows(ctx)[0], T)["p"]
        assert np.allclose(emit[ctx] / rp, p, rtol=0, atol=1e-12), (ctx, emit[ctx] / rp, p)


def _exact_outcome_law(zt, zd, T, F, C, parent, tokens):
    """Law of (stopping node, bonus) for fixed rows and drafted tokens."""
    kids = O.tree_children(parent)
    N1, V = zt.shape
    law = np.zeros((N1, V))
    pr = {0: 1.0}
    for n in range(N1):
        if pr.get(n, 0.0) == 0.0:
            continue
        p = O.softmax_t(zt[n], T)["p"]
        acc, bon = _rrs(p, O.sigma(zd[n], T, F, C)["sigma"], [tokens[m] for m in kids[n]])
        for m, a in zip(kids[n], acc):
            pr[m] = pr[n] * a
        law[n] += pr[n] * (bon if kids[n] else p)
    return law


def test_seeded_tree_matches_exact_law():
    parent = TREES["three-wide"]
    N1, V, T, F, C = len(parent), 6, 1.0, 2, 0.5
    rng = np.random.default_rng(31)
    zt = rng.standard_normal((1, N1, V)) * 1.5
    zd = zt + rng.standard_normal((1, N1, V)) * 0.7
    tokens = np.array([[0, 2, 2, 5, 1, 3]])
    law = _exact_outcome_law(zt[0], zd[0], T, F, C, parent, tokens[0])
    assert abs(law.sum() - 1.0) < 1e-12
    n = 6000
    counts = np.zeros_like(law)
    for seed in range(n):
        v = O.verify_tree(zt, zd, [T], F, C, seed, parent, tokens, blk=4)
        counts[v["last"][0], v["bonus"][0]] += 1
        assert v["accept_len"][0] == O.tree_depth(parent)[v["last"][0]]
    m = law.ravel() > 0
    assert np.all(counts.ravel()[~m] == 0)
    assert stats.chisquare(counts.ravel()[m], law.ravel()[m] * n).pvalue > 1e-4


def test_chain_tree_reduces_to_verify():
    rng = np.random.default_rng(32)
    for trial in range(40):
        K = int(rng.integers(0, 5))
        V = int(rng.integers(2, 40))
        B = 3
        T = [1.0, 0.6, 0.0]
        zt = rng.standard_normal((B, K + 1, V)) * 2
        zd = zt + rng.standard_normal((B, K + 1, V))
        F, C = int(rng.integers(0, min(V, 4) + 1)), float(rng.choice([0.3, 0.5, 1.0]))
        d = O.draft_sample(zd, T, F, C, trial, blk=8)
        v = O.verify(zt, zd, T, F, C, trial, d["tokens"], blk=8)
        tok = np.concatenate([np.zeros((B, 1), np.int64), d["tokens"]], axis=1)
        t = O.verify_tree(zt, zd, T, F, C, trial, [-1] + list(range(K)), tok, blk=8)
        for b in range(B):
            if np.any(v["acc_margin"][b] < 1e-9) or v["bonus_margin"][b] < 1e-9:
                continue
            assert t["accept_len"][b] == v["accept_len"][b] == t["last"][b], (trial, b)
            assert t["bonus"][b] == v["bonus"][b], (trial, b)


def test_tree_greedy_and_degenerate_cases():
    parent = [-1, 0, 0, 1, 2, 2]
    V = 6
    rng = np.random.default_rng(33)
    zt = rng.standard_normal((2, 6, V))
    am = np.argmax(zt, axis=2)
    # greedy: the first child holding the argmax is taken, bonus = argmax where the walk stops
    tok = np.array([[0, (am[0, 0] + 1) % V, am[0, 0], 0, am[0, 2], 0],
                    [0, 0, 0, 0, 0, 0]])
    tok[1, 1] = (am[1, 0] + 1) % V
    tok[1, 2] = (am[1, 0] + 2) % V
    t = O.verify_tree(zt, zt, [0.0, 0.0], 2, 0.5, 1, parent, tok)
    assert t["last"][0] == 4 and t["accept_len"][0] == 2 and t["bonus"][0] == am[0, 4]
    assert t["last"][1] == 0 and t["accept_len"][1] == 0 and t["bonus"][1] == am[1, 0]
    # identical draft and target: the first child is always accepted
    z = rng.standard_normal((1, 6, V))
    for seed in range(20):
        toks = np.array([[0, 1, 3, 2, 5, 4]])
        s = O.verify_tree(z, z, [1.0], 2, 1.0, seed, parent, toks)
        assert s["last"][0] == 3 and s["accept_len"][0] == 2
    # a token outside [0, V) is rejected (ratio 0); with p = sigma the residual
    # has no mass and stays p, so the next sibling and its first child are
    # accepted with ratio 1
    toks = np.array([[0, V, 2, 0, 0, 0]])
    for seed in range(20):
        s = O.verify_tree(z, z, [1.0], 2, 1.0, seed, parent, toks)
        assert s["last"][0] == 4 and s["accept_len"][0] == 2
        assert 0.0 < s["acc_margin"][0, 1] < 1.0
