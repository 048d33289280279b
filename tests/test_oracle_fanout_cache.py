"""Pins of the fan-out allocation and the speculation-cache lookup."""
import itertools
import os

import numpy as np
import pytest

from oracle import ssd as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    rows = []
    with open(os.path.join(GOLDEN, "fanout_closed_form.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            t = line.split()
            rows.append((int(t[0]), int(t[1]), float(t[2]), int(t[3]), [int(x) for x in t[4:]]))
    return rows


@pytest.mark.parametrize("Bgt,K,ratio,V,expect", _golden())
def test_fanout_hand_worked_values(Bgt, K, ratio, V, expect):
    assert O.fanout(Bgt, K, ratio, V) == expect


@pytest.mark.parametrize("Bgt,K,ratio", [(64, 7, 0.6), (100, 5, 0.3), (13, 3, 0.9), (0, 4, 0.5)])
def test_fanout_sum_and_shape(Bgt, K, ratio):
    F = O.fanout(Bgt, K, ratio, 10 ** 6)
    assert sum(F) == Bgt and len(F) == K + 1
    assert all(F[k] >= F[k + 1] for k in range(K))
    ideal = [Bgt * ratio ** k / sum(ratio ** i for i in range(K + 1)) for k in range(K + 1)]
    assert all(abs(F[k] - ideal[k]) < 1 for k in range(K + 1))


def _compositions(n, parts):
    for cut in itertools.combinations(range(n + parts - 1), parts - 1):
        prev = -1
        out = []
        for c in cut + (n + parts - 1,):
            out.append(c - prev - 1)
            prev = c
        yield out


@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.6, 0.95, 1.0])
@pytest.mark.parametrize("K", [0, 1, 3, 6])
def test_depth_probs_by_enumeration(alpha, K):
    """P(k* = k) for K positions accepted independently with probability
    alpha: every accept/reject pattern enumerated with its probability, k* the
    position of the first rejection (K if none); the mean is also the closed
    form E[k*] = alpha + alpha^2 + ... + alpha^K."""
    want = [0.0] * (K + 1)
    for pat in itertools.product([True, False], repeat=K):
        pr = 1.0
        for acc in pat:
            pr *= alpha if acc else 1.0 - alpha
        ks = pat.index(False) if False in pat else K
        want[ks] += pr
    got = O.depth_probs(alpha, K)
    assert len(got) == K + 1
    assert all(abs(g - w) < 1e-12 for g, w in zip(got, want))
    assert abs(sum(got) - 1.0) < 1e-12
    assert abs(sum(k * g for k, g in enumerate(got)) - sum(alpha ** k for k in range(1, K + 1))) < 1e-12


def test_depth_probs_match_the_oracles_verification():
    """depth_probs against the accepted lengths the oracle's verification
    produces: identical target and draft rows at every position with a fixed
    per-position acceptance rate alpha = sum_x min(p, sigma); chi-square over
    seeds (the verification's own Philox draws)."""
    V, K, T, F, C = 5, 3, 1.0, 1, 0.4
    zt = np.array([0.3, -0.2, 1.1, 0.0, -1.0])
    zd = np.array([0.9, -0.5, 0.2, 0.4, -0.3])
    p = O.softmax_t(zt, T)["p"]
    s = O.sigma(zd, T, F, C)["sigma"]
    alpha = O.acceptance_rate(p, s)
    ZT = np.tile(zt, (1, K + 1, 1))
    ZD = np.tile(zd, (1, K + 1, 1))
    n = 3000
    counts = np.zeros(K + 1)
    for seed in range(n):
        tok = O.draft_sample(ZD, [T], F, C, seed)["tokens"]
        counts[O.verify(ZT, ZD, [T], F, C, seed, tok)["accept_len"][0]] += 1
    e = n * np.array(O.depth_probs(alpha, K))
    chi2 = float(np.sum((counts - e) ** 2 / e))
    assert chi2 < 16.27, (chi2, counts, e)  # chi-square, 3 degrees of freedom, p = 0.001


@pytest.mark.parametrize("alpha,r", [(0.6, 1.0), (0.8, 0.5), (0.3, 2.0), (0.9, 1.5)])
@pytest.mark.parametrize("Bgt,K", [(6, 2), (10, 3), (12, 3)])
def test_greedy_fanout_is_optimal_by_brute_force(alpha, r, Bgt, K):
    a = O.depth_probs(alpha, K)
    best = max(O.fanout_objective(a, r, F) for F in _compositions(Bgt, K + 1))
    g = O.optimal_fanout(a, r, Bgt)
    assert sum(g) == Bgt
    assert abs(O.fanout_objective(a, r, g) - best) < 1e-12


@pytest.mark.parametrize("alpha,r,Bgt,K", [(0.6, 1.0, 64, 5), (0.8, 0.5, 40, 7), (0.5, 2.0, 30, 6)])
def test_optimal_fanout_is_truncated_geometric(alpha, r, Bgt, K):
    """Continuous optimum (Lagrange): 1 + F_k = (a_k r / lam)^(1/(1+r)),
    truncated at F_k = 0 -- geometric in k with ratio alpha^(1/(1+r)) for
    k < K.  The integer optimum stays within one unit of it."""
    a = O.depth_probs(alpha, K)

    def total(lam):
        return sum(max(0.0, (ak * r / lam) ** (1 / (1 + r)) - 1) for ak in a)

    lo, hi = 1e-12, 1e3
    for _ in range(200):
        mid = (lo * hi) ** 0.5
        if total(mid) > Bgt:
            lo = mid
        else:
            hi = mid
    cont = [max(0.0, (ak * r / lo) ** (1 / (1 + r)) - 1) for ak in a]
    g = O.optimal_fanout(a, r, Bgt)
    assert all(abs(g[k] - cont[k]) <= 1.0 + 1e-9 for k in range(K + 1))
    beta = alpha ** (1 / (1 + r))
    act = [k for k in range(K) if cont[k] > 0 and k + 1 < K and cont[k + 1] > 0]
    for k in act:
        assert abs((1 + cont[k + 1]) / (1 + cont[k]) - beta) < 1e-9


def test_cache_lookup_brute_force():
    rng = np.random.default_rng(21)
    B, K, V = 40, 5, 50
    Fk = O.fanout(64, K, 0.6, V)
    topf = np.stack([np.stack([rng.permutation(V)[:max(Fk)] for _ in range(K + 1)]) for _ in range(B)])
    keys, off = O.build_keys(topf, Fk)
    payload = rng.integers(0, V, size=(B, off[-1], K))
    kst = rng.integers(0, K + 1, size=B)
    kst[0] = K + 1  # invalid accepted length: a miss
    bonus = rng.integers(0, V, size=B)
    for b in range(0, B, 3):  # force some hits
        if 0 <= kst[b] <= K and Fk[kst[b]] > 0:
            bonus[b] = topf[b, kst[b], rng.integers(0, Fk[kst[b]])]
    hit, slot, toks = O.cache_lookup(keys, off, payload, kst, bonus)
    for b in range(B):
        table = {}
        if 0 <= kst[b] <= K:
            for i in range(Fk[kst[b]]):
                table.setdefault(int(topf[b, kst[b], i]), off[kst[b]] + i)
        s = table.get(int(bonus[b]), -1)
        assert hit[b] == (s >= 0) and slot[b] == s
        if s >= 0:
            assert list(toks[b]) == list(payload[b, s])
        else:
            assert np.all(toks[b] == -1)
    assert hit.sum() > 5


def _concave_curves(rng, K1, Fmax):
    inc = np.sort(rng.uniform(0.0, 1.0, (K1, Fmax)), axis=1)[:, ::-1]
    h = np.concatenate([np.zeros((K1, 1)), np.cumsum(inc, axis=1)], axis=1)
    return h / h[:, -1:] * rng.uniform(0.3, 1.0, (K1, 1))


@pytest.mark.parametrize("seed", range(6))
def test_fanout_from_stats_is_optimal_on_concave_curves(seed):
    # brute force over every allocation of the budget
    rng = np.random.default_rng(seed)
    K1, Fmax = int(rng.integers(2, 4)), 6
    a = rng.dirichlet(np.ones(K1))
    h = _concave_curves(rng, K1, Fmax)
    for Bgt in range(0, K1 * Fmax + 1, 2):
        F = O.fanout_from_stats(a, h, Bgt)
        assert sum(F) == Bgt and max(F) <= Fmax
        best = max(O.fanout_stats_objective(a, h, c)
                   for c in itertools.product(range(Fmax + 1), repeat=K1) if sum(c) == Bgt)
        assert O.fanout_stats_objective(a, h, F) >= best - 1e-12


def test_fanout_from_stats_matches_the_parametric_model():
    # measured curves equal to the model h(F) = 1 - (1+F)^-r give the model's allocation
    r, Fmax = 0.7, 64
    for alpha, K, Bgt in ((0.6, 5, 64), (0.8, 7, 100), (0.4, 3, 20)):
        a = O.depth_probs(alpha, K)
        h = [[1 - (1 + F) ** -r for F in range(Fmax + 1)] for _ in range(K + 1)]
        assert O.fanout_from_stats(a, h, Bgt) == O.optimal_fanout(a, r, Bgt)


def test_fanout_from_stats_ties_and_caps():
    h = [[0.0, 0.5, 0.75], [0.0, 0.5, 0.75]]
    assert O.fanout_from_stats([0.5, 0.5], h, 1) == [1, 0]   # tie: smaller depth
    assert O.fanout_from_stats([0.9, 0.1], h, 3) == [2, 1]   # depth 0 capped at Fmax
    with pytest.raises(ValueError):
        O.fanout_from_stats([0.5, 0.5], h, 5)
