"""Pins of the acceptance test, accepted prefix and bonus token.

Losslessness (the emitted tokens follow the target distribution, as the SSD
pages state for SSD and plain speculative decoding alike) is checked by exact
enumeration over all draft sequences for V <= 8, K <= 3.  The seeded oracle is
then checked against the exact joint law of (accepted length, bonus) by a
chi-square test over seeds, and the expected acceptance against sum min(p, q).
"""
import itertools
import math

import numpy as np
import pytest
from scipy import stats

from oracle import ssd as O


def _rows(zt, zd, T, F, C):
    K = zt.shape[0] - 1
    p = [O.softmax_t(zt[j], T)["p"] for j in range(K + 1)]
    s = [O.sigma(zd[j], T, F, C)["sigma"] for j in range(K + 1)]
    return p, s


def _emitted(zt, zd, T, F, C):
    """P(emitted token at j = y | position j reached), by enumeration of all
    V^K drafts weighted by prod sigma_j(x_j)."""
    K = zt.shape[0] - 1
    V = zt.shape[1]
    p, s = _rows(zt, zd, T, F, C)
    reach = np.zeros(K + 1)
    emit = np.zeros((K + 1, V))
    acc = np.zeros(K)
    for xs in itertools.product(range(V), repeat=K):
        pr = 1.0
        for j, x in enumerate(xs):
            pr *= s[j][x]
        if pr == 0:
            continue
        cur = pr
        for j in range(K):
            reach[j] += cur
            a = O.accept_prob(p[j], s[j], xs[j])
            acc[j] += cur * a
            emit[j, xs[j]] += cur * a
            emit[j] += cur * (1 - a) * O.residual(p[j], s[j])
            cur *= a
        reach[K] += cur
        emit[K] += cur * p[K]
    return emit / reach[:, None], acc / reach[:K], p, s


CASES = [  # (V, K, T, F, C): the tiny-verify workload's (T, F, C) at V=6, K=2 and variants
    (6, 2, 1.0, 2, 0.5),
    (6, 2, 1.0, 2, 1.0),
    (6, 2, 1.0, 2, 0.1),
    (6, 2, 0.0, 2, 0.5),
    (8, 3, 0.7, 3, 0.3),
    (5, 3, 1.3, 1, 0.6),
]


@pytest.mark.parametrize("V,K,T,F,C", CASES)
def test_losslessness_by_enumeration(V, K, T, F, C):
    rng = np.random.default_rng(V * 100 + K)
    zt = rng.standard_normal((K + 1, V)) * 2
    zd = zt + rng.standard_normal((K + 1, V)) * 0.5
    emit, acc, p, s = _emitted(zt, zd, T, F, C)
    for j in range(K + 1):
        assert np.allclose(emit[j], p[j], rtol=0, atol=1e-12)
    for j in range(K):
        assert math.isclose(acc[j], O.acceptance_rate(p[j], s[j]), abs_tol=1e-12)


def _exact_joint(p, s, K, V):
    """Exact law of (k*, bonus)."""
    alpha = [O.acceptance_rate(p[j], s[j]) for j in range(K)]
    P = np.zeros((K + 1, V))
    reach = 1.0
    for k in range(K):
        P[k] = reach * (1 - alpha[k]) * O.residual(p[k], s[k])
        reach *= alpha[k]
    P[K] = reach * p[K]
    return P, alpha


def test_seeded_verify_matches_exact_joint_law():
    V, K, T, F, C = 6, 2, 1.0, 2, 0.5
    rng = np.random.default_rng(11)
    zt = rng.standard_normal((1, K + 1, V)) * 2
    zd = zt + rng.standard_normal((1, K + 1, V)) * 0.5
    p, s = _rows(zt[0], zd[0], T, F, C)
    P, alpha = _exact_joint(p, s, K, V)
    n = 5000
    counts = np.zeros((K + 1, V))
    ks = []
    for seed in range(n):
        d = O.draft_sample(zd, [T], F, C, seed, blk=4)
        v = O.verify(zt, zd, [T], F, C, seed, d["tokens"], blk=4)
        counts[v["accept_len"][0], v["bonus"][0]] += 1
        ks.append(v["accept_len"][0])
    m = P.ravel() > 0
    assert np.all(counts.ravel()[~m] == 0)
    assert stats.chisquare(counts.ravel()[m], P.ravel()[m] * n).pvalue > 1e-4
    # E[k*] = sum_{k=1..K} prod_{i<k} alpha_i
    ek = sum(math.prod(alpha[:k]) for k in range(1, K + 1))
    sd = np.std(ks) / math.sqrt(n)
    assert abs(np.mean(ks) - ek) < 4 * sd


def test_identical_distributions_accept_everything():
    rng = np.random.default_rng(12)
    B, K, V = 3, 4, 9
    z = rng.standard_normal((B, K + 1, V))
    for seed in range(30):
        d = O.draft_sample(z, [1.0] * B, 3, 1.0, seed, blk=4)
        v = O.verify(z, z, [1.0] * B, 3, 1.0, seed, d["tokens"], blk=4)
        assert np.all(v["accept_len"] == K)


def test_disjoint_supports_reject_at_first_position():
    V, K = 6, 2
    zt = np.zeros((1, K + 1, V))
    zd = np.zeros((1, K + 1, V))
    zt[..., :3] = -np.inf
    zd[..., 3:] = -np.inf
    for seed in range(30):
        d = O.draft_sample(zd, [1.0], 1, 0.5, seed, blk=4)
        assert np.all(d["tokens"] < 3)
        v = O.verify(zt, zd, [1.0], 1, 0.5, seed, d["tokens"], blk=4)
        assert v["accept_len"][0] == 0
        assert v["bonus"][0] >= 3
        assert v["p"][0, 0] == 0.0


def test_greedy_verify():
    zt = np.array([[[0, 5, 1, 5], [2, 0, 0, 1], [0, 0, 9, 0]]], dtype=float)
    zd = np.array([[[0, 6, 1, 0], [3, 0, 0, 1], [0, 0, 0, 0]]], dtype=float)
    d = O.draft_sample(zd, [0.0], 2, 0.5, 0)
    assert list(d["tokens"][0]) == [1, 0]
    v = O.verify(zt, zd, [0.0], 2, 0.5, 0, d["tokens"])
    assert v["accept_len"][0] == 2 and v["bonus"][0] == 2
    v = O.verify(zt, zd, [0.0], 2, 0.5, 0, np.array([[3, 0]]))
    assert v["accept_len"][0] == 0 and v["bonus"][0] == 1
    assert list(v["p"][0]) == [0.0, 1.0]


def test_k_zero_bonus_follows_target():
    rng = np.random.default_rng(13)
    V = 7
    zt = rng.standard_normal((1, 1, V))
    p = O.softmax_t(zt[0, 0], 0.9)["p"]
    n = 6000
    counts = np.zeros(V)
    for seed in range(n):
        v = O.verify(zt, zt, [0.9], 2, 0.5, seed, np.zeros((1, 0), np.int64), blk=4)
        assert v["accept_len"][0] == 0
        counts[v["bonus"][0]] += 1
    assert stats.chisquare(counts, p * n).pvalue > 1e-4


def test_out_of_range_tokens_are_rejected():
    rng = np.random.default_rng(14)
    zt = rng.standard_normal((2, 3, 5))
    for toks in ([[5, 0]], [[-1, 0]]):
        v = O.verify(zt[:1], zt[:1], [1.0], 1, 0.5, 3, np.array(toks))
        assert v["accept_len"][0] == 0 and v["p"][0, 0] == 0.0
