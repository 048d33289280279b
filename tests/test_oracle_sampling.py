"""Pins of the two-level Gumbel-max sampler and of draft sampling.

The distribution of the sampler is fixed by the Gumbel-max theorem and the
chain rule (P(block) * P(token | block) = w_x / sum w); the chi-square tests
check the oracle's draws against w / sum(w) computed here directly.
"""
import math

import numpy as np
import pytest
from scipy import stats

from oracle import philox as ph
from oracle import ssd as O


def _chi2_ok(counts, probs, n):
    nz = probs > 0
    assert np.all(counts[~nz] == 0), "a zero-weight token was sampled"
    exp = probs[nz] * n
    return stats.chisquare(counts[nz], exp).pvalue


@pytest.mark.parametrize("blk", [4, 2048])
def test_gsample_distribution_chi_square(blk):
    rng = np.random.default_rng(5)
    V = 13  # ragged: 3 full blocks of 4 and a tail of 1
    w = rng.random(V) ** 2
    w[[2, 9]] = 0.0
    n = 12000
    counts = np.zeros(V)
    for s in range(n):
        x, _ = O.gsample(w, s, 1, 2, ph.DRAFT_TOKEN, ph.DRAFT_BLOCK, blk)
        counts[x] += 1
    assert _chi2_ok(counts, w / w.sum(), n) > 1e-4


def test_gsample_single_support_and_whole_zero_block():
    w = np.zeros(20)
    w[17] = 0.3
    for s in range(50):
        assert O.gsample(w, s, 0, 0, ph.BONUS_TOKEN, ph.BONUS_BLOCK, 4)[0] == 17
    # margins: one candidate block and one candidate token -> infinite gap
    assert O.gsample(w, 0, 0, 0, ph.BONUS_TOKEN, ph.BONUS_BLOCK, 4)[1] == math.inf


def test_gsample_margin_is_the_decision_gap():
    """Raising the runner-up's log-weight by just under the reported margin
    keeps the winner; by just over it, flips the winner."""
    rng = np.random.default_rng(9)
    V = 16
    w = rng.random(V) + 0.1
    seed = 4242
    x, m = O.gsample(w, seed, 0, 1, ph.DRAFT_TOKEN, ph.DRAFT_BLOCK, 2048)
    g = ph.gumbels(seed, 0, 1, ph.DRAFT_TOKEN, np.arange(V))
    sc = np.log(w) + g
    order = np.argsort(-sc)
    assert order[0] == x
    y = order[1]
    w2 = w.copy()
    w2[y] *= math.exp(m * 0.99)
    assert O.gsample(w2, seed, 0, 1, ph.DRAFT_TOKEN, ph.DRAFT_BLOCK, 2048)[0] == x
    w2 = w.copy()
    w2[y] *= math.exp(m * 1.01)
    assert O.gsample(w2, seed, 0, 1, ph.DRAFT_TOKEN, ph.DRAFT_BLOCK, 2048)[0] == y


def test_draft_sample_follows_sigma():
    rng = np.random.default_rng(6)
    V, K, F, C, T = 13, 2, 3, 0.4, 0.8
    zd = rng.standard_normal((1, K + 1, V)) * 1.5
    n = 6000
    counts = np.zeros((K, V))
    for s in range(n):
        out = O.draft_sample(zd, [T], F, C, s, blk=4)
        for j in range(K):
            counts[j, out["tokens"][0, j]] += 1
    for j in range(K):
        sg = O.sigma(zd[0, j], T, F, C)["sigma"]
        assert _chi2_ok(counts[j], sg, n) > 1e-4
    out = O.draft_sample(zd, [T], F, C, 0, F_out=5, blk=4)
    for j in range(K):
        x = out["tokens"][0, j]
        assert out["q"][0, j] == O.sigma(zd[0, j], T, F, C)["sigma"][x]
    assert out["topf_idx"].shape == (1, K + 1, 5)


def test_draft_sample_greedy_rows():
    zd = np.array([[[0.0, 2.0, 2.0, 1.0], [3.0, 0.0, 3.0, -1.0], [0.0, 0.0, 0.0, 5.0]]])
    out = O.draft_sample(zd, [0.0], 2, 0.5, 7)
    assert list(out["tokens"][0]) == [1, 0]
    assert list(out["q"][0]) == [1.0, 1.0]
    assert np.all(out["margin"] == math.inf)
