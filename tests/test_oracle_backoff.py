"""Pins of the cache-miss fallback (random stand-in tokens) and of the
back-off rule that chooses between an accurate and a fast backup speculator."""
import math

import numpy as np
import pytest

from oracle import philox as ph
from oracle import ssd as O


def test_token_from_word_is_the_exact_integer_quotient():
    # floor(w V / 2^32) against exact integer arithmetic: t 2^32 <= w V < (t+1) 2^32
    rng = np.random.default_rng(3)
    for V in (1, 2, 3, 7, 1000, 128256, 151936, 262144):
        w = rng.integers(0, 2 ** 32, 2000, dtype=np.uint64)
        w = np.concatenate([w, np.array([0, 1, 2 ** 32 - 1, 2 ** 31], dtype=np.uint64)])
        t = ph.token_from_word(w, V)
        for wi, ti in zip(w.tolist(), t.tolist()):
            assert 0 <= ti < V
            assert ti * 2 ** 32 <= wi * V < (ti + 1) * 2 ** 32


def test_token_from_word_power_of_two_takes_the_top_bits():
    w = np.random.default_rng(4).integers(0, 2 ** 32, 500, dtype=np.uint64)
    for k in (1, 5, 17):
        assert np.array_equal(ph.token_from_word(w, 2 ** k), (w >> np.uint64(32 - k)).astype(np.int64))


def test_fallback_tokens_follow_the_stream_layout():
    # token i of sequence b: word (i & 3) of Philox at counter (i >> 2, b, 0, FALLBACK)
    seed, b, K, V = (5 << 32) | 9, 3, 7, 1000
    got = O.fallback_tokens(seed, b, K, V)
    for i in range(K):
        words = ph.philox4x32_10((i >> 2, b, 0, ph.FALLBACK), (9, 5))
        assert got[i] == (int(words[i & 3]) * V) >> 32
    assert O.fallback_tokens(seed, b, 0, V).size == 0


def test_fallback_tokens_are_uniform():
    # chi-square over 200 sequences x 50 tokens at V = 7 (99.9% bound, 6 dof)
    V = 7
    toks = np.concatenate([O.fallback_tokens(123, b, 50, V) for b in range(200)])
    cnt = np.bincount(toks, minlength=V)
    e = toks.size / V
    chi2 = float(((cnt - e) ** 2 / e).sum())
    assert chi2 < 22.46


def test_lookup_fill_only_touches_misses():
    rng = np.random.default_rng(5)
    B, K, V = 40, 4, 50
    Fk = [6, 4, 2, 1, 1]
    off = O.depth_offsets(Fk)
    keys = rng.integers(0, V, (B, off[-1]))
    payload = rng.integers(0, V, (B, off[-1], K))
    acc = rng.integers(-1, K + 2, B)
    bonus = rng.integers(0, V, B)
    h0, s0, t0 = O.cache_lookup(keys, off, payload, acc, bonus)
    h1, s1, t1 = O.cache_lookup(keys, off, payload, acc, bonus, seed=77, V=V, miss_fill=True)
    assert np.array_equal(h0, h1) and np.array_equal(s0, s1)
    assert 0 < h0.sum() < B
    for b in range(B):
        if h0[b]:
            assert np.array_equal(t1[b], t0[b])
        else:
            assert np.all(t0[b] == -1) and np.array_equal(t1[b], O.fallback_tokens(77, b, K, V))


COSTS = [dict(t_round=1.0, t_slow=2.0, t_fast=0.05, e_acc=3.0, e_fast=1.0),
         dict(t_round=1.0, t_slow=0.5, t_fast=0.0, e_acc=2.5, e_fast=1.1),
         dict(t_round=2.0, t_slow=3.0, t_fast=0.1, e_acc=4.0, e_fast=1.0)]


@pytest.mark.parametrize("c", COSTS)
def test_backoff_all_hits_keeps_the_accurate_backup(c):
    # no sequence can miss: both rates are B e_acc / t_round, a tie
    use, gain = O.backoff(np.ones(64), **c)
    assert gain == 1.0 and not use


@pytest.mark.parametrize("c", COSTS)
@pytest.mark.parametrize("p", [0.6, 0.9, 0.97, 0.995])
def test_backoff_switches_once_at_the_critical_batch(c, p):
    # uniform hit chance: the rate ratio grows with B, so the choice flips at
    # most once, at the closed-form B* = ln(1 - q*) / ln p
    Bs = np.arange(1, 2001)
    use = np.array([O.backoff(np.full(B, p), **c)[0] for B in Bs])
    assert np.all(np.diff(use.astype(int)) >= 0)
    Bc = O.backoff_critical_batch(p, **c)
    if math.isinf(Bc):
        assert not use.any()
    else:
        first = int(Bs[use][0]) if use.any() else None
        assert first is not None and first - 1 <= Bc <= first, (Bc, first)


def test_backoff_equal_quality_prefers_the_faster_backup():
    # a fast backup as good as the accurate one wins whenever a miss can occur
    c = dict(t_round=1.0, t_slow=1.0, t_fast=0.1, e_acc=2.0, e_fast=2.0)
    for B in (1, 3, 50):
        assert O.backoff(np.full(B, 0.9), **c)[0]
    assert O.backoff_critical_batch(0.9, **c) == 0.0


def test_backoff_equal_latency_keeps_the_accurate_backup():
    # same wait, fewer tokens: the fast backup never wins
    c = dict(t_round=1.0, t_slow=0.3, t_fast=0.3, e_acc=3.0, e_fast=1.0)
    for B in (1, 10, 1000):
        use, gain = O.backoff(np.full(B, 0.8), **c)
        assert not use and gain < 1.0
    assert math.isinf(O.backoff_critical_batch(0.8, **c))
