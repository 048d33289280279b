"""Pins of the oracle's Philox4x32-10, uniforms and Gumbel draws."""
import os

import numpy as np
import pytest
from scipy import stats

from oracle import philox as ph

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _kat():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            v = [int(t, 16) for t in line.split()]
            rows.append((v[0:4], v[4:6], v[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat())
def test_known_answer_vectors(ctr, key, expect):
    out = [int(x) for x in ph.philox4x32_10(ctr, key)]
    assert out == expect


def test_stream_layout_uses_word_idx_mod_4():
    # draws idx 4c..4c+3 are the four output words of one call at counter c
    seed = (7 << 32) | 11
    idx = np.arange(8, 12)
    w = ph.draw_words(seed, 3, 5, ph.BONUS_TOKEN, idx)
    ref = ph.philox4x32_10((2, 3, 5, ph.BONUS_TOKEN), (11, 7))
    assert [int(x) for x in w] == [int(x) for x in ref]


def test_uniform_endpoints_and_fp32_exactness():
    w = np.array([0, 1 << 9, 0xFFFFFFFF, 0x80000000], dtype=np.uint64)
    u = ph.uniform_from_word(w)
    assert u[0] == 2.0 ** -24
    assert u[1] == 3 * 2.0 ** -24
    assert u[2] == 1 - 2.0 ** -24
    assert u[3] == 0.5 + 2.0 ** -24
    rng = np.random.default_rng(0)
    ww = rng.integers(0, 2 ** 32, size=100000, dtype=np.uint64)
    uu = ph.uniform_from_word(ww)
    assert np.all(uu.astype(np.float32).astype(np.float64) == uu)
    assert np.all((uu > 0) & (uu < 1))


def test_uniform_and_gumbel_distributions():
    idx = np.arange(200000)
    u = ph.uniforms(12345, 1, 2, ph.DRAFT_TOKEN, idx)
    assert stats.kstest(u, "uniform").pvalue > 1e-4
    g = ph.gumbel_from_uniform(u)
    assert stats.kstest(g, "gumbel_r").pvalue > 1e-4
    # distinct streams / positions give unrelated draws
    u2 = ph.uniforms(12345, 1, 3, ph.DRAFT_TOKEN, idx)
    assert abs(np.corrcoef(u, u2)[0, 1]) < 0.01
