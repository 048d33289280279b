"""The GPU parity checker must flag every kind of disagreement (checked on the
CPU with oracle outputs standing in for GPU outputs, then perturbed)."""
import copy

import numpy as np
import pytest

from oracle import ssd as O
from parity import Report, compare_draft, compare_verify


def _case():
    rng = np.random.default_rng(3)
    B, K, V = 4, 3, 5000
    zt = rng.standard_normal((B, K + 1, V)) * 2
    zd = zt + rng.standard_normal((B, K + 1, V))
    T = np.array([1.0, 0.7, 0.0, 1.3])
    d = O.draft_sample(zd, T, 3, 0.5, 11, F_out=5)
    v = O.verify(zt, zd, T, 3, 0.5, 11, d["tokens"])
    g_s = dict(tokens=d["tokens"].copy(), q=d["q"].copy(),
               stats=(d["lse"].copy(), d["max"].copy(), d["argmax"].copy()),
               topf_idx=d["topf_idx"].copy(), topf_val=d["topf_val"].copy())
    g_v = dict(accept_len=v["accept_len"].copy(), bonus=v["bonus"].copy(), p=v["p"].copy(),
               stats=(v["lse"].copy(), v["max"].copy(), v["argmax"].copy()))
    return d, v, g_s, g_v, T


def _run(d, v, g_s, g_v, T):
    r = Report()
    compare_draft(r, g_s, d, T)
    compare_verify(r, g_v, v, T)
    return r


def test_identical_outputs_pass():
    d, v, g_s, g_v, T = _case()
    r = _run(d, v, g_s, g_v, T)
    assert r.ok(), r.fails
    assert r.units > 0


@pytest.mark.parametrize("what", ["token", "q", "max", "argmax", "lse", "topf_idx", "topf_val",
                                  "accept_len", "bonus", "p"])
def test_each_perturbation_is_caught(what):
    d, v, g_s, g_v, T = _case()
    g_s, g_v = copy.deepcopy(g_s), copy.deepcopy(g_v)
    if what == "token":
        g_s["tokens"][0, 0] += 1
    elif what == "q":
        g_s["q"][1, 1] *= 1 + 3e-5
    elif what == "max":
        g_s["stats"][1][0, 2] += 1e-3
    elif what == "argmax":
        g_s["stats"][2][3, 0] += 1
    elif what == "lse":
        g_s["stats"][0][1, 1] += 3e-5 * max(1, abs(g_s["stats"][0][1, 1]))
    elif what == "topf_idx":
        g_s["topf_idx"][2, 1, 4] += 1
    elif what == "topf_val":
        g_s["topf_val"][2, 1, 4] += 0.5
    elif what == "accept_len":
        g_v["accept_len"][0] = (g_v["accept_len"][0] + 1) % 4
    elif what == "bonus":
        g_v["bonus"][1] += 1
    elif what == "p":
        g_v["p"][3, 2] = g_v["p"][3, 2] * (1 + 2e-5) + 1e-6
    r = _run(d, v, g_s, g_v, T)
    assert not r.ok(), what
