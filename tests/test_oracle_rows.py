"""Pins of decode, softmax_t, topf and sigma_{F,C} (Saguaro sampling)."""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st
from scipy import special

from oracle import ssd as O


def test_decode_matches_torch_conversions():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 16, size=5000, dtype=np.uint16)
    # drop NaN patterns (not valid logits)
    t_bf = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    t_h = torch.from_numpy(bits.view(np.int16)).view(torch.float16).float().numpy()
    ok_b = ~np.isnan(t_bf)
    ok_h = ~np.isnan(t_h)
    assert np.array_equal(O.decode(bits, "bf16")[ok_b], t_bf[ok_b].astype(np.float64))
    assert np.array_equal(O.decode(bits, "f16")[ok_h], t_h[ok_h].astype(np.float64))
    f = rng.standard_normal(100).astype(np.float32)
    assert np.array_equal(O.decode(f, "f32"), f.astype(np.float64))


@pytest.mark.parametrize("T", [0.3, 0.7, 1.0, 1.2, 5.0])
def test_softmax_t_against_scipy(T):
    rng = np.random.default_rng(2)
    z = rng.standard_normal(3001) * 3
    z[[5, 77, 3000]] = -np.inf
    st_ = O.softmax_t(z, T)
    zz = z / T
    assert math.isclose(st_["lse"] + st_["max"] / T, special.logsumexp(zz), rel_tol=1e-13)
    assert np.allclose(st_["p"], special.softmax(zz), rtol=1e-12, atol=0)
    assert st_["max"] == z.max()


def test_softmax_t_greedy_first_argmax():
    z = np.array([1.0, 3.0, -2.0, 3.0, 0.5])
    for T in (0.0, -1.0, float("nan")):
        st_ = O.softmax_t(z, T)
        assert st_["argmax"] == 1 == int(np.argmax(z))
        assert st_["lse"] == 0.0
        assert np.array_equal(st_["p"], np.eye(5)[1])


def _brute_topf(z, F):
    order = sorted(range(len(z)), key=lambda i: (-z[i], i))
    return order[:F]


@pytest.mark.parametrize("seed", range(6))
def test_topf_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(1, 400))
    z = rng.integers(-4, 5, size=V).astype(np.float64)  # many exact ties
    if seed % 2:
        z[rng.integers(0, V, size=3)] = -np.inf
    for F in (1, 2, 4, 8, 27, 64):
        F = min(F, V)
        idx, val = O.topf(z, F)
        assert list(idx) == _brute_topf(z, F)
        assert np.array_equal(val, z[idx])


def test_topf_negative_zero_ties_positive_zero():
    z = np.array([-0.0, 0.0, -1.0, -0.0])
    idx, _ = O.topf(z, 3)
    assert list(idx) == [0, 1, 3]


def _rand_case(rng, V):
    z = rng.standard_normal(V) * 2
    return z


@pytest.mark.parametrize("T", [0.5, 1.0, 1.7])
def test_sigma_special_cases_and_identities(T):
    rng = np.random.default_rng(3)
    z = _rand_case(rng, 500)
    q = special.softmax(z / T)
    for F, C in ((0, 0.3), (4, 1.0)):
        s = O.sigma(z, T, F, C)
        assert np.allclose(s["sigma"], q, rtol=1e-12, atol=0)
    F, C = 5, 0.4
    s = O.sigma(z, T, F, C)
    sg = s["sigma"]
    S = s["S"]
    assert list(S) == _brute_topf(z, F)
    assert math.isclose(sg.sum(), 1.0, rel_tol=1e-13)
    out = np.setdiff1d(np.arange(500), S)
    x, y = S[2], out[7]
    assert math.isclose(sg[x] / sg[y], C * q[x] / q[y], rel_tol=1e-12)
    assert math.isclose(sg[S[0]] / sg[S[1]], q[S[0]] / q[S[1]], rel_tol=1e-12)
    assert math.isclose(sg[out[0]] / sg[out[3]], q[out[0]] / q[out[3]], rel_tol=1e-12)
    lw = (z - z.max()) / T
    lw[S] += math.log(C)
    assert math.isclose(s["lse"], special.logsumexp(lw), rel_tol=1e-13, abs_tol=1e-13)


def test_sigma_greedy_is_onehot():
    z = np.array([0.1, 2.0, 2.0, -1.0])
    s = O.sigma(z, 0.0, 2, 0.5)
    assert np.array_equal(s["sigma"], np.eye(4)[1])
    assert s["lse"] == 0.0


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10 ** 6), F=st.integers(1, 6),
       c1=st.floats(0.05, 1.0), c2=st.floats(0.05, 1.0), T=st.floats(0.3, 2.0))
def test_lower_C_moves_residual_mass_onto_top_set(seed, F, c1, c2, T):
    """Saguaro sampling down-weights the draft's top tokens so that the
    residual max(0, p - sigma) concentrates on them: the residual mass on S
    does not decrease, and the mass off S does not increase, as C falls."""
    lo, hi = min(c1, c2), max(c1, c2)
    rng = np.random.default_rng(seed)
    V = 40
    zt = rng.standard_normal(V) * 2
    zd = zt + rng.standard_normal(V)
    p = O.softmax_t(zt, T)["p"]
    r_lo = np.maximum(0, p - O.sigma(zd, T, F, lo)["sigma"])
    r_hi = np.maximum(0, p - O.sigma(zd, T, F, hi)["sigma"])
    S = O.sigma(zd, T, F, lo)["S"]
    off = np.setdiff1d(np.arange(V), S)
    assert r_lo[S].sum() >= r_hi[S].sum() - 1e-12
    assert r_lo[off].sum() <= r_hi[off].sum() + 1e-12
