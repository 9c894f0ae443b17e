"""Pins of the oracle's Attention Matching fit (CPU only).

Each test would fail on a plausible mistake: a wrong sign or scale in the exponentials, a
different objective than the page's (e.g. a row-normalised one), a multiplicative update that
is not a descent step, a Landweber step that diverges, or V_C fitted to the wrong target."""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.optimize import nnls
from scipy.special import softmax

from oracle import oracle as O


def _problem(seed, R=12, n=24, d=6, every=3, scale=0.6):
    rng = np.random.default_rng(seed)
    Q, K, V = rng.standard_normal((R, d)), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    kept = np.arange(0, n, every)
    z, Y, M, L = O.am_targets(Q, K, V, scale)
    return Q, K, V, kept, z, Y, M, L, O.am_design(Q, K[kept], scale, M)


def test_targets_are_the_page_quantities():
    Q, K, V, kept, z, Y, M, L, E = _problem(1)
    S = 0.6 * (Q @ K.T)
    np.testing.assert_allclose(z * math.exp(M), np.exp(S).sum(axis=1), rtol=1e-12)
    np.testing.assert_allclose(Y, softmax(S, axis=1) @ V, rtol=1e-12)
    np.testing.assert_allclose(E * math.exp(M), np.exp(S[:, kept]), rtol=1e-12)


def test_scaled_objective_has_the_page_minimiser():
    """|| exp(c Q K_C^T + beta) 1 - exp(c Q K^T) 1 ||^2 = e^{2M} || E w - z ||^2 for every w."""
    Q, K, V, kept, z, Y, M, L, E = _problem(2)
    S = 0.6 * (Q @ K.T)
    for w in (np.ones(len(kept)), np.linspace(0.5, 3.0, len(kept))):
        page = np.sum((np.exp(S[:, kept] + np.log(w)[None, :]).sum(axis=1) - np.exp(S).sum(axis=1)) ** 2)
        assert abs(page - math.exp(2 * M) * np.sum((E @ w - z) ** 2)) <= 1e-9 * page


def test_multiplicative_updates_reach_the_nnls_optimum():
    Q, K, V, kept, z, Y, M, L, E = _problem(3)
    w_opt, r_opt = nnls(E, z)
    w = O.am_fit_beta(E, z, 20000)
    assert np.linalg.norm(E @ w - z) <= r_opt * (1 + 1e-3) + 1e-12
    assert np.all(w >= 0)


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 2 ** 31 - 1))
def test_multiplicative_updates_never_increase_the_objective(seed):
    Q, K, V, kept, z, Y, M, L, E = _problem(seed, R=8, n=15, every=2)
    prev = np.linalg.norm(E @ np.ones(E.shape[1]) - z)
    for it in range(1, 25):
        cur = np.linalg.norm(E @ O.am_fit_beta(E, z, it) - z)
        assert cur <= prev * (1 + 1e-12) + 1e-15
        prev = cur


def test_duplicated_keys_give_beta_ln2_in_one_step():
    """Every key appears twice and the first copies are kept: w = 2 matches exactly and the first
    multiplicative step lands on it, so beta = ln 2."""
    rng = np.random.default_rng(4)
    Q, K1 = rng.standard_normal((7, 5)), rng.standard_normal((6, 5))
    K = np.repeat(K1, 2, axis=0)
    z, Y, M, L = O.am_targets(Q, K, np.zeros((12, 5)), 0.8)
    E = O.am_design(Q, K[::2], 0.8, M)
    np.testing.assert_allclose(O.am_fit_beta(E, z, 1), 2.0, rtol=1e-12)


def test_keeping_every_key_changes_nothing():
    Q, K, V, kept, z, Y, M, L, E0 = _problem(5)
    allk = np.arange(K.shape[0])
    E = O.am_design(Q, K, 0.6, M)
    w = O.am_fit_beta(E, z, 30)
    np.testing.assert_allclose(w, 1.0, rtol=1e-12)
    np.testing.assert_allclose(O.am_fit_values(E, w, Y, V, 30), V, rtol=1e-10, atol=1e-12)
    beta, Vc = O.am_unit(Q.astype(np.float32), K.astype(np.float32), V.astype(np.float32), allk, "f32", 0.6, 5, 5)
    np.testing.assert_allclose(beta, 0.0, atol=1e-12)


def test_landweber_reaches_least_squares():
    """On a well-conditioned compacted attention (each row dominated by one kept key) the
    iteration lands on numpy's least-squares solution; its residual never grows on the way."""
    rng = np.random.default_rng(6)
    R, m, d = 30, 10, 4
    E = rng.random((R, m)) * 0.2
    E[np.arange(R), np.arange(R) % m] += 1.0
    w = rng.random(m) + 0.5
    Y = rng.standard_normal((R, d))
    P = E * w[None, :]
    P = P / P.sum(axis=1, keepdims=True)
    Vls, *_ = np.linalg.lstsq(P, Y, rcond=None)
    Vc = O.am_fit_values(E, w, Y, np.zeros((m, d)), 3000)
    np.testing.assert_allclose(Vc, Vls, rtol=1e-8, atol=1e-8)
    prev = np.inf
    for it in (0, 1, 5, 50, 500):
        r = np.linalg.norm(P @ O.am_fit_values(E, w, Y, np.zeros((m, d)), it) - Y)
        assert r <= prev * (1 + 1e-12)
        prev = r


def test_landweber_keeps_an_exact_fit():
    """When the original values already reproduce the target (Y = P V_0) nothing moves."""
    Q, K, V, kept, z, Y, M, L, E = _problem(7)
    w = O.am_fit_beta(E, z, 10)
    Ew = E * w[None, :]
    P = Ew / Ew.sum(axis=1, keepdims=True)
    V0 = V[kept]
    np.testing.assert_allclose(O.am_fit_values(E, w, P @ V0, V0, 50), V0, rtol=1e-12, atol=1e-12)
