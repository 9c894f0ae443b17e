"""Pins of the oracle's ActKV retention functions (CPU only): attention mass, the
action-critical set, LRFU values and the order in which a compaction leaves per-entry state.

Each test would fail on a plausible mistake: a mass taken over keys instead of rows or squared,
a critical set built from ranks instead of attention, a wrong tie rule, a threshold off by one
entry, an LRFU decay applied with the wrong sign or exponent, or a side array left in the old
order after the paged slot plan."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.special import softmax

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EX = json.load(open(os.path.join(GOLDEN, "actkv_examples.json")))


def _ln(v):
    return [[math.log(x) for x in row] for row in v]


# ------------------------------------------------------------------- attention mass

@pytest.mark.parametrize("ex", EX["mass_examples"], ids=lambda e: e["name"])
def test_mass_worked_examples(ex):
    Q = np.array(ex["queries"], dtype=np.float64)
    K = np.array(_ln(ex["keys_ln"]), dtype=np.float64)
    lse_rows = None if ex["lse_ln"] is None else np.log(np.array(ex["lse_ln"], dtype=np.float64))
    got = O.attention_mass(Q, K, 1.0, lse_rows=lse_rows)
    np.testing.assert_allclose(got, [float(Fraction(x)) for x in ex["mass"]], rtol=1e-14)


def test_mass_example_b_by_hand():
    a1 = [Fraction(1, 6), Fraction(2, 6), Fraction(3, 6)]
    a2 = [Fraction(6, 11), Fraction(3, 11), Fraction(2, 11)]
    assert [(x + y) / 2 for x, y in zip(a1, a2)] == [Fraction(47, 132), Fraction(40, 132), Fraction(45, 132)]


def test_mass_single_row_is_softmax_and_sums_to_one():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((50, 8))
    q = rng.standard_normal((1, 8))
    b = rng.standard_normal(50) * 0.3
    np.testing.assert_allclose(O.attention_mass(q, K, 0.7, bias=b), softmax(0.7 * (q @ K.T)[0] + b), rtol=1e-12)
    Q = rng.standard_normal((9, 8))
    assert abs(O.attention_mass(Q, K, 0.5, bias=b).sum() - 1.0) < 1e-12


def test_mass_is_mean_and_score_is_rms_of_the_same_weights():
    # s_j (root mean square over rows) >= mass_j (mean), equal only when every row agrees
    rng = np.random.default_rng(6)
    Q, K = rng.standard_normal((12, 16)), rng.standard_normal((40, 16))
    m, s = O.attention_mass(Q, K, 0.3), O.te_scores(Q, K, 0.3)
    assert np.all(s >= m * (1 - 1e-12))
    Qs = np.repeat(Q[:1], 5, axis=0)
    np.testing.assert_allclose(O.te_scores(Qs, K, 0.3), O.attention_mass(Qs, K, 0.3), rtol=1e-12)


def test_mass_brute_force_loops():
    rng = np.random.default_rng(7)
    Q, K = rng.standard_normal((3, 4)), rng.standard_normal((5, 4))
    want = []
    for j in range(5):
        tot = 0.0
        for r in range(3):
            z = sum(math.exp(0.9 * float(Q[r] @ K[jj])) for jj in range(5))
            tot += math.exp(0.9 * float(Q[r] @ K[j])) / z
        want.append(tot / 3)
    np.testing.assert_allclose(O.attention_mass(Q, K, 0.9), want, rtol=1e-12)


# ------------------------------------------------------------------- action-critical set

@pytest.mark.parametrize("ex", EX["critical_examples"], ids=lambda e: e["name"])
def test_critical_worked_examples(ex):
    hit = O.action_critical(np.array(ex["mass"], dtype=np.float32), ex["top_p"])
    assert np.flatnonzero(hit).tolist() == ex["critical"]


def test_quantised_mass_exact():
    assert O.quantised_mass(np.array([0.5, 0.25, 0.0, 1.0], np.float32)) == [2 ** 31, 2 ** 30, 0, 2 ** 32]
    assert O.quantised_mass(np.array([2.0 ** -33, 3.0 * 2 ** -32], np.float32)) == [0, 3]
    assert O.quantised_mass(np.array([1000.0], np.float32)) == [2 ** 40]


@settings(max_examples=200, deadline=None)
@given(st.lists(st.sampled_from([0.0, 0.01, 0.05, 0.1, 0.125, 0.2, 0.25, 0.3]), min_size=1, max_size=9),
       st.sampled_from([0.1, 0.5, 0.75, 0.9, 0.95, 1.0]))
def test_critical_is_the_shortest_sufficient_top_k(masses, top_p):
    """The set equals select_topm(mass, k) for the smallest k whose top-k holds the target,
    found here by trying every k (a different route than the ordered walk)."""
    v = np.array(masses, dtype=np.float32)
    u = O.quantised_mass(v)
    total = sum(u)
    hit = O.action_critical(v, top_p)
    if total == 0:
        assert not hit.any()
        return
    target = math.ceil(top_p * total)
    for k in range(len(v) + 1):
        top = O.select_topm(v.astype(np.float64), k)
        if sum(u[j] for j in top) >= target:
            assert np.flatnonzero(hit).tolist() == top.tolist()
            break
    else:
        raise AssertionError("unreachable: the whole set holds the total")


# ------------------------------------------------------------------- LRFU

@pytest.mark.parametrize("ex", EX["lrfu_examples"], ids=lambda e: e["name"])
def test_lrfu_worked_examples(ex):
    assert abs(O.lrfu_crf(ex["hits"], ex["now"], ex["lam"]) - float(Fraction(ex["crf"]))) < 1e-15


@settings(max_examples=100, deadline=None)
@given(st.lists(st.booleans(), min_size=1, max_size=20), st.sampled_from([0.0, 0.5, 1.0, 2.0]))
def test_lrfu_steps_equal_the_crf_definition(hits, lam):
    """Iterating the per-step update from 0 gives LRFU's combined recency-frequency value."""
    state = np.zeros(1)
    for h in hits:
        state = O.lrfu_step(state, np.array([h]), 2.0 ** -lam)
    steps = [t + 1 for t, h in enumerate(hits) if h]
    assert abs(state[0] - O.lrfu_crf(steps, len(hits), lam)) < 1e-12


# ------------------------------------------------------------------- side arrays through compaction

@pytest.mark.parametrize("ex", EX["side_examples"], ids=lambda e: e["name"])
def test_side_order_worked_examples(ex):
    assert O.side_order(ex["n"], ex["m"], ex["B"], ex["kept"]) == ex["order"]


@settings(max_examples=150, deadline=None)
@given(st.integers(1, 40), st.sampled_from([1, 2, 4, 16]), st.data())
def test_side_order_follows_the_paged_copy(n, B, data):
    """Tag every slot of a one-head pool with its position, apply the plan's copies, read the
    window: the tags found there are the side order (a route through apply_paged_copy)."""
    m = data.draw(st.integers(0, n))
    kept = sorted(data.draw(st.permutations(range(n)))[:m])
    N = -(-n // B)
    table = np.arange(N + 1, dtype=np.int32)
    kp = np.full((N + 1, B, 1, 1), -1, dtype=np.int64)
    for p in range(n):
        kp[p // B, p % B, 0, 0] = p
    vp = kp.copy()
    plan = O.paged_plan(n, m, B, kept)
    O.apply_paged_copy(kp, vp, table, 0, plan)
    found = [int(kp[w // B, w % B, 0, 0]) for w in range(plan.start, plan.start + m)]
    assert found == O.side_order(n, m, B, kept)
    assert sorted(found) == kept


# ------------------------------------------------------------------------- causal proxy rows

def test_causal_hand_worked_example():
    """Keys (0, ln 2, ln 3), d = 1, scale 1, three rows q = 1 at positions 0, 1, 2: the rows'
    weights are (1, 0, 0), (1/3, 2/3, 0), (1/6, 1/3, 1/2), so the squared scores are 41/108,
    20/108, 9/108 and the masses 1/2, 1/3, 1/6."""
    K = np.array([[0.0], [math.log(2.0)], [math.log(3.0)]])
    Q = np.ones((3, 1))
    pos = [0, 1, 2]
    s, L = O.causal_weights(Q, K, 1.0, pos)
    np.testing.assert_allclose(s ** 2, np.array([41, 20, 9]) / 108.0, rtol=1e-14)
    np.testing.assert_allclose(L, [0.0, math.log(3.0), math.log(6.0)], rtol=1e-14, atol=1e-15)
    mass, _ = O.causal_weights(Q, K, 1.0, pos, power=1)
    np.testing.assert_allclose(mass, [1 / 2, 1 / 3, 1 / 6], rtol=1e-14)


def _causal_problem(seed, R=9, n=17, d=5):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((R, d)), rng.standard_normal((n, d)), rng.integers(-2, n + 2, R), rng


@pytest.mark.parametrize("seed", range(5))
def test_causal_rows_are_softmax_over_their_prefix(seed):
    """Brute force: each row's weights are scipy's softmax over the keys up to its position."""
    Q, K, pos, rng = _causal_problem(seed)
    bias = rng.standard_normal(K.shape[0])
    R, n = Q.shape[0], K.shape[0]
    for power in (1, 2):
        got, _ = O.causal_weights(Q, K, 0.7, pos, bias=bias, power=power)
        acc = np.zeros(n)
        for r in range(R):
            p = min(int(pos[r]), n - 1)
            if p < 0:
                continue
            w = softmax(0.7 * (K[:p + 1] @ Q[r]) + bias[:p + 1])
            acc[:p + 1] += w ** power
        want = np.sqrt(acc / R) if power == 2 else acc / R
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-300)


def test_causal_mask_that_hides_nothing_is_the_plain_score():
    Q, K, _, _ = _causal_problem(7)
    n = K.shape[0]
    pos = np.full(Q.shape[0], n - 1)
    s, L = O.causal_weights(Q, K, 0.3, pos)
    np.testing.assert_allclose(s, O.te_scores(Q, K, 0.3), rtol=1e-13)
    np.testing.assert_allclose(L, O.lse(Q, K, 0.3), rtol=1e-13)
    mass, _ = O.causal_weights(Q, K, 0.3, pos + 5, power=1)
    np.testing.assert_allclose(mass, O.attention_mass(Q, K, 0.3), rtol=1e-13)


def test_a_row_that_sees_nothing_only_dilutes_the_mean():
    """A row at position -1 sees no key: it adds nothing, but it counts in R."""
    Q, K, pos, _ = _causal_problem(8)
    pos = np.clip(pos, 0, None)
    s, _ = O.causal_weights(Q, K, 0.5, pos)
    Q2 = np.vstack([Q, np.ones((1, Q.shape[1]))])
    s2, L2 = O.causal_weights(Q2, K, 0.5, np.concatenate([pos, [-1]]))
    np.testing.assert_allclose(s2 ** 2, s ** 2 * Q.shape[0] / (Q.shape[0] + 1), rtol=1e-13)
    assert L2[-1] == -np.inf


def test_causal_supplied_lse_is_used_as_given():
    """A supplied LSE larger by ln 2 halves every weight (quarters the squares)."""
    Q, K, pos, _ = _causal_problem(9)
    pos = np.clip(pos, 0, None)
    s, L = O.causal_weights(Q, K, 0.5, pos)
    s2, _ = O.causal_weights(Q, K, 0.5, pos, lse_rows=L + math.log(2.0))
    np.testing.assert_allclose(s2, s / 2.0, rtol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_causal_through_a_live_mask_is_brute_force_with_dead_logits(seed):
    """Dead positions take no part: the same as giving them logit -inf by brute force (each row
    a softmax over its visible live keys), and a dead position scores exactly 0."""
    Q, K, pos, rng = _causal_problem(20 + seed, R=11, n=23)
    Q, K = Q.astype(np.float32).astype(np.float64), K.astype(np.float32).astype(np.float64)  # stored as f32
    n = K.shape[0]
    live = rng.random(n) >= 0.4
    live[0] = True  # every row that sees a key sees a live one (position >= 0 includes key 0)
    bias = rng.standard_normal(n)
    for power in (1, 2):
        got, L = O.causal_unit_live(Q, K, live, pos, "f32", 0.6, bias=bias, power=power)
        acc = np.zeros(n)
        for r in range(Q.shape[0]):
            p = min(int(pos[r]), n - 1)
            if p < 0:
                assert L[r] == -np.inf
                continue
            x = np.where(live[:p + 1], 0.6 * (K[:p + 1] @ Q[r]) + bias[:p + 1], -np.inf)
            acc[:p + 1] += softmax(x) ** power
            np.testing.assert_allclose(L[r], np.log(np.exp(x - x.max()).sum()) + x.max(), rtol=1e-13)
        want = np.sqrt(acc / Q.shape[0]) if power == 2 else acc / Q.shape[0]
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-300)
        assert np.all(got[~live] == 0.0)
