"""Pins of the oracle's layout-preserving eviction (CPU only): the dead-slot redirect and the
logit-mask reading of the dead slot.

Each test would fail on a plausible mistake: redirecting kept positions (or past n), letting a
dead position stay in the softmax, giving it a nonzero score, or normalising over the wrong keys."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.special import softmax

from oracle import oracle as O

EX = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "sentinel_examples.json")))


@pytest.mark.parametrize("ex", EX["redirect_examples"], ids=lambda e: e["name"])
def test_redirect_worked_examples(ex):
    assert O.evict_redirect(ex["slots"], ex["kept"], ex["n"], ex["dead"]).tolist() == ex["after"]


@pytest.mark.parametrize("ex", EX["masked_score_examples"], ids=lambda e: e["name"])
def test_masked_score_worked_examples(ex):
    Q = np.array(ex["queries"], dtype=np.float32)
    K = np.log(np.array(ex["keys_ln"], dtype=np.float64)).astype(np.float32)
    s = O.score_unit_live(Q, K, ex["live"], "f32", 1.0)
    if "scores" in ex:
        want = [float(Fraction(x)) for x in ex["scores"]]
        np.testing.assert_allclose(s, want, rtol=1e-6, atol=0)  # keys are float32-rounded logs
    else:
        np.testing.assert_allclose(s * s, [float(Fraction(x)) for x in ex["scores_squared"]], rtol=1e-6, atol=0)


def test_literal_constant_key_does_not_mask():
    """The page's constant sentinel key (-1e4) attracts a query with a negative component sum;
    this is why the dead slot is read as a logit mask."""
    ex = EX["constant_key_example"]
    keys = [math.log(x) for x in ex["keys_ln"]] + [ex["sentinel_key"]]
    w = softmax(ex["query"] * np.array(keys))
    assert w[-1] > 0.999
    # the logit-mask reading gives the sentinel nothing and renormalises the live keys
    s = O.score_unit_live(np.array([[ex["query"]]], np.float32), np.array(keys, np.float32)[:, None],
                          [True, True, False], "f32", 1.0)
    assert s[-1] == 0.0 and abs(s[:2].sum() - 1.0) < 1e-6


@settings(max_examples=60, deadline=None)
@given(st.integers(2, 30), st.integers(0, 2 ** 31 - 1))
def test_mask_equals_minus_infinity_bias(n, seed):
    """Scoring with dead positions equals scoring every key with a -inf logit bias on the dead
    ones (the mask taken through the softmax instead of by removing rows)."""
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((5, 8)).astype(np.float32)
    K = rng.standard_normal((n, 8)).astype(np.float32)
    live = rng.random(n) < 0.6
    live[rng.integers(n)] = True
    bias = np.where(live, 0.0, -np.inf)
    with np.errstate(invalid="ignore"):
        ref = O.te_scores(Q.astype(np.float64), K.astype(np.float64), 0.4, bias=bias)
        mref = O.attention_mass(Q.astype(np.float64), K.astype(np.float64), 0.4, bias=bias)
    np.testing.assert_allclose(O.score_unit_live(Q, K, live, "f32", 0.4), ref, rtol=1e-12, atol=1e-300)
    m = O.score_unit_live(Q, K, live, "f32", 0.4, power=1)
    np.testing.assert_allclose(m, mref, rtol=1e-12, atol=1e-300)
    assert abs(m.sum() - 1.0) < 1e-12 and np.all(m[~live] == 0)


def test_slot_keys_follow_the_map():
    pool = np.arange(6 * 2 * 3, dtype=np.int64).reshape(6, 2, 3)
    keys = O.slot_unit_keys(pool, [5, 0, 3], 3, 1)
    assert keys.tolist() == [pool[5, 1].tolist(), pool[0, 1].tolist(), pool[3, 1].tolist()]
