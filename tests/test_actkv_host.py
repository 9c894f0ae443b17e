"""Host side of ActKV's retention policy (CPU): the budget ratchet and its confidence monitor."""
import numpy as np
import pytest

from online_compaction_amd.actkv import BudgetRatchet, ls_slope, min_pool, token_confidence


def test_ratchet_budgets_closed_form():
    """512 x 1.75^k floored, capped at 30000; 8403 and 14706 at k = 5, 6 (not 8404 / 14705)."""
    r = BudgetRatchet()
    seen = []
    for k in range(10):
        r.expansions = k
        seen.append(r.budget)
    assert seen == [512, 896, 1568, 2744, 4802, 8403, 14706, 25735, 30000, 30000]


def test_ratchet_only_grows():
    r = BudgetRatchet()
    down = np.linspace(5.0, 1.0, 200)
    up = np.linspace(1.0, 5.0, 200)
    assert r.observe(down) and r.budget == 896
    assert not r.observe(up) and r.budget == 896      # recovery does not shrink it
    assert not r.observe(np.full(200, 2.0)) and r.budget == 896
    assert r.observe(down) and r.budget == 1568
    r.expansions = 8
    assert not r.observe(down) and r.budget == 30000  # capped


def test_min_pool_windows():
    x = np.arange(100.0)
    np.testing.assert_array_equal(min_pool(x, 64, 8), [0, 8, 16, 24, 32])
    assert min_pool(np.arange(63.0)).size == 0
    y = np.full(80, 3.0)
    y[70] = -1.0  # a dip inside the last two windows only
    np.testing.assert_array_equal(min_pool(y, 64, 8), [3.0, -1.0, -1.0])


def test_short_step_makes_no_decision():
    r = BudgetRatchet()
    assert not r.observe(np.linspace(5, 1, 70))  # one pooled point: no slope
    assert r.budget == 512


def test_ls_slope():
    assert ls_slope([3, 2, 1]) == pytest.approx(-1.0)
    assert ls_slope([1, 1, 1, 1]) == 0.0
    assert ls_slope([0, 2, 1, 3]) == pytest.approx(0.8)
    assert ls_slope([7]) == 0.0


def test_token_confidence_is_mean_negative_logprob():
    lp = np.log(np.array([[0.5, 0.25, 0.25], [0.9, 0.05, 0.05]]))
    np.testing.assert_allclose(token_confidence(lp), [-(np.log(0.5) + 2 * np.log(0.25)) / 3,
                                                      -(np.log(0.9) + 2 * np.log(0.05)) / 3])
    # a sure model (one dominant candidate, tiny tail) scores higher than a hesitant one
    sure = np.log(np.r_[0.999, np.full(19, 0.001 / 19)])
    unsure = np.log(np.full(20, 0.05))
    assert token_confidence(sure[None])[0] > token_confidence(unsure[None])[0]
