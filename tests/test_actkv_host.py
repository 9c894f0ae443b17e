"""Host side of ActKV's retention policy (CPU): the one-way budget ratchet."""
from online_compaction_amd.actkv import BudgetRatchet


def test_ratchet_budgets_closed_form():
    """512 x 1.75^k floored, capped at 30000; 8403 and 14706 at k = 5, 6 (not 8404 / 14705)."""
    r = BudgetRatchet()
    seen = []
    for k in range(10):
        r.expansions = k
        seen.append(r.budget)
    assert seen == [512, 896, 1568, 2744, 4802, 8403, 14706, 25735, 30000, 30000]


def test_ratchet_only_grows_and_stops_at_the_cap():
    r = BudgetRatchet()
    assert r.expand() and r.budget == 896
    assert r.expand() and r.budget == 1568
    r.expansions = 8
    assert r.budget == 30000
    assert not r.expand() and r.expansions == 8 and r.budget == 30000
