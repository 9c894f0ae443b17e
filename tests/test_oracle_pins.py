"""Pins of the float64 oracle to facts the pages and mathematics fix (CPU only).

Each test would fail on a plausible mistake in the oracle: a dropped square or square root, a
mean over keys instead of rows, a sign error in the LSE, a transposed product, a wrong tie rule,
a mis-paired or conflicting slot plan, or a wrong freed-block count.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.special import logsumexp, softmax

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _ln(v):
    return [[math.log(x) for x in row] for row in v]


# ------------------------------------------------------------------- worked examples (golden)

@pytest.mark.parametrize("ex", _load("te_examples.json")["examples"], ids=lambda e: e["name"])
def test_worked_examples(ex):
    Q = np.array(ex["queries"], dtype=np.float64)
    K = np.array(_ln(ex["keys_ln"]), dtype=np.float64)
    lse_rows = None if ex["lse_ln"] is None else np.log(np.array(ex["lse_ln"], dtype=np.float64))
    s = O.te_scores(Q, K, 1.0, lse_rows=lse_rows)
    if "scores" in ex:
        want = np.array([float(Fraction(x)) for x in ex["scores"]])
    else:
        want = np.sqrt(np.array([float(Fraction(x)) for x in ex["scores_squared"]]))
        np.testing.assert_allclose(s, ex["scores_decimal"], rtol=1e-14)
    np.testing.assert_allclose(s, want, rtol=1e-14)
    for m, kept in ex["topm"].items():
        assert O.select_topm(s, int(m)).tolist() == kept


def test_example_b_fractions_by_hand():
    # the two rows' weights, written out: (1,2,3)/6 and (6,3,2)/11
    a1 = [Fraction(1, 6), Fraction(2, 6), Fraction(3, 6)]
    a2 = [Fraction(6, 11), Fraction(3, 11), Fraction(2, 11)]
    s2 = [(x * x + y * y) / 2 for x, y in zip(a1, a2)]
    assert s2 == [Fraction(1417, 8712), Fraction(101, 1089), Fraction(137, 968)]


# ------------------------------------------------------------------- special cases / closed forms

def test_single_query_equals_softmax_row():
    rng = np.random.default_rng(0)
    Q = rng.standard_normal((1, 16))
    K = rng.standard_normal((50, 16))
    c = 0.3
    s = O.te_scores(Q, K, c)
    np.testing.assert_allclose(s, softmax(c * (K @ Q[0])), rtol=1e-12)


def test_single_query_with_bias_equals_softmax_row():
    rng = np.random.default_rng(1)
    Q = rng.standard_normal((1, 8))
    K = rng.standard_normal((30, 8))
    b = rng.standard_normal(30)
    s = O.te_scores(Q, K, 0.5, bias=b)
    np.testing.assert_allclose(s, softmax(0.5 * (K @ Q[0]) + b), rtol=1e-12)


def test_equal_logits_give_one_over_n():
    K = np.tile(np.array([[0.3, -1.0, 2.0]]), (37, 1))
    Q = np.random.default_rng(2).standard_normal((5, 3))
    np.testing.assert_allclose(O.te_scores(Q, K, 0.7), np.full(37, 1 / 37), rtol=1e-13)


def test_lse_matches_library_logsumexp():
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((70, 32)) * 3
    K = rng.standard_normal((300, 32)) * 3
    b = rng.standard_normal(300)
    want = logsumexp(0.25 * (Q @ K.T) + b[None, :], axis=1)
    np.testing.assert_allclose(O.lse(Q, K, 0.25, b, row_chunk=16), want, rtol=1e-13, atol=1e-12)


def test_lse_equal_logits_closed_form():
    K = np.zeros((12, 4))
    Q = np.ones((3, 4))
    np.testing.assert_allclose(O.lse(Q, K, 1.0), np.full(3, math.log(12)), rtol=1e-15)


def test_scores_rms_of_attention_rows_small_brute_force():
    # pure-Python loops over a tiny case: softmax per row, then RMS over rows
    rng = np.random.default_rng(4)
    R, n, d = 3, 5, 2
    Q = rng.standard_normal((R, d))
    K = rng.standard_normal((n, d))
    c = 0.9
    s_ref = []
    rows = []
    for r in range(R):
        ls = [c * sum(Q[r, t] * K[j, t] for t in range(d)) for j in range(n)]
        z = sum(math.exp(v) for v in ls)
        rows.append([math.exp(v) / z for v in ls])
    for j in range(n):
        s_ref.append(math.sqrt(sum(rows[r][j] ** 2 for r in range(R)) / R))
    np.testing.assert_allclose(O.te_scores(Q, K, c, row_chunk=2), s_ref, rtol=1e-13)


# ------------------------------------------------------------------- invariants

def _rand_case(seed, R=6, n=40, d=8, scale=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((R, d)) * scale, rng.standard_normal((n, d)) * scale


@pytest.mark.parametrize("seed", range(5))
def test_score_range_and_square_sum_bounds(seed):
    Q, K = _rand_case(seed, scale=2.0)
    s = O.te_scores(Q, K, 0.5)
    assert np.all(s >= 0) and np.all(s <= 1)
    ss = (s * s).sum()
    assert 1 / K.shape[0] - 1e-12 <= ss <= 1 + 1e-12


@pytest.mark.parametrize("seed", range(3))
def test_bias_shift_invariance_with_internal_lse(seed):
    Q, K = _rand_case(seed)
    b = np.random.default_rng(seed + 10).standard_normal(K.shape[0])
    s1 = O.te_scores(Q, K, 0.4, bias=b)
    s2 = O.te_scores(Q, K, 0.4, bias=b + 3.25)
    np.testing.assert_allclose(s1, s2, rtol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_key_permutation_equivariance(seed):
    Q, K = _rand_case(seed)
    p = np.random.default_rng(seed + 20).permutation(K.shape[0])
    np.testing.assert_allclose(O.te_scores(Q, K[p], 0.4), O.te_scores(Q, K, 0.4)[p], rtol=1e-12)


def test_row_order_invariance():
    Q, K = _rand_case(7, R=9)
    p = np.random.default_rng(8).permutation(9)
    np.testing.assert_allclose(O.te_scores(Q[p], K, 0.4), O.te_scores(Q, K, 0.4), rtol=1e-12)


def test_supplied_exact_lse_equals_internal():
    Q, K = _rand_case(9)
    b = np.random.default_rng(9).standard_normal(K.shape[0])
    L = logsumexp(0.4 * (Q @ K.T) + b[None, :], axis=1)
    np.testing.assert_allclose(O.te_scores(Q, K, 0.4, lse_rows=L, bias=b), O.te_scores(Q, K, 0.4, bias=b), rtol=1e-12)


def test_supplied_lse_is_used_as_given():
    # LSE raised by delta scales every weight by exp(-delta), hence every score
    Q, K = _rand_case(11)
    L = O.lse(Q, K, 0.4)
    np.testing.assert_allclose(O.te_scores(Q, K, 0.4, lse_rows=L + 0.5), O.te_scores(Q, K, 0.4) * math.exp(-0.5),
                               rtol=1e-12)


def test_row_slab_size_does_not_matter():
    Q, K = _rand_case(12, R=37)
    np.testing.assert_allclose(O.te_scores(Q, K, 0.4, row_chunk=5), O.te_scores(Q, K, 0.4, row_chunk=1000),
                               rtol=1e-13)


def test_gqa_unit_rows_take_the_groups_query_heads():
    # Q [S=1][H*G=6][q=2][d=3] with H = 3, G = 2: KV head 1 uses query heads 2 and 3
    Q = np.arange(1 * 6 * 2 * 3, dtype=np.float64).reshape(1, 6, 2, 3)
    rows = O.unit_rows(Q, 0, 1, 2)
    assert rows.shape == (4, 3)
    np.testing.assert_array_equal(rows, np.concatenate([Q[0, 2], Q[0, 3]]))


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F7F], dtype=np.uint16)
    got = O.widen(bits, "bf16")
    assert got.tolist() == [1.0, -1.0, 3.140625, 0.0, 3.3895313892515355e38]


# ------------------------------------------------------------------- selection

def _brute_topm(s, m):
    """The unique m-subset where every kept position beats every dropped one under (s desc, j asc)."""
    n = len(s)
    hits = []
    for sub in itertools.combinations(range(n), m):
        ks = set(sub)
        ok = all((s[i] > s[j]) or (s[i] == s[j] and i < j) for i in ks for j in range(n) if j not in ks)
        if ok:
            hits.append(list(sub))
    assert len(hits) == 1
    return hits[0]


@settings(max_examples=60, deadline=None)
@given(st.lists(st.integers(0, 4), min_size=1, max_size=9), st.data())
def test_select_matches_brute_force_with_ties(vals, data):
    s = np.array(vals, dtype=np.float64) / 4.0
    m = data.draw(st.integers(0, len(vals)))
    assert O.select_topm(s, m).tolist() == _brute_topm(list(s), m)


def test_select_edges():
    s = np.array([0.1, 0.3, 0.3, 0.2])
    assert O.select_topm(s, 0).tolist() == []
    assert O.select_topm(s, 4).tolist() == [0, 1, 2, 3]
    assert O.select_topm(s, 1).tolist() == [1]
    with pytest.raises(ValueError):
        O.select_topm(s, 5)


def test_gather_keeps_rows_in_ascending_order():
    X = np.arange(40, dtype=np.uint16).reshape(10, 4)
    kept = np.array([1, 4, 7])
    out = O.gather(X, kept)
    np.testing.assert_array_equal(out, X[[1, 4, 7]])
    assert out.dtype == X.dtype


# ------------------------------------------------------------------- paged plan

@pytest.mark.parametrize("ex", _load("paged_examples.json")["examples"], ids=lambda e: e["name"])
def test_paged_worked_examples(ex):
    p = O.paged_plan(ex["n"], ex["m"], ex["B"], ex["kept"])
    assert (p.N, p.X, p.start) == (ex["N"], ex["X"], ex["start"])
    assert p.src == ex["src"] and p.dst == ex["dst"]
    new, freed = O.table_update(np.array(ex["table"], dtype=np.int32), ex["n"], ex["m"], ex["B"])
    assert new.tolist() == ex["new_table"] and freed.tolist() == ex["freed"]
    assert p.freed_count == len(ex["freed"])


def _simulate(n, m, B, kept, H=1, seed=0):
    """Apply plan + table update to a pool whose slots hold their own position tag."""
    N = -(-n // B)
    rng = np.random.default_rng(seed)
    table = rng.permutation(N + 3)[:N].astype(np.int32)  # physical ids, some unused
    pool = np.full((N + 3, B, H, 1), -7, dtype=np.int64)
    for p in range(n):
        pool[table[p // B], p % B, :, 0] = p
    vpool = pool.copy() * 10
    before = pool.copy()
    plan = O.paged_plan(n, m, B, kept)
    for h in range(H):
        O.apply_paged_copy(pool, vpool, table, h, plan)
    new, freed = O.table_update(table, n, m, B)
    return plan, table, new, freed, pool, vpool, before


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 70), st.sampled_from([1, 2, 4, 16]), st.data())
def test_paged_plan_invariants(n, B, data):
    m = data.draw(st.integers(0, n))
    kept = sorted(data.draw(st.lists(st.integers(0, n - 1), min_size=m, max_size=m, unique=True)))
    plan, table, new, freed, pool, vpool, before = _simulate(n, m, B, kept)
    W = set(range(plan.start, plan.start + m))
    ks = set(kept)
    assert set(plan.src) == ks - W and set(plan.dst) == W - ks
    assert len(plan.src) == len(plan.dst) and not set(plan.src) & set(plan.dst)
    assert plan.src == sorted(plan.src) and plan.dst == sorted(plan.dst)
    # after the move, the first m new logical slots hold exactly the kept tags
    tags = []
    for p in range(m):
        tags.append(int(pool[new[p // B], p % B, 0, 0]))
    assert sorted(tags) == kept
    # the V pool moved with K (tags x10)
    assert sorted(int(vpool[new[p // B], p % B, 0, 0]) // 10 for p in range(m)) == kept
    # stationary kept tokens never moved
    for j in ks & W:
        q = j - plan.start
        assert pool[new[q // B], q % B, 0, 0] == j
    # freed blocks: the first N - X logical blocks, and no kept tag is read from them afterwards
    N, X = -(-n // B), -(-m // B)
    assert freed.tolist() == table[:N - X].tolist()
    assert len(freed) == N - X
    assert set(freed.tolist()).isdisjoint(set(new[:X].tolist()))
    assert all(v == -1 for v in new[X:N])
    # only hole slots were written
    changed = np.argwhere(pool != before)
    written = {(int(b), int(sl)) for b, sl, _, _ in changed}
    holes = {(int(table[p // B]), p % B) for p in plan.dst}
    assert written <= holes


def test_paged_freed_count_is_ceil_n_minus_ceil_m_and_ratchet_budgets():
    # the action-token trajectory: n = 33000, B = 16, m_k = min(30000, floor(512 * 1.75^k))
    want = {0: (512, 2031), 1: (896, 2007), 2: (1568, 1965), 3: (2744, 1891),
            4: (4802, 1762), 5: (8403, 1537), 6: (14706, 1143)}
    from workloads import c4_budget
    for k, (m, freed) in want.items():
        assert c4_budget(k) == m
        kept = list(range(33000 - m, 33000))
        assert O.paged_plan(33000, m, 16, kept).freed_count == freed


def test_paged_rejects_bad_kept():
    with pytest.raises(ValueError):
        O.paged_plan(10, 3, 4, [1, 1, 2])
    with pytest.raises(ValueError):
        O.paged_plan(10, 3, 4, [1, 2, 10])


@pytest.mark.parametrize("n,B,H", [(37, 16, 3), (48, 16, 2), (1, 16, 1), (13, 4, 4), (16, 1, 2)])
def test_paged_unit_keys_reads_through_the_table(n, B, H):
    """The paged reader returns, for every head, exactly the keys that were written slot by slot
    at pool[table[p // B], p % B, h] for p < n -- through a permuted table with unused physical
    blocks, spare table entries past ceil(n/B) and a ragged last block whose padding slots hold
    other values -- and reads nothing else."""
    d = 5
    N = -(-n // B)
    rng = np.random.default_rng(n * 100 + B * 10 + H)
    nblocks = N + 4
    table = np.full(N + 3, -1, dtype=np.int32)
    table[:N] = rng.permutation(nblocks)[:N]
    table[N] = int(np.setdiff1d(np.arange(nblocks), table[:N])[0])  # a spare entry past ceil(n/B)
    pool = rng.integers(1000, 2000, (nblocks, B, H, d)).astype(np.int64)  # not a key anywhere
    want = rng.integers(-999, 0, (H, n, d)).astype(np.int64)              # distinct range from the filler
    for h in range(H):
        for p in range(n):
            pool[table[p // B], p % B, h, :] = want[h, p]
    for h in range(H):
        got = O.paged_unit_keys(pool, table, n, h, B)
        assert got.shape == (n, d)
        np.testing.assert_array_equal(got, want[h])
    # a block id outside [0, ceil(n/B)) of the table never matters: scramble the spare and the pads
    pool2 = pool.copy()
    pool2[table[N]] = -5
    for p in range(n, N * B):
        pool2[table[p // B], p % B] = -6
    for h in range(H):
        np.testing.assert_array_equal(O.paged_unit_keys(pool2, table, n, h, B), want[h])


# ------------------------------------------------------------------- segments (delayed turns)

@pytest.mark.parametrize("ex", _load("segment_examples.json")["examples"], ids=lambda e: e["name"])
def test_segment_worked_examples(ex):
    B, a, n, L, m = ex["B"], ex["start"], ex["n"], ex["cache_len"], ex["m"]
    plan = O.paged_plan(n, m, B, ex["kept"])
    assert [a + plan.start, a + plan.start + m] == ex["window"]
    assert [a + x for x in plan.src] == ex["src_abs"] and [a + x for x in plan.dst] == ex["dst_abs"]
    new, freed = O.table_update_segment(np.array(ex["table"], dtype=np.int32), a, n, L, m, B)
    assert new.tolist() == ex["new_table"] and freed.tolist() == ex["freed"]
    new_len = a + m if a + n == L else L - plan.freed_count * B
    assert new_len == ex["new_len"]


def test_segment_update_reduces_to_whole_sequence():
    t = np.array([3, 1, 4, 0, 2, -1], dtype=np.int32)
    for n, m in ((17, 5), (16, 16), (20, 0), (9, 9)):
        a1, f1 = O.table_update(t, n, m, 4)
        a2, f2 = O.table_update_segment(t, 0, n, n, m, 4)
        assert a1.tolist() == a2.tolist() and f1.tolist() == f2.tolist()


@settings(max_examples=150, deadline=None)
@given(st.sampled_from([1, 2, 4, 8]), st.integers(0, 5), st.integers(1, 6), st.integers(0, 20), st.data())
def test_segment_compaction_keeps_prefix_kept_suffix(B, pre_blocks, seg_blocks, suffix, data):
    """Compacting a block-aligned middle segment: the prefix is untouched, the segment's first m
    slots hold exactly the kept tokens, and the suffix follows in order right after them."""
    a = pre_blocks * B
    n = seg_blocks * B if suffix else data.draw(st.integers(1, seg_blocks * B))
    L = a + n + suffix
    m = B * data.draw(st.integers(0, n // B)) if suffix else data.draw(st.integers(0, n))
    kept = sorted(data.draw(st.lists(st.integers(0, n - 1), min_size=m, max_size=m, unique=True)))
    NT = -(-L // B)
    rng = np.random.default_rng(B * 1000 + a + n)
    table = rng.permutation(NT + 2)[:NT].astype(np.int32)
    pool = np.full((NT + 2, B, 1, 1), -9, dtype=np.int64)
    for p in range(L):
        pool[table[p // B], p % B, 0, 0] = p
    vpool = pool.copy()
    plan = O.paged_plan(n, m, B, kept)
    O.apply_paged_copy(pool, vpool, table, 0, plan, offset=a)
    new, freed = O.table_update_segment(table, a, n, L, m, B)
    new_len = a + m if not suffix else L - plan.freed_count * B
    read = [int(pool[new[p // B], p % B, 0, 0]) for p in range(new_len)]
    assert read[:a] == list(range(a))
    assert sorted(read[a:a + m]) == [a + j for j in kept]
    assert read[a + m:] == list(range(a + n, L))
    assert len(freed) == plan.freed_count and set(freed.tolist()).isdisjoint(new[: -(-new_len // B)].tolist())
