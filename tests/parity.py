"""Shared checks for the GPU parity tests: the HIP path against the float64 oracle.

Acceptance (scores within 1e-3 relative; selection equal up to swaps inside the 1e-3 tie band
around the m-th score; compaction bit-exact) follows the stated target of the path. Scores whose
exact value is below 1e-30 are compared with an absolute bound of 1e-33: their squared weights
fall under float32's range even with the 2^100 accumulation offset.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import oracle as O

SCORE_RTOL = 1e-3
TINY = 1e-30
TINY_ATOL = 1e-33


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_scores(got: np.ndarray, ref: np.ndarray, what: str = "") -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite scores"
    big = ref >= TINY
    rel = np.abs(got[big] - ref[big]) / ref[big]
    worst = float(rel.max()) if rel.size else 0.0
    bad = np.flatnonzero(big)[rel > SCORE_RTOL]
    assert bad.size == 0, f"{what}: {bad.size} scores off by > {SCORE_RTOL} rel (worst {worst:.3g} at {bad[:5]})"
    small = ~big
    if small.any():
        assert np.all(np.abs(got[small] - ref[small]) <= TINY_ATOL), f"{what}: tiny scores off"
    return worst


def check_kept_form(kept: np.ndarray, m: int, n: int, what: str = ""):
    k = np.asarray(kept[:m], dtype=np.int64)
    assert k.size == m
    if m:
        assert k.min() >= 0 and k.max() < n, f"{what}: kept index out of range"
        assert np.all(np.diff(k) > 0), f"{what}: kept not strictly ascending"


def check_selection_exact(kept: np.ndarray, s_gpu: np.ndarray, m: int, what: str = ""):
    """The GPU's kept set is exactly top-m of its own float32 scores (ties to lower index)."""
    want = O.select_topm(np.asarray(s_gpu, dtype=np.float32).astype(np.float64), m)
    got = np.asarray(kept[:m], dtype=np.int64)
    assert np.array_equal(got, want), f"{what}: selection differs from top-m of the GPU's own scores"


def check_selection_band(kept: np.ndarray, s_ref: np.ndarray, m: int, what: str = "") -> int:
    """Against the oracle: |G| = m and G xor O lies in the 1e-3 band around the m-th score."""
    ref_kept = O.select_topm(s_ref, m)
    got = set(np.asarray(kept[:m], dtype=np.int64).tolist())
    ora = set(ref_kept.tolist())
    diff = got ^ ora
    if not diff:
        return 0
    sstar = np.sort(s_ref)[::-1][m - 1]
    band = {j for j in diff if abs(s_ref[j] - sstar) <= SCORE_RTOL * sstar}
    assert band == diff, f"{what}: {len(diff - band)} selection differences outside the tie band"
    return len(diff) // 2


def check_gather(X: np.ndarray, kept: np.ndarray, out: np.ndarray, m: int, what: str = ""):
    want = O.gather(X, np.asarray(kept[:m], dtype=np.int64))
    assert np.array_equal(out[:m].view(np.uint8), want.view(np.uint8)), f"{what}: compacted rows differ"


def oracle_lse_units(w, data_Q, keys_of, units, bias_of=None) -> dict:
    """Oracle LSE (float64) per unit, from stored inputs."""
    out = {}
    for s, h in units:
        rows = O.unit_rows(data_Q, s, h, w.G)
        b = None if bias_of is None else bias_of(s)
        out[(s, h)] = O.lse_unit(rows, keys_of(s, h), w.dtype, w.logit_scale, b)
    return out
