"""Shared checks for the GPU parity tests: the HIP path against the float64 oracle.

Acceptance (scores within 1e-3 relative; selection equal up to swaps inside the 1e-3 tie band
around the m-th score; compaction bit-exact) follows the stated target of the path. Scores whose
exact value is below 1e-30 are compared with an absolute bound of 1e-33: their squared weights
fall under float32's range even with the 2^100 accumulation offset.
"""
from __future__ import annotations

import sys

import numpy as np

import workloads as W
from oracle import oracle as O

SCORE_RTOL = 1e-3
TINY = 1e-30
TINY_ATOL = 1e-33


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ----------------------------------------------------------------------------- oracle process pool

_JOB: dict = {}


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def _job_call(i):
    return _JOB["fn"](*_JOB["items"][i])


def shared_array(shape, dtype) -> np.ndarray:
    """Zeroed array in an anonymous shared mapping: forked workers write into it in place."""
    import mmap
    count = int(np.prod(shape))
    mm = mmap.mmap(-1, max(count * np.dtype(dtype).itemsize, 1))
    return np.frombuffer(mm, dtype=dtype, count=count).reshape(shape)


def pool_map(fn, items, workers: int | None = None) -> list:
    """fn(*item) for every item, in forked worker processes with one BLAS thread each; results in
    item order. fn may be a closure: it and the arrays it reads reach the workers through fork,
    so only the item index and the (small) results are pickled. Outputs that are large go to
    arrays from `shared_array`. An assertion in a worker is raised here."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    items = list(items)
    workers = min(workers or W.gen.default_workers(), max(1, len(items)))
    if workers <= 1:
        return [fn(*it) for it in items]
    _JOB.update(fn=fn, items=items)
    try:
        with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("fork"),
                                 initializer=_one_blas_thread) as ex:
            return list(ex.map(_job_call, range(len(items)), chunksize=1))
    finally:
        _JOB.clear()


def check_unit_outputs(scores, kept, ref, m, what, gathers=()) -> tuple:
    """Every check of one unit: scores against the oracle's, the kept list's form, selection
    exact on the GPU's own scores and within the tie band of the oracle's, and bit-exact gathers
    (pairs of (stored rows [n][d], compacted rows [m_max][d])). Returns (worst rel err, swaps)."""
    n = ref.shape[0]
    worst = check_scores(scores[:n], ref, what)
    check_kept_form(kept, m, n, what)
    check_selection_exact(kept, scores[:n], m, what)
    swaps = check_selection_band(kept, ref, m, what)
    for X, out in gathers:
        check_gather(X, kept, out, m, what)
    return worst, swaps


def summarize_units(results: dict, name: str, group: str = "s") -> float:
    """Log the worst score error (and tie-band swaps) of every unit, one line per sequence or
    layer, and return the overall worst."""
    by_s: dict = {}
    for (s, h), (worst, swaps) in sorted(results.items()):
        by_s.setdefault(s, []).append((h, worst, swaps))
    for s, row in by_s.items():
        say(f"  {name} {group}={s}: " + " ".join(f"h{h} {wv:.2e}/{sw}" for h, wv, sw in row))
    overall = max(wv for wv, _ in results.values())
    say(f"[ok] {name}: {len(results)} units against the oracle; worst score rel err {overall:.3g}; "
        f"tie-band swaps {sum(sw for _, sw in results.values())}")
    return overall


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


def _am_rownorm(E, w):
    Ew = E * w[None, :]
    rs = Ew.sum(axis=1)
    return np.where(rs[:, None] > 0, Ew / np.where(rs > 0, rs, 1.0)[:, None], 0.0)


def check_am_unit(rows, K, V, lse_rows, kept, beta_row, vc_rows, dtype, scale, iters_beta, iters_v,
                  what: str = "") -> dict:
    """One unit's Attention Matching outputs (beta_row [m_max], vc_rows [m_max][d]; the first
    m = len(kept) filled, the rest holding the sentinel 7.0) against the oracle running the same
    iterations in float64.

    AM's parameters are only determined where the proxy rows see them: a key that only rows
    with a negligible partition function attend to can take almost any bias. Parity is therefore
    checked on what the fit determines -- the objective, the fitted partition functions and the
    compacted attention output of the rows that carry weight, and beta / V_C of the keys with
    real support -- each against the oracle within 2e-3, and every finite bias within 1e-2 (the
    float32 iterations drift a little along the fit's poorly determined directions)."""
    m = len(kept)
    rb, rv = O.am_unit(rows, K, V, kept, dtype, scale, iters_beta, iters_v, lse_rows)
    gb, gv = beta_row[:m].astype(np.float64), vc_rows[:m].astype(np.float64)
    t = what
    assert np.all(np.isfinite(gv)) and not np.any(np.isnan(gb)), f"{t}: non-finite output"
    Q64, K64, V64 = O.widen(rows, dtype), O.widen(K, dtype), O.widen(V, dtype)
    z, Y, M, _ = O.am_targets(Q64, K64, V64, scale, lse_rows)
    E = O.am_design(Q64, K64[kept], scale, M)
    wg, wr = np.exp(gb), np.exp(rb)
    og, orf = np.linalg.norm(E @ wg - z), np.linalg.norm(E @ wr - z)
    d_obj = abs(og - orf) / max(orf, 1e-300)
    assert d_obj <= 1e-3 or abs(og - orf) <= 2e-5 * np.linalg.norm(z), f"{t}: objective {og:.6g} vs {orf:.6g}"
    heavy = z >= 1e-3 * z.max()
    fit_g, fit_r = (E @ wg)[heavy] / z[heavy], (E @ wr)[heavy] / z[heavy]
    d_fit = float(np.max(np.abs(fit_g - fit_r)))
    assert d_fit <= 2e-3, f"{t}: fitted partition functions differ by {d_fit:.3g}"
    Pg, Pr = _am_rownorm(E, wg), _am_rownorm(E, wr)
    outg, outr = Pg @ gv, Pr @ rv
    d_out = float(np.max(np.abs(outg[heavy] - outr[heavy]) / (1.0 + np.abs(outr[heavy]))))
    assert d_out <= 2e-3, f"{t}: compacted attention outputs differ by {d_out:.3g}"
    supp_b = (E.T @ z) >= 1e-2 * (E.T @ z).max()
    d_beta = float(np.max(np.abs(gb[supp_b] - rb[supp_b]))) if supp_b.any() else 0.0
    assert d_beta <= 2e-3, f"{t}: beta of supported keys differs by {d_beta:.3g}"
    supp_v = Pr[heavy].sum(axis=0) >= 1e-2 * Pr[heavy].sum(axis=0).max()
    d_vc = float(np.max(np.abs(gv[supp_v] - rv[supp_v]) / (1.0 + np.abs(rv[supp_v])))) if supp_v.any() else 0.0
    assert d_vc <= 2e-3, f"{t}: V_C of supported keys differs by {d_vc:.3g}"
    fin = np.isfinite(rb)
    d_all = float(np.max(np.abs(gb[fin] - rb[fin]))) if fin.any() else 0.0
    assert np.array_equal(np.isfinite(gb), fin) and d_all <= 1e-2, f"{t}: beta differs by {d_all:.3g}"
    assert og <= np.linalg.norm(E @ np.ones_like(wr) - z) * (1 + 1e-6) + 2e-5 * np.linalg.norm(z), \
        f"{t}: the fit made things worse"
    assert np.all(beta_row[m:] == 7.0) and np.all(vc_rows[m:] == 7.0), f"{t}: rows past m touched"
    return {"obj": d_obj, "fit": d_fit, "out": d_out, "beta": d_beta, "vc": d_vc}


def slot_setup(w, data, dead_frac, rng):
    """A slot pool from the paged pool plus one sentinel block (K = -1e4 as on the page, V = 0);
    per-(sequence, head) slot maps from the block table, with a random share of positions
    already redirected to the dead slot."""
    nb, B, H, d = data["k_pool"].shape
    sent = np.full((1, B, H, d), W.f32_to_bf16_bits(np.float32(-1.0e4)) if w.dtype == "bf16" else -1.0e4,
                   dtype=data["k_pool"].dtype)
    pool = np.concatenate([data["k_pool"], sent]).reshape(-1, H, d)
    dead = nb * B
    smap = np.zeros((w.S, H, w.n_max), dtype=np.int32)
    live = np.zeros((w.S, H, w.n_max), dtype=bool)
    for s in range(w.S):
        n = w.n[s]
        pos = np.arange(n)
        base = data["table"][s][pos // B].astype(np.int64) * B + pos % B
        for h in range(H):
            lv = rng.random(n) >= dead_frac
            smap[s, h, :n] = np.where(lv, base, dead)
            live[s, h, :n] = lv
    return pool, smap, live, dead


def score_key_subtiles(lens, H: int, causal: bool = False, slot_bias: bool = False) -> int:
    """The keys per wave (in 16-key subtiles) that the library picks for the MFMA score kernel,
    restated here so that a test can make sure it runs the variant it names: 8, unless 4 or 9 is
    estimated at least 5 % faster (per CU, ceil(workgroups / 256) workgroups of (subtiles + 1)
    units each, one alone counting 1.4; 9 never with causal rows or a biased slot map)."""
    def cost(ks):
        wg = sum(H * -(-n // (64 * ks)) for n in lens)
        per = -(-wg // 256)
        return (per if per >= 2 else 1.4) * (ks + 1)
    best, best_cost = 8, 0.95 * cost(8)
    for ks in (9, 4):
        if ks == 9 and (causal or slot_bias):
            continue
        if cost(ks) < best_cost:
            best, best_cost = ks, cost(ks)
    return best
