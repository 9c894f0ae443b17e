"""Plain float64 CPU oracle for proxy-query token eviction: score -> select -> compact.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module: only the test
suite, the smoke check and the benchmark's CPU-baseline leg use it. It shares no code with the
HIP library; both sides read the same stored input bytes, produced by ``workloads``.

Sources (page titles as they appear on the pages):
  [TE]  "Practical Online KV Cache Compaction for LLM Agents: An Empirical Study"
        (agifrontier tutorial page), section on the design space, the Token Eviction score
        equation: s_j(Q, K) = ((1/q) * sum_i alpha_ij^2)^(1/2) over q proxy queries, then keep
        the top-m positions with their original keys and values.
  [ACT] "ActKV" analysis page (zhichai.net topic), paragraph on the paged-memory system
        component: attention recovered block by block as exp(logit - LSE) with the LSE a
        byproduct of paged attention; conflict-free slot plan where the tail X logical blocks
        become the target region, kept entries outside it are paired one-to-one with holes
        inside it, all pairs are copied in one parallel pass and the emptied blocks go back
        to the scheduler.

Readings where the pages leave a step open (each is listed with its reason in the design notes):
  * alpha_ij = softmax_j(c * q_i . k_j + b_j) with c = 1/sqrt(d) unless the caller gives another
    scale; b is an optional per-key additive logit bias (0 when absent).
  * GQA: the G*q proxy rows of the G query heads that share a KV head are stacked and the mean
    in the score runs over all R = G*q rows.
  * A supplied LSE is used as given (natural log, one value per proxy row).
  * Ties in the score go to the lower position; the kept list is returned ascending.
  * Paged: N = ceil(n/B), X = ceil(m/B), window W = [(N-X)*B, (N-X)*B + m); sources are kept
    positions outside W, holes are positions of W that are not kept, both ascending, the i-th
    source fills the i-th hole. The new block table is old[N-X .. N), entries X .. N-1 become
    -1, and old[0 .. N-X) are freed, i.e. ceil(n/B) - ceil(m/B) blocks.
  * ActKV retention ([ACT], paragraph on action-critical entries and LRFU): the attention that
    the action tokens pay an entry is their mean weight on it; "within the top 90 %" is read as
    the shortest run of entries, in descending attention order (ties to the lower position),
    that holds 90 % of the total attention, the sums taken on the float32 masses quantised to
    multiples of 2^-32 (so that the membership decision is exact on both sides); LRFU's value
    decays by 2^-lambda per policy step and a hit adds 1.
  * Attention Matching ([TE], design-space section, the AM equations): after the top-m keys
    K_C are chosen, beta minimises || exp(Q K_C^T + beta) 1 - exp(Q K^T) 1 ||^2 and V_C
    minimises || A_hat(Q; K_C, beta, V_C) - A(Q; K, V) ||_F^2. The pages name no optimiser;
    read here as: logits carry the scale c like every other logit, w = exp(beta) >= 0 is fitted
    by multiplicative non-negative least-squares updates from w = 1 (beta = 0, plain eviction),
    the exponentials of a unit taken relative to its largest LSE (a common factor that does not
    move the minimiser); V_C by Landweber iterations from the kept keys' original values with
    step 1 / (largest column sum of the compacted attention), a fixed number of each.
  * Layout-preserving eviction ([IKV] "IntentKV" page, layout-preserving eviction): evicted
    positions are redirected to one reserved dead slot in a per-position slot map; the page's
    constant sentinel key cannot cancel every query's attention (a query whose components sum
    below zero favours it), so the dead slot is read as a logit mask: a position mapped to it
    takes no part in the softmax and its own score is 0.
  * Causal proxy rows (optional; [ACT] tallies the attention that the action tokens pay the
    entries, and an action token inside the trajectory attends only to what came before it):
    row r sees the keys at positions j <= row_pos[r]; the softmax of a row runs over its
    visible keys, masked weights are 0, and the mean over rows still divides by all R rows.

Every function below has pins in the CPU test suite (worked examples, closed forms, brute
force and invariants); none is "parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


# ----------------------------------------------------------------------------- inputs

def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly. bf16 arrives as 16-bit patterns."""
    if dtype == "bf16":
        u32 = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return u32.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- scoring

def logits(Q: np.ndarray, K: np.ndarray, scale: float, bias: np.ndarray | None = None) -> np.ndarray:
    """l_rj = c * (q_r . k_j) + b_j for proxy rows Q [R][d] and keys K [n][d] ([TE] alpha's argument)."""
    L = scale * (Q @ K.T)
    if bias is not None:
        L = L + bias[None, :]
    return L


def lse(Q: np.ndarray, K: np.ndarray, scale: float, bias: np.ndarray | None = None,
        row_chunk: int = 256) -> np.ndarray:
    """Per proxy row, LSE_r = ln sum_j exp(l_rj) over the same n keys ([ACT] softmax normaliser).

    Written as max + ln(sum exp(l - max)) so it does not overflow; rows are independent, so the
    logits are formed a slab of rows at a time only to bound memory.
    """
    R = Q.shape[0]
    out = np.empty(R, dtype=np.float64)
    for r0 in range(0, R, row_chunk):
        L = logits(Q[r0:r0 + row_chunk], K, scale, bias)
        mx = L.max(axis=1)
        out[r0:r0 + row_chunk] = mx + np.log(np.exp(L - mx[:, None]).sum(axis=1))
    return out


def te_scores(Q: np.ndarray, K: np.ndarray, scale: float, lse_rows: np.ndarray | None = None,
              bias: np.ndarray | None = None, row_chunk: int = 256) -> np.ndarray:
    """Token Eviction score of every key ([TE] score equation).

    alpha_rj = exp(l_rj - LSE_r) (the softmax weight, [ACT] LSE recovery),
    s_j = sqrt((1/R) * sum_r alpha_rj^2). The row sum is accumulated a slab of rows at a time.
    """
    R, n = Q.shape[0], K.shape[0]
    if lse_rows is None:
        lse_rows = lse(Q, K, scale, bias, row_chunk)
    lse_rows = np.asarray(lse_rows, dtype=np.float64)
    acc = np.zeros(n, dtype=np.float64)
    for r0 in range(0, R, row_chunk):
        L = logits(Q[r0:r0 + row_chunk], K, scale, bias)
        alpha = np.exp(L - lse_rows[r0:r0 + row_chunk, None])
        acc += (alpha * alpha).sum(axis=0)
    return np.sqrt(acc / R)


# ----------------------------------------------------------------------------- selection

def select_topm(s: np.ndarray, m: int) -> np.ndarray:
    """Top-m positions by score, ties to the lower position, returned ascending ([TE] top-m)."""
    n = s.shape[0]
    if not 0 <= m <= n:
        raise ValueError("need 0 <= m <= n")
    order = np.lexsort((np.arange(n), -np.asarray(s, dtype=np.float64)))  # s desc, then j asc
    return np.sort(order[:m]).astype(np.int64)


# ----------------------------------------------------------------------------- compaction

def gather(X: np.ndarray, kept: np.ndarray) -> np.ndarray:
    """Contiguous compaction: row r of the output is the stored row kept[r] ([TE] keep original K, V)."""
    return np.ascontiguousarray(X[np.asarray(kept, dtype=np.int64)])


@dataclass
class PagedPlan:
    n: int
    m: int
    B: int
    N: int            # logical blocks before compaction
    X: int            # logical blocks kept (the target region)
    start: int        # first logical slot of the window
    src: list         # kept positions outside the window, ascending
    dst: list         # holes of the window, ascending

    @property
    def freed_count(self) -> int:
        return self.N - self.X


def paged_plan(n: int, m: int, B: int, kept) -> PagedPlan:
    """Conflict-free slot plan for one (sequence, head) ([ACT] paged compaction paragraph).

    Built with plain sets, independently of how a parallel planner would locate pairs.
    """
    if not 0 <= m <= n:
        raise ValueError("need 0 <= m <= n")
    N = -(-n // B)
    X = -(-m // B)
    start = (N - X) * B
    kept_set = set(int(j) for j in kept)
    if len(kept_set) != m or any(j < 0 or j >= n for j in kept_set):
        raise ValueError("kept must hold m distinct positions in [0, n)")
    window = set(range(start, start + m))
    src = sorted(kept_set - window)
    dst = sorted(window - kept_set)
    if len(src) != len(dst):
        raise AssertionError("plan is unbalanced")
    if set(src) & set(dst):
        raise AssertionError("a slot is both read and written")
    return PagedPlan(n, m, B, N, X, start, src, dst)


def apply_paged_copy(k_pool: np.ndarray, v_pool: np.ndarray, table_row: np.ndarray, h: int,
                     plan: PagedPlan, offset: int = 0) -> None:
    """Copy K and V rows of head h from each source slot to its paired hole, in place.

    Pools are [num_blocks][B][H][d]; table_row maps logical block -> physical block; plan
    positions are relative to a segment that starts at cache position `offset`. Sources are never
    holes and holes are never read, so the order of the copies does not matter.
    """
    B = plan.B
    for a, b in zip(plan.src, plan.dst):
        a, b = a + offset, b + offset
        pa, sa = int(table_row[a // B]), a % B
        pb, sb = int(table_row[b // B]), b % B
        k_pool[pb, sb, h, :] = k_pool[pa, sa, h, :]
        v_pool[pb, sb, h, :] = v_pool[pa, sa, h, :]


def table_update(table_row: np.ndarray, n: int, m: int, B: int) -> tuple[np.ndarray, np.ndarray]:
    """New block table and the freed physical blocks (logical order) for one sequence."""
    N = -(-n // B)
    X = -(-m // B)
    old = np.asarray(table_row, dtype=np.int32)
    new = old.copy()
    new[:X] = old[N - X:N]
    new[X:N] = -1
    freed = old[:N - X].copy()
    return new, freed


def table_update_segment(table_row: np.ndarray, start: int, n: int, cache_len: int, m: int,
                         B: int) -> tuple[np.ndarray, np.ndarray]:
    """Block table after compacting the segment [start, start + n) of a sequence of cache_len
    tokens: the segment's first N - X logical blocks are freed and every later block slides down
    by that many entries (the kept window, then the rest of the sequence); the vacated tail
    becomes -1. With start = 0 and cache_len = n this is `table_update`.
    """
    if start % B:
        raise ValueError("a paged segment starts on a block boundary")
    N = -(-n // B)
    X = -(-m // B)
    F = N - X
    b = start // B
    NT = -(-cache_len // B)
    old = list(int(x) for x in table_row)
    freed = old[b:b + F]
    kept_blocks = old[:b] + old[b + F:NT]
    new = np.array(kept_blocks + [-1] * F + old[NT:], dtype=np.int32)
    return new, np.array(freed, dtype=np.int32)


# ----------------------------------------------------------------------------- ActKV retention

def attention_mass(Q: np.ndarray, K: np.ndarray, scale: float, lse_rows: np.ndarray | None = None,
                   bias: np.ndarray | None = None, row_chunk: int = 256) -> np.ndarray:
    """Attention the proxy rows pay each key, averaged over the rows ([ACT]: for every entry,
    the attention scores of all action tokens on it): mass_j = (1/R) * sum_r alpha_rj, with
    alpha_rj = exp(l_rj - LSE_r) as in the score."""
    R, n = Q.shape[0], K.shape[0]
    if lse_rows is None:
        lse_rows = lse(Q, K, scale, bias, row_chunk)
    lse_rows = np.asarray(lse_rows, dtype=np.float64)
    acc = np.zeros(n, dtype=np.float64)
    for r0 in range(0, R, row_chunk):
        L = logits(Q[r0:r0 + row_chunk], K, scale, bias)
        acc += np.exp(L - lse_rows[r0:r0 + row_chunk, None]).sum(axis=0)
    return acc / R


def causal_weights(Q: np.ndarray, K: np.ndarray, scale: float, row_pos, lse_rows=None,
                   bias: np.ndarray | None = None, power: int = 2, row_chunk: int = 256):
    """Scores (power 2) or attention masses (power 1) when proxy row r only sees the keys at
    positions j <= row_pos[r] (a causal mask for in-trajectory action tokens, [ACT]: the
    attention each action token actually paid). Per row the weights are the softmax over its
    visible keys, alpha_rj = exp(l_rj - LSE_r) with LSE_r over the visible keys (or the supplied
    value); masked weights are 0, and a row that sees no key contributes nothing. The mean over
    rows still divides by all R rows. Returns (scores or masses, the LSE used per row)."""
    R, n = Q.shape[0], K.shape[0]
    pos = np.asarray(row_pos, dtype=np.int64)
    j = np.arange(n)
    lse_out = np.full(R, -np.inf, dtype=np.float64)
    acc = np.zeros(n, dtype=np.float64)
    for r0 in range(0, R, row_chunk):
        r1 = min(R, r0 + row_chunk)
        vis = j[None, :] <= pos[r0:r1, None]
        L = np.where(vis, logits(Q[r0:r1], K, scale, bias), -np.inf)
        if lse_rows is None:
            for r in range(r1 - r0):
                if vis[r].any():
                    lv = L[r, vis[r]]
                    mx = lv.max()
                    lse_out[r0 + r] = mx + np.log(np.exp(lv - mx).sum())
        else:
            lse_out[r0:r1] = np.asarray(lse_rows, dtype=np.float64)[r0:r1]
        with np.errstate(invalid="ignore"):
            alpha = np.where(vis, np.exp(L - lse_out[r0:r1, None]), 0.0)
        acc += (alpha ** power).sum(axis=0)
    out = np.sqrt(acc / R) if power == 2 else acc / R
    return out, lse_out


def causal_unit(Qs, Ks, row_pos, dtype, scale, bias=None, lse_rows=None, power: int = 2):
    """causal_weights of one unit from stored rows/keys (widened exactly to float64)."""
    b = None if bias is None else np.asarray(bias, dtype=np.float64)
    return causal_weights(widen(Qs, dtype), widen(Ks, dtype), scale, row_pos, lse_rows, b, power)


def causal_unit_live(Qs, Ks, live, row_pos, dtype, scale, bias=None, lse_rows=None, power: int = 2):
    """causal_unit when only the `live` positions take part (the dead slot of [IKV]'s
    layout-preserving eviction read as a logit mask, combined with causal [ACT] rows): row r sees
    the live keys at positions j <= row_pos[r]. The live keys keep their order, so a row sees
    the first (number of live positions <= row_pos[r]) of them; dead positions score 0.
    Returns (scores or masses over all positions, the LSE used per row)."""
    live = np.asarray(live, dtype=bool)
    n = live.shape[0]
    pos = np.asarray(row_pos, dtype=np.int64)
    seen = np.concatenate([[0], np.cumsum(live)])           # live positions among the first i
    vis_live = seen[np.clip(pos + 1, 0, n)] - 1             # last live index each row sees
    out = np.zeros(n, dtype=np.float64)
    b = None if bias is None else np.asarray(bias)[live]
    sub, lse_out = causal_unit(Qs, np.asarray(Ks)[live], vis_live, dtype, scale, b, lse_rows, power)
    out[live] = sub
    return out, lse_out


MASS_QUANTUM = 2 ** 32   # a mass of 1 is this many integer units
MASS_CAP = 2 ** 40       # per-entry cap of the integer mass (masses above 256)


def quantised_mass(mass_f32) -> list:
    """Integer mass of each float32 value: min(floor(mass * 2^32), 2^40), as Python ints."""
    return [min(math.floor(float(x) * MASS_QUANTUM), MASS_CAP) for x in np.asarray(mass_f32, dtype=np.float32)]


def action_critical(mass_f32, top_p: float) -> np.ndarray:
    """Action-critical entries of one unit ([ACT]: entries within the top 90 % of the action
    attention). Walk the entries in descending float32 mass, ties to the lower position, and
    take them until their integer masses add up to at least ceil(top_p * U), U the total
    integer mass (nothing when U = 0). Returns a boolean mask over the entries."""
    v = np.asarray(mass_f32, dtype=np.float32)
    n = v.shape[0]
    u = quantised_mass(v)
    total = sum(u)
    hit = np.zeros(n, dtype=bool)
    if total == 0:
        return hit
    target = math.ceil(float(top_p) * float(total))
    order = np.lexsort((np.arange(n), -v.astype(np.float64)))  # mass desc, then position asc
    acc = 0
    for j in order:
        hit[j] = True
        acc += u[j]
        if acc >= target:
            break
    return hit


def lrfu_step(state: np.ndarray, hit: np.ndarray, decay: float) -> np.ndarray:
    """One LRFU step ([ACT]: LRFU whose hit signal is "hit by action attention"): every
    entry's combined recency-frequency value is multiplied by decay = 2^-lambda and a hit adds 1."""
    return float(decay) * np.asarray(state, dtype=np.float64) + np.asarray(hit, dtype=np.float64)


def lrfu_crf(hit_steps, now: int, lam: float) -> float:
    """LRFU's combined recency-frequency value at step `now` of an entry hit at the given steps:
    the sum over hits of (1/2)^(lam * (now - t))."""
    return float(sum(0.5 ** (lam * (now - t)) for t in hit_steps))


def side_order(n: int, m: int, B: int, kept) -> list:
    """Old position of the entry found at each new position 0..m-1 after compaction: the kept
    list itself for contiguous compaction (B = 0); for the paged slot plan, window slot start + p
    keeps its own entry when kept, else holds the source paired with that hole."""
    kept = [int(j) for j in kept]
    if B == 0:
        return kept
    plan = paged_plan(n, m, B, kept)
    filled = dict(zip(plan.dst, plan.src))
    return [filled.get(w, w) for w in range(plan.start, plan.start + m)]


def mass_unit(Qs, Ks, dtype, scale, bias=None, lse_rows=None):
    """Attention mass of one unit from stored rows/keys (widened exactly to float64)."""
    Qd = widen(Qs, dtype)
    Kd = widen(Ks, dtype)
    b = None if bias is None else np.asarray(bias, dtype=np.float64)
    return attention_mass(Qd, Kd, scale, lse_rows=lse_rows, bias=b)


# ----------------------------------------------------------------------------- layout-preserving eviction

def evict_redirect(slot_row, kept, n: int, dead: int) -> np.ndarray:
    """[IKV] sentinel dead slot: every position of [0, n) that is not kept is redirected to the
    dead slot; kept positions and positions past n keep their slots."""
    out = np.array(slot_row, dtype=np.int64, copy=True)
    keep = set(int(j) for j in kept)
    for p in range(n):
        if p not in keep:
            out[p] = dead
    return out


def slot_unit_keys(pool, slot_row, n: int, h: int):
    """Stored keys [n][d] of head h read through a per-position slot map (pool [slots][H][d])."""
    return pool[np.asarray(slot_row[:n], dtype=np.int64), h, :]


def score_unit_live(Qs, Ks, live, dtype, scale, bias=None, lse_rows=None, power: int = 2):
    """TE score (power 2) or attention mass (power 1) of one unit when only the `live` positions
    take part in the softmax (the logit-mask reading of the dead slot); dead positions score 0."""
    live = np.asarray(live, dtype=bool)
    out = np.zeros(live.shape[0], dtype=np.float64)
    if not live.any():
        return out
    Kl = np.asarray(Ks)[live]
    b = None if bias is None else np.asarray(bias)[live]
    f = score_unit if power == 2 else mass_unit
    out[live] = f(Qs, Kl, dtype, scale, b, lse_rows)
    return out


# ----------------------------------------------------------------------------- Attention Matching

def am_targets(Q, K, V, scale, lse_rows=None):
    """What AM matches ([TE] AM equations): the partition function of every proxy row over all n
    keys, relative to the unit's largest LSE, z_i = exp(LSE_i - M), and the attention output
    Y = softmax(c Q K^T) V. Returns (z, Y, M, LSE)."""
    if lse_rows is None:
        lse_rows = lse(Q, K, scale)
    lse_rows = np.asarray(lse_rows, dtype=np.float64)
    M = float(lse_rows.max())
    P = np.exp(logits(Q, K, scale) - lse_rows[:, None])
    return np.exp(lse_rows - M), P @ np.asarray(V, dtype=np.float64), M, lse_rows


def am_design(Q, KC, scale, M):
    """E_ij = exp(c q_i . k_Cj - M): the kept keys' unnormalised weights, on the same scale as z."""
    return np.exp(logits(Q, KC, scale) - M)


def am_fit_beta(E, z, iters: int):
    """Non-negative least squares for w = exp(beta) in || E w - z ||^2 by multiplicative updates
    w <- w * (E^T z) / (E^T E w), from w = 1 (beta = 0). A zero denominator leaves w_j at 0."""
    E = np.asarray(E, dtype=np.float64)
    b = E.T @ z
    w = np.ones(E.shape[1])
    for _ in range(iters):
        g = E.T @ (E @ w)
        w = np.where(g > 0, w * b / np.where(g > 0, g, 1.0), 0.0)
    return w


def am_fit_values(E, w, Y, V0, iters: int):
    """Least squares for V_C in || P V_C - Y ||_F^2, P the compacted attention (rows of E w-weighted
    and normalised), by Landweber iterations V <- V - eta P^T (P V - Y) from V_0 (the kept keys'
    values), eta = 1 / max_j sum_i P_ij (then eta ||P||_2^2 <= 1, so the iteration is stable)."""
    Ew = np.asarray(E, dtype=np.float64) * np.asarray(w, dtype=np.float64)[None, :]
    rs = Ew.sum(axis=1)
    P = np.where(rs[:, None] > 0, Ew / np.where(rs > 0, rs, 1.0)[:, None], 0.0)
    cmax = P.sum(axis=0).max()
    eta = 1.0 / cmax if cmax > 0 else 0.0
    Vc = np.asarray(V0, dtype=np.float64).copy()
    for _ in range(iters):
        Vc = Vc - eta * (P.T @ (P @ Vc - Y))
    return Vc


def am_unit(Qs, Ks, Vs, kept, dtype, scale, iters_beta: int, iters_v: int, lse_rows=None):
    """Attention Matching of one unit from stored rows/keys/values: returns (beta, V_C)."""
    Q, K, V = widen(Qs, dtype), widen(Ks, dtype), widen(Vs, dtype)
    kept = np.asarray(kept, dtype=np.int64)
    z, Y, M, _ = am_targets(Q, K, V, scale, lse_rows)
    E = am_design(Q, K[kept], scale, M)
    w = am_fit_beta(E, z, iters_beta)
    with np.errstate(divide="ignore"):
        beta = np.log(w)
    return beta, am_fit_values(E, w, Y, V[kept], iters_v)


# ----------------------------------------------------------------------------- whole batches

def unit_rows(Q: np.ndarray, s: int, h: int, G: int) -> np.ndarray:
    """The R = G*q proxy rows of KV head h: query heads h*G .. h*G+G-1 of Q [S][H*G][q][d]."""
    sub = Q[s, h * G:(h + 1) * G]
    return sub.reshape(-1, sub.shape[-1])


def unit_lse(Q, s, h, G, lse_all) -> np.ndarray | None:
    if lse_all is None:
        return None
    return np.asarray(lse_all[s, h * G:(h + 1) * G], dtype=np.float64).reshape(-1)


def score_unit(Qs, Ks, dtype, scale, bias=None, lse_rows=None):
    """Scores of one unit from stored rows/keys (widened exactly to float64)."""
    Qd = widen(Qs, dtype)
    Kd = widen(Ks, dtype)
    b = None if bias is None else np.asarray(bias, dtype=np.float64)
    return te_scores(Qd, Kd, scale, lse_rows=lse_rows, bias=b)


def lse_unit(Qs, Ks, dtype, scale, bias=None):
    Qd = widen(Qs, dtype)
    Kd = widen(Ks, dtype)
    b = None if bias is None else np.asarray(bias, dtype=np.float64)
    return lse(Qd, Kd, scale, b)


def paged_unit_keys(k_pool, table_row, n, h, B):
    """Stored keys [n][d] of head h, read through the block table."""
    blocks = np.asarray(table_row[:-(-n // B)], dtype=np.int64)
    rows = k_pool[blocks, :, h, :].reshape(-1, k_pool.shape[-1])
    return rows[:n]


def run_contiguous(data: dict, G: int, dtype: str, scale: float, lse_all=None, units=None):
    """score -> select -> gather for every (s, h) of a contiguous batch.

    Returns per-unit dicts with scores, kept, K_c and V_c. ``units`` limits the work to a list
    of (s, h) pairs.
    """
    K, V, Q, n, m = data["K"], data["V"], data["Q"], data["n"], data["m"]
    S, H = K.shape[0], K.shape[1]
    bias = data.get("bias")
    out = {}
    for s, h in (units if units is not None else [(s, h) for s in range(S) for h in range(H)]):
        ns = int(n[s])
        b = None if bias is None else bias[s, :ns]
        sc = score_unit(unit_rows(Q, s, h, G), K[s, h, :ns], dtype, scale, b, unit_lse(Q, s, h, G, lse_all))
        kept = select_topm(sc, int(m[s]))
        out[(s, h)] = dict(scores=sc, kept=kept, K_c=gather(K[s, h, :ns], kept), V_c=gather(V[s, h, :ns], kept))
    return out


def run_paged(data: dict, G: int, dtype: str, scale: float, B: int, lse_all=None, seqs=None):
    """score -> select -> paged plan/copy -> table update for whole sequences (all heads).

    Works on copies of the pools and table; returns them with per-unit scores and kept sets and
    per-sequence freed lists.
    """
    k_pool = data["k_pool"].copy()
    v_pool = data["v_pool"].copy()
    table = data["table"].copy()
    Q, n, m = data["Q"], data["n"], data["m"]
    bias = data.get("bias")
    H = k_pool.shape[2]
    S = table.shape[0]
    res = dict(units={}, freed={})
    for s in (seqs if seqs is not None else range(S)):
        ns, ms = int(n[s]), int(m[s])
        b = None if bias is None else bias[s, :ns]
        plans = []
        for h in range(H):
            Ks = paged_unit_keys(k_pool, table[s], ns, h, B)
            sc = score_unit(unit_rows(Q, s, h, G), Ks, dtype, scale, b, unit_lse(Q, s, h, G, lse_all))
            kept = select_topm(sc, ms)
            plans.append(paged_plan(ns, ms, B, kept))
            res["units"][(s, h)] = dict(scores=sc, kept=kept, plan=plans[-1])
        for h in range(H):
            apply_paged_copy(k_pool, v_pool, table[s], h, plans[h])
        new, freed = table_update(table[s], ns, ms, B)
        table[s] = new
        res["freed"][s] = freed
    res.update(k_pool=k_pool, v_pool=v_pool, table=table)
    return res
