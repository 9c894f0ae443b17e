"""Seeded synthetic inputs shaped like the agent trajectories the compaction pages measure on.

This module only draws and lays out inputs: keys, values, proxy queries, the per-key logit
bias, block tables and the per-sequence budgets m. It computes no score, LSE, selection or
compaction; the oracle and the HIP path both consume the bytes it returns.

Recipe (every array is drawn per unit u = (sequence s, KV head h) from its own generator
``np.random.default_rng([config_id, s, h, tag])``, in float32, then rounded
round-to-nearest-even to bfloat16 where the workload is bf16):

* "normal" keys / values / queries: i.i.d. N(0, 1).
* "mixture" keys: 64 cluster means mu_c ~ N(0, I_d); key j >= 4 is mu_{c_j} + 0.5 * eps_j with
  c_j uniform over the 64 clusters; the 4 attention-sink keys j = 0..3 are drawn the same way
  and multiplied by 8.
* "boundary" queries: one N(0, I) query per query head (the end-of-turn token's query).
* "cluster" queries (delayed future-turn proxies): z + 0.5 * mu_c, z ~ N(0, I), c uniform.
* "action" queries: 10 non-overlapping spans of q/10 positions at seeded starts in
  [4, n - q/10]; the query for position p is z + 0.5 * mu_{c_p} (the cluster of key p).
* causal row positions (row_positions): the action tokens' own positions, or seeded uniform
  integers over [-2, n + 1].
* values: N(0, 1) (they never influence scores, only the compacted bytes).
* bias (1-layer paged trajectory): +b on the last floor(n/4) keys, 0 elsewhere.
* paged pools: vLLM-style [num_blocks][B][H][d]; identity block table, or a seeded
  permutation of one shared pool of sum(ceil(n_s / B)) blocks.

Budgets: ratio 0.2 means m = round(n / 5) (n / 5 never ends in .5); the action-token
trajectory uses the ratchet budget m_k = min(30000, floor(512 * 1.75**k)).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
import mmap
import multiprocessing
import os

import numpy as np

# generator tags: one independent stream per kind of draw
(T_CLUSTERS, T_ASSIGN, T_KEYNOISE, T_VALUES, T_QUERIES, T_QCLUSTER, T_LENGTHS, T_PERM, T_SPANS, T_KEYS,
 T_POSITIONS) = range(11)
NUM_CLUSTERS = 64
NUM_SINKS = 4
SINK_GAIN = 8.0
NUM_SPANS = 10


def _rng(cfg_id: int, s: int, h: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([cfg_id, s, h, tag])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF)          # finite inputs: cannot wrap (largest is 0xFF7FFFFF)
    r += (u >> 16) & np.uint32(1)
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def c4_budget(k: int) -> int:
    """Ratchet budget after k expansions: start 512, grow x1.75, cap 30000 (closed form, floored)."""
    return min(30000, int(math.floor(512 * 1.75 ** k)))


def ratio_budget(n: int) -> int:
    """Keep ratio 0.2: round(n / 5); n / 5 has fraction .0/.2/.4/.6/.8, so this is exact."""
    return (n + 2) // 5


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    S: int                 # sequences (or layers of one trajectory, or sessions)
    H: int                 # KV heads
    G: int                 # query heads per KV head
    q: int                 # proxy queries per query head
    d: int
    n: tuple               # keys per sequence
    m: tuple               # kept positions per sequence
    dtype: str             # "f32" | "bf16"
    keys: str              # "normal" | "mixture"
    queries: str           # "normal" | "boundary" | "cluster" | "action"
    paged: bool = False
    block_size: int = 16
    table: str = "identity"  # "identity" | "permuted"
    max_blocks: int = 0
    lse_supplied: bool = False
    bias_tail: float = 0.0
    scale: float = 0.0     # 0 -> 1/sqrt(d)
    seg_start: int = 0     # > 0 or seg_len > 0: compact only this segment (one agent turn)
    seg_len: int = 0
    causal: bool = False   # action-query rows see only the keys up to their own positions

    @property
    def R(self) -> int:
        return self.G * self.q

    @property
    def logit_scale(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.d)

    @property
    def n_max(self) -> int:
        return max(self.n)

    @property
    def m_max(self) -> int:
        return max(self.m)

    @property
    def units(self) -> int:
        return self.S * self.H

    def blocks_of(self, s: int) -> int:
        return -(-self.n[s] // self.block_size)


def _c5_lengths() -> tuple:
    g = _rng(5, 0, 0, T_LENGTHS)
    return tuple(int(x) for x in g.integers(8192, 131072, size=64, endpoint=True))


def spec(name: str, k: int | None = None) -> Workload:
    """The named workloads (c4 takes the expansion count k = 0..6)."""
    if name == "c1":
        return Workload("c1", 1, 1, 1, 1, 32, 128, (4096,), (819,), "f32", "normal", "normal")
    if name in ("c2a", "c2b"):
        q, qs = (1, "boundary") if name == "c2a" else (512, "cluster")
        return Workload(name, 2, 1, 8, 4, q, 128, (16384,), (ratio_budget(16384),), "bf16", "mixture", qs)
    if name == "c3":
        return Workload("c3", 3, 36, 8, 4, 1024, 128, (33000,) * 36, (ratio_budget(33000),) * 36,
                        "bf16", "mixture", "cluster", lse_supplied=True)
    if name == "c4":
        kk = 0 if k is None else k
        n = 33000
        return Workload(f"c4k{kk}", 4, 1, 8, 4, 330, 128, (n,), (c4_budget(kk),), "bf16", "mixture", "action",
                        paged=True, block_size=16, table="identity", max_blocks=-(-n // 16), bias_tail=0.5)
    if name == "actkv":
        # ActKV's retention step on the action-token trajectory: the inputs of "c4" (same seed),
        # budget 14706 (six ratchet expansions); scored by attention mass, kept by LRFU state
        n = 33000
        return Workload("actkv", 4, 1, 8, 4, 330, 128, (n,), (c4_budget(6),), "bf16", "mixture", "action",
                        paged=True, block_size=16, table="identity", max_blocks=-(-n // 16), bias_tail=0.5)
    if name == "sentinel":
        # layout-preserving eviction on the action-token trajectory: the inputs of "c4" (same
        # seed), read through a per-(layer, head) slot map; the evicted positions of budget 14706
        # are redirected to a dead slot instead of being compacted
        n = 33000
        return Workload("sentinel", 4, 1, 8, 4, 330, 128, (n,), (c4_budget(6),), "bf16", "mixture", "action",
                        paged=True, block_size=16, table="identity", max_blocks=-(-n // 16), bias_tail=0.5)
    if name == "am":
        # Attention Matching on the cluster-query snapshot: the inputs of "c2b" (same seed); the
        # top-m keys by Token Eviction score, then beta and V_C fitted for them
        return Workload("am", 2, 1, 8, 4, 512, 128, (16384,), (ratio_budget(16384),), "bf16", "mixture", "cluster")
    if name == "turn":
        # one 4096-token turn in the middle of a 33000-token trajectory held in 36 layers' paged
        # caches, scored with the 512 queries per query head of the turn that followed it; the
        # keep budget is round(0.2 * 4096) rounded up to whole 16-token blocks
        n, a, L = 33000, 16000, 4096
        m = -(-ratio_budget(L) // 16) * 16
        return Workload("turn", 6, 36, 8, 4, 512, 128, (n,) * 36, (m,) * 36, "bf16", "mixture", "cluster",
                        paged=True, block_size=16, table="permuted", max_blocks=-(-n // 16), seg_start=a,
                        seg_len=L)
    if name == "c5":
        n = _c5_lengths()
        return Workload("c5", 5, 64, 4, 8, 256, 128, n, tuple(ratio_budget(x) for x in n), "bf16", "mixture",
                        "cluster", paged=True, block_size=16, table="permuted", max_blocks=8192)
    raise KeyError(name)


def custom(name: str = "custom", cfg_id: int = 100, **kw) -> Workload:
    """A small workload for tests; unspecified fields default to a 1x1 f32 normal case."""
    base = Workload(name, cfg_id, 1, 1, 1, 4, 128, (64,), (13,), "f32", "normal", "normal")
    w = replace(base, **kw)
    if "m" not in kw:
        w = replace(w, m=tuple(ratio_budget(x) for x in w.n))
    if w.paged and w.max_blocks == 0:
        w = replace(w, max_blocks=max(w.blocks_of(s) for s in range(w.S)))
    return w


def _store(w: Workload, x: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(x) if w.dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _mixture_means(w: Workload, s: int, h: int) -> np.ndarray:
    return _rng(w.cfg_id, s, h, T_CLUSTERS).standard_normal((NUM_CLUSTERS, w.d), dtype=np.float32)


def _mixture_assign(w: Workload, s: int, h: int) -> np.ndarray:
    return _rng(w.cfg_id, s, h, T_ASSIGN).integers(0, NUM_CLUSTERS, size=w.n[s])


def _keys_f32(w: Workload, s: int, h: int) -> np.ndarray:
    n, d = w.n[s], w.d
    if w.keys == "normal":
        return _rng(w.cfg_id, s, h, T_KEYS).standard_normal((n, d), dtype=np.float32)
    if w.keys == "mixture":
        mu = _mixture_means(w, s, h)
        a = _mixture_assign(w, s, h)
        k = _rng(w.cfg_id, s, h, T_KEYNOISE).standard_normal((n, d), dtype=np.float32)
        k *= np.float32(0.5)
        k += mu[a]
        k[:NUM_SINKS] *= np.float32(SINK_GAIN)
        return k
    raise ValueError(w.keys)


def unit_keys(w: Workload, s: int, h: int) -> np.ndarray:
    """Stored keys of unit (s, h): [n_s][d] float32 or bfloat16 bits."""
    return _store(w, _keys_f32(w, s, h))


def unit_values(w: Workload, s: int, h: int) -> np.ndarray:
    return _store(w, _rng(w.cfg_id, s, h, T_VALUES).standard_normal((w.n[s], w.d), dtype=np.float32))


def action_positions(w: Workload, s: int) -> np.ndarray:
    """Positions of the q action-token queries: NUM_SPANS disjoint spans at seeded starts."""
    n, L = w.n[s], w.q // NUM_SPANS
    assert L * NUM_SPANS == w.q and n >= NUM_SINKS + L * NUM_SPANS
    g = _rng(w.cfg_id, s, 0, T_SPANS)
    while True:
        starts = np.sort(g.integers(NUM_SINKS, n - L, size=NUM_SPANS, endpoint=True))
        if np.all(np.diff(starts) >= L):
            break
    return np.concatenate([np.arange(a, a + L) for a in starts])


def row_positions(w: Workload, kind: str = "action") -> np.ndarray:
    """Causal positions of the proxy rows, int32 [S][H*G][q]: row r of a unit sees the keys at
    segment positions j <= its entry. "action": each action-token query sits at its own position
    in the trajectory (every query head of every KV head shares them); "spread": seeded uniform
    over [-2, n + 1] per row (rows that see no key, rows that see every key, and all between);
    "all": n - 1 (every row sees every key); "none": -1 (no row sees any key)."""
    out = np.zeros((w.S, w.H * w.G, w.q), dtype=np.int32)
    for s in range(w.S):
        n = w.n[s]
        if kind == "action":
            out[s] = action_positions(w, s)[None, :]
        elif kind == "spread":
            out[s] = _rng(w.cfg_id, s, 0, T_POSITIONS).integers(-2, n + 1, size=(w.H * w.G, w.q), endpoint=True)
        elif kind == "all":
            out[s] = n - 1
        elif kind == "none":
            out[s] = -1
        else:
            raise ValueError(kind)
    return out


def unit_queries(w: Workload, s: int, h: int) -> np.ndarray:
    """Stored proxy queries of the G query heads of KV head h: [G*q][d] (head-major)."""
    R, d = w.R, w.d
    z = _rng(w.cfg_id, s, h, T_QUERIES).standard_normal((R, d), dtype=np.float32)
    if w.queries in ("normal", "boundary"):
        pass
    elif w.queries == "cluster":
        c = _rng(w.cfg_id, s, h, T_QCLUSTER).integers(0, NUM_CLUSTERS, size=R)
        z += np.float32(0.5) * _mixture_means(w, s, h)[c]
    elif w.queries == "action":
        pos = action_positions(w, s)
        a = _mixture_assign(w, s, h)
        c = np.tile(a[pos], w.G)
        z += np.float32(0.5) * _mixture_means(w, s, h)[c]
    else:
        raise ValueError(w.queries)
    return _store(w, z)


def bias_row(w: Workload, s: int) -> np.ndarray | None:
    """Per-key additive logit bias of sequence s ([n_s] float32), or None."""
    if not w.bias_tail:
        return None
    n = w.n[s]
    b = np.zeros(n, dtype=np.float32)
    b[n - n // 4:] = np.float32(w.bias_tail)
    return b


def block_tables(w: Workload) -> tuple[np.ndarray, int]:
    """Block table [S][max_blocks] int32 (unused entries -1) and the pool's block count."""
    nb = [w.blocks_of(s) for s in range(w.S)]
    total = int(sum(nb))
    ids = np.arange(total, dtype=np.int32)
    if w.table == "permuted":
        ids = _rng(w.cfg_id, 0, 0, T_PERM).permutation(total).astype(np.int32)
    elif w.table != "identity":
        raise ValueError(w.table)
    mb = w.max_blocks or max(nb)
    t = np.full((w.S, mb), -1, dtype=np.int32)
    off = 0
    for s in range(w.S):
        t[s, :nb[s]] = ids[off:off + nb[s]]
        off += nb[s]
    return t, total


def _shared_zeros(shape, dtype) -> np.ndarray:
    """Zeroed array in an anonymous shared mapping, so forked workers can fill it in place."""
    count = int(np.prod(shape))
    nbytes = count * np.dtype(dtype).itemsize
    mm = mmap.mmap(-1, max(nbytes, 1))
    return np.frombuffer(mm, dtype=dtype, count=count).reshape(shape)


def _run_all(fn, items):
    for x in items:
        fn(x)


def _pfill(fn, items, workers):
    """Run fn over items in forked worker processes that write into shared arrays."""
    if workers <= 1 or len(items) <= 1:
        _run_all(fn, items)
        return
    ctx = multiprocessing.get_context("fork")
    procs = [ctx.Process(target=_run_all, args=(fn, items[i::workers])) for i in range(min(workers, len(items)))]
    for p in procs:
        p.start()
    for p in procs:
        p.join()
    bad = [p.exitcode for p in procs if p.exitcode != 0]
    if bad:
        raise RuntimeError(f"input generation worker failed with exit codes {bad}")


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _storage_dtype(w: Workload):
    return np.uint16 if w.dtype == "bf16" else np.float32


def _queries_and_bias(w: Workload, workers: int):
    Q = _shared_zeros((w.S, w.H * w.G, w.q, w.d), _storage_dtype(w))

    def fill(args):
        _, s, h = args
        Q[s, h * w.G:(h + 1) * w.G] = unit_queries(w, s, h).reshape(w.G, w.q, w.d)

    _pfill(fill, [(w, s, h) for s in range(w.S) for h in range(w.H)], workers)
    bias = None
    if w.bias_tail:
        bias = np.zeros((w.S, w.n_max), dtype=np.float32)
        for s in range(w.S):
            bias[s, :w.n[s]] = bias_row(w, s)
    return Q, bias


def build_contiguous(w: Workload, workers: int = 1) -> dict:
    """Contiguous layout: K, V [S][H][n_max][d]; Q [S][H*G][q][d]; bias [S][n_max] or None."""
    dt = _storage_dtype(w)
    K = _shared_zeros((w.S, w.H, w.n_max, w.d), dt)
    V = _shared_zeros((w.S, w.H, w.n_max, w.d), dt)

    def fill(args):
        _, s, h = args
        K[s, h, :w.n[s]] = unit_keys(w, s, h)
        V[s, h, :w.n[s]] = unit_values(w, s, h)

    _pfill(fill, [(w, s, h) for s in range(w.S) for h in range(w.H)], workers)
    Q, bias = _queries_and_bias(w, workers)
    return dict(K=K, V=V, Q=Q, bias=bias, n=np.array(w.n, dtype=np.int32), m=np.array(w.m, dtype=np.int32))


def build_paged(w: Workload, workers: int = 1) -> dict:
    """Paged layout: pools [num_blocks][B][H][d], table [S][max_blocks] int32, Q, bias."""
    table, total = block_tables(w)
    B = w.block_size
    dt = _storage_dtype(w)
    k_pool = _shared_zeros((total, B, w.H, w.d), dt)
    v_pool = _shared_zeros((total, B, w.H, w.d), dt)
    def fill(args):
        _, s, h = args
        nb, n = w.blocks_of(s), w.n[s]
        blk = table[s, :nb]
        for pool, x in ((k_pool, unit_keys(w, s, h)), (v_pool, unit_values(w, s, h))):
            xp = np.zeros((nb * B, w.d), dtype=dt)
            xp[:n] = x
            pool[blk, :, h, :] = xp.reshape(nb, B, w.d)

    # units write disjoint (block, head) slices of the pools
    _pfill(fill, [(w, s, h) for s in range(w.S) for h in range(w.H)], workers)
    Q, bias = _queries_and_bias(w, workers)
    return dict(k_pool=k_pool, v_pool=v_pool, table=table, Q=Q, bias=bias,
                n=np.array(w.n, dtype=np.int32), m=np.array(w.m, dtype=np.int32))


def score_rows(seed: int, lens, kind: str, n_max: int | None = None) -> np.ndarray:
    """Synthetic non-negative float32 score rows [len(lens)][n_max] for exercising selection on
    its own (zeros past each length). kind: "uniform" (U[0, 1)), "levels" (8 distinct values,
    heavy ties), "zeros" (70 % exact zeros, the rest U[0, 1)), "tiny" (subnormal and normal
    values spanning 2^-149 .. 1), "narrow" (all within one binade, [0.5, 0.5 + 2^-12))."""
    n_max = int(n_max or max(lens))
    out = np.zeros((len(lens), n_max), dtype=np.float32)
    for s, n in enumerate(lens):
        rng = _rng(900, s, seed, 50)
        if kind == "uniform":
            x = rng.random(n, dtype=np.float32)
        elif kind == "levels":
            x = rng.integers(0, 8, n).astype(np.float32) / 8.0
        elif kind == "zeros":
            x = np.where(rng.random(n) < 0.7, 0.0, rng.random(n)).astype(np.float32)
        elif kind == "tiny":
            bits = rng.integers(1, 0x3F800000, n, dtype=np.uint32)
            x = bits.view(np.float32)
        elif kind == "narrow":
            x = (0.5 + rng.random(n) * 2.0 ** -12).astype(np.float32)
        else:
            raise ValueError(kind)
        out[s, :n] = x
    return out


def device_normal_bf16(shape, seed: int, device="cuda", chunk_rows: int = 1 << 20):
    """Standard normal values rounded to bfloat16 (round to nearest even), generated on the device
    by torch's seeded generator: for inputs of several GiB that the host could not generate in a
    test's time. The leading axes are filled `chunk_rows` rows at a time to bound the float32
    staging; the values are fixed by the seed, the shape, `chunk_rows` and the device type."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1, shape[-1])
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(r0 + chunk_rows, flat.shape[0])
        flat[r0:r1] = torch.randn((r1 - r0, shape[-1]), generator=g, device=device, dtype=torch.float32)
    return out
