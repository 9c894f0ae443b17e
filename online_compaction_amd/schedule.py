"""Delayed future-turn compaction of an agent session held in a paged KV cache.

"Practical Online KV Cache Compaction for LLM Agents", section on the proxy-query sources (delayed
future-turn queries) and the finding that one turn of delay recovers most of the accuracy lost by
immediate compaction: turn t is kept raw for k turns; at the end of turn t + k it is scored with
the queries the model produced during turns t+1 .. t+k, compacted to its top positions with
their original K/V, and frozen. The compaction itself is the library's segment path
(kvc_score / kvc_select_topm / kvc_compact_paged with a segment start), i.e. ActKV's
conflict-free slot plan applied to the turn's own blocks; the freed blocks go back to this
object's free list.

Host policy only (which turn, which queries, which budget); every step on the data runs in
libkvc. Reading of the pages used here: a turn is compacted over the whole blocks inside it
(its first block starts at or after the turn start, its last ends at or before the turn end);
the keep budget round(ratio * n) is rounded up to whole blocks so the compacted turn stays
dense and later turns only change block-table entries.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import _abi as A


@dataclass
class Turn:
    start: int                    # cache position of the turn's first token
    length: int                   # tokens in the cache
    queries: torch.Tensor         # proxy rows produced during the turn: [H*G][q_t][d], K's dtype
    compacted: bool = False


@dataclass
class Compaction:
    turn: int
    start: int                    # segment start (cache position)
    n: int                        # keys scored
    m: int                        # kept
    cache_len: int                # sequence length before
    freed: list                   # physical blocks returned
    scores: torch.Tensor          # [1][H][n]
    kept: torch.Tensor            # [1][H][m]


@dataclass
class DelayedCompactor:
    """One session (sequence) of one layer's paged pool [num_blocks][B][H][d]."""
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    table: torch.Tensor           # device int32 [1][max_blocks]
    block_size: int
    num_kv_heads: int
    group: int
    scale: float
    delay: int = 1
    ratio: float = 0.2
    turns: list = field(default_factory=list)
    length: int = 0               # tokens in the cache
    free_blocks: list = field(default_factory=list)

    @property
    def dtype(self) -> int:
        return A.KVC_BF16 if self.k_pool.dtype == torch.bfloat16 else A.KVC_F32

    def budget(self, n: int) -> int:
        """Keep ratio, rounded to the nearest token, then up to whole blocks (at most n)."""
        B = self.block_size
        m = int(np.floor(self.ratio * n + 0.5))
        return min(n, -(-m // B) * B)

    def append_turn(self, num_tokens: int, queries: torch.Tensor) -> list:
        """Register a finished turn whose K/V the engine has written at cache positions
        [length, length + num_tokens); compact the turn that is now `delay` turns old."""
        self.turns.append(Turn(self.length, num_tokens, queries))
        self.length += num_tokens
        done = []
        t = len(self.turns) - 1 - self.delay
        if t >= 0 and not self.turns[t].compacted:
            c = self._compact(t)
            if c is not None:
                done.append(c)
        return done

    def _compact(self, t: int):
        B = self.block_size
        turn = self.turns[t]
        turn.compacted = True
        a = -(-turn.start // B) * B
        e = (turn.start + turn.length) // B * B
        n = e - a
        if n <= 0:
            return None
        m = self.budget(n)
        # proxy rows: every query of the turns that followed, per query head
        q = torch.cat([self.turns[u].queries for u in range(t + 1, t + 1 + self.delay)], dim=1).contiguous()
        H, G, d = self.num_kv_heads, self.group, q.shape[-1]
        shape = A.Shape(1, H, G, q.shape[1], d, n, np.array([n], dtype=np.int32), self.scale,
                        np.array([a], dtype=np.int32))
        kv = A.KView(self.k_pool, self.dtype, B, self.table, self.table.shape[1])
        dev = self.k_pool.device
        scores = torch.empty((1, H, n), dtype=torch.float32, device=dev)
        wsb = A.kvc_score_workspace_size(shape, kv, False)
        ws = torch.empty(max(256, wsb), dtype=torch.uint8, device=dev)
        A.kvc_score(shape, q.unsqueeze(0), kv, None, None, scores, ws)
        kept = torch.empty((1, H, max(m, 1)), dtype=torch.int32, device=dev)
        A.kvc_select_topm(shape, scores, [m], max(m, 1), kept)
        freed = torch.full((1, self.table.shape[1]), -1, dtype=torch.int32, device=dev)
        L = self.length
        counts = A.kvc_compact_paged(shape, self.dtype, self.k_pool, self.v_pool, B, self.table,
                                     self.table.shape[1], kept, [m], max(m, 1), freed, [L])
        F = int(counts[0])
        freed_ids = freed[0, :F].cpu().tolist()
        self.free_blocks.extend(freed_ids)
        # the turn shrinks by F blocks and every later turn slides down with the table entries
        turn.length -= F * B
        for u in range(t + 1, len(self.turns)):
            self.turns[u].start -= F * B
        self.length -= F * B
        return Compaction(t, a, n, m, L, freed_ids, scores, kept[:, :, :m])
