"""ActKV's retention policy on top of the library: action-critical entries feed an LRFU state,
retention keeps the entries with the largest state, and a one-way ratchet sets the budget
("ActKV" analysis page on zhichai.net: the paragraph on the eviction policy and the paragraph
on the adaptive budget).

Host policy only (which budget, when to evict); every step on the data runs in libkvc:
kvc_attention_mass (the attention the action tokens pay each entry), kvc_lrfu_update (the
action-critical set and the LRFU step), kvc_select_topm on the state, kvc_compact_paged for the
K/V and kvc_compact_side to carry the state along.

Readings of the page used here:
  * the attention the action tokens pay an entry is their mean weight on it;
  * "within the top 90 %" is the shortest run of entries, in descending attention, that holds
    90 % of the total attention (the library takes this decision on exact integer masses);
  * LRFU's value decays by 2^-lambda per policy step and a hit adds 1 (lambda = 0.5);
  * budget_k = min(30000, floor(512 * 1.75^k)) after k expansions; it never shrinks. When to
    expand is the model's signal (the page derives it from next-token confidence); the caller
    passes that decision in.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

from . import _abi as A


@dataclass
class BudgetRatchet:
    """One-way budget: starts at `initial` and is multiplied by `factor` (capped) on each
    expansion; it never shrinks."""
    initial: int = 512
    factor: float = 1.75
    cap: int = 30000
    expansions: int = 0

    @property
    def budget(self) -> int:
        return min(self.cap, math.floor(self.initial * self.factor ** self.expansions))

    def expand(self) -> bool:
        """One expansion; False (and no change) once the cap is reached."""
        if self.budget >= self.cap:
            return False
        self.expansions += 1
        return True


@dataclass
class ActKVRetention:
    """One sequence of one layer held in a paged pool [num_blocks][B][H][d] (bf16 or f32)."""
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    table: torch.Tensor              # device int32 [1][max_blocks]
    block_size: int
    num_kv_heads: int
    group: int
    scale: float
    top_p: float = 0.9
    lam: float = 0.5
    ratchet: BudgetRatchet = field(default_factory=BudgetRatchet)
    length: int = 0                  # tokens in the cache
    free_blocks: list = field(default_factory=list)
    state: torch.Tensor | None = None  # device float32 [1][H][max_blocks * B], LRFU value per entry

    def __post_init__(self):
        cap = self.table.shape[1] * self.block_size
        if self.state is None:
            self.state = torch.zeros((1, self.num_kv_heads, cap), dtype=torch.float32, device=self.k_pool.device)

    @property
    def dtype(self) -> int:
        return A.KVC_BF16 if self.k_pool.dtype == torch.bfloat16 else A.KVC_F32

    def _shape(self, n: int, q: int, d: int) -> A.Shape:
        return A.Shape(1, self.num_kv_heads, self.group, q, d, self.state.shape[2], np.array([n], dtype=np.int32),
                       self.scale)

    def step(self, new_tokens: int, action_queries: torch.Tensor, expand: bool = False) -> dict:
        """One policy step: update() then evict()."""
        out = self.update(new_tokens, action_queries, expand)
        out.update(self.evict())
        return out

    def update(self, new_tokens: int, action_queries: torch.Tensor, expand: bool = False) -> dict:
        """The engine has written `new_tokens` more K/V rows at [length, length + new_tokens)
        and produced `action_queries` ([H*G][q][d], K's dtype) in this step. Update the LRFU
        state with their attention over the whole cache; `expand` (the model's signal that
        confidence collapsed during the step) grows the budget once."""
        self.length += new_tokens
        n = self.length
        q, d = action_queries.shape[1], action_queries.shape[2]
        shape = self._shape(n, q, d)
        kv = A.KView(self.k_pool, self.dtype, self.block_size, self.table, self.table.shape[1])
        dev = self.k_pool.device
        mass = torch.empty_like(self.state)
        ws = torch.empty(max(256, A.kvc_score_workspace_size(shape, kv, False)), dtype=torch.uint8, device=dev)
        A.kvc_attention_mass(shape, action_queries.unsqueeze(0).contiguous(), kv, None, None, mass, ws)
        counts = torch.zeros((1, self.num_kv_heads), dtype=torch.int32, device=dev)
        A.kvc_lrfu_update(shape, mass, self.top_p, 2.0 ** -self.lam, self.state, counts)
        grew = self.ratchet.expand() if expand else False
        return {"n": n, "budget": self.ratchet.budget, "grew": grew, "mass": mass, "critical": counts}

    def evict(self) -> dict:
        """Keep the budget's worth of entries with the largest LRFU state (ties to the older
        position) when the cache is larger; the state follows its entries."""
        n, m = self.length, self.ratchet.budget
        if n <= m:
            return {"evicted": False}
        dev = self.k_pool.device
        shape = self._shape(n, 1, self.k_pool.shape[-1])
        kept = torch.empty((1, self.num_kv_heads, m), dtype=torch.int32, device=dev)
        A.kvc_select_topm(shape, self.state, [m], m, kept)
        side = torch.empty((1, self.num_kv_heads, m), dtype=torch.float32, device=dev)
        A.kvc_compact_side(shape, self.block_size, kept, [m], m, self.state, side)
        freed = torch.full((1, self.table.shape[1]), -1, dtype=torch.int32, device=dev)
        F = int(A.kvc_compact_paged(shape, self.dtype, self.k_pool, self.v_pool, self.block_size, self.table,
                                    self.table.shape[1], kept, [m], m, freed)[0])
        self.free_blocks.extend(freed[0, :F].cpu().tolist())
        self.state[:, :, :m] = side
        self.state[:, :, m:] = 0.0
        self.length = m
        return {"evicted": True, "kept": kept, "freed": F}
