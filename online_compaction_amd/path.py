"""The whole hot path over one batch: score -> select -> compact, through the C ABI.

Torch only provides device memory and the stream. `Batch` holds device-resident inputs,
`Outputs` the preallocated outputs and workspace, and `run` enqueues kvc_score,
kvc_select_topm and kvc_compact_contig / kvc_compact_paged on the current stream.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import _abi as A


def device_tensor(arr: np.ndarray, device="cuda") -> torch.Tensor:
    """Upload a numpy array; uint16 arrays are bfloat16 bit patterns."""
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(arr).to(device)


def host_array(t: torch.Tensor) -> np.ndarray:
    """Download a tensor; bfloat16 comes back as uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@dataclass
class Batch:
    shape: A.Shape
    dtype: int
    q: torch.Tensor
    m: np.ndarray
    m_max: int
    k: torch.Tensor = None            # contiguous [S][H][n_max][d]
    v: torch.Tensor = None
    k_pool: torch.Tensor = None       # paged [num_blocks][B][H][d]
    v_pool: torch.Tensor = None
    table: torch.Tensor = None        # paged [S][max_blocks] int32
    block_size: int = 0
    max_blocks: int = 0
    bias: torch.Tensor = None
    lse: torch.Tensor = None          # supplied LSE [S][H*G][q] or None
    cache_lens: np.ndarray = None     # paged: total length of each sequence (segment compaction)

    @property
    def paged(self) -> bool:
        return self.block_size != 0

    def kview(self) -> A.KView:
        if self.paged:
            return A.KView(self.k_pool, self.dtype, self.block_size, self.table, self.max_blocks)
        return A.KView(self.k, self.dtype)


def _dtype_of(arr: np.ndarray) -> int:
    return A.KVC_BF16 if arr.dtype == np.uint16 else A.KVC_F32


def contiguous_batch(Q, K, V, n, m, group: int, scale: float, bias=None, lse=None, starts=None,
                     device="cuda") -> Batch:
    """Score/select/gather n[s] keys of each sequence, starting at cache row starts[s] (default 0)."""
    S, H, n_max, d = K.shape
    q = Q.shape[2]
    shape = A.Shape(S, H, group, q, d, n_max, np.asarray(n, dtype=np.int32), scale, starts)
    m = np.asarray(m, dtype=np.int32)
    return Batch(shape, _dtype_of(K), device_tensor(Q, device), m, max(1, int(m.max())),
                 k=device_tensor(K, device), v=device_tensor(V, device),
                 bias=None if bias is None else device_tensor(np.asarray(bias, dtype=np.float32), device),
                 lse=None if lse is None else device_tensor(np.asarray(lse, dtype=np.float32), device))


def paged_batch(Q, k_pool, v_pool, table, n, m, group: int, scale: float, block_size: int, n_max=None, bias=None,
                lse=None, starts=None, cache_lens=None, device="cuda") -> Batch:
    """Paged pool; n[s] keys scored from logical position starts[s] (default 0) of a sequence whose
    total length is cache_lens[s] (default starts[s] + n[s])."""
    S, max_blocks = table.shape
    H, d = k_pool.shape[2], k_pool.shape[3]
    q = Q.shape[2]
    n = np.asarray(n, dtype=np.int32)
    n_max = int(n_max if n_max is not None else (bias.shape[1] if bias is not None else n.max()))
    shape = A.Shape(S, H, group, q, d, n_max, n, scale, starts)
    m = np.asarray(m, dtype=np.int32)
    return Batch(shape, _dtype_of(k_pool), device_tensor(Q, device), m, max(1, int(m.max())),
                 k_pool=device_tensor(k_pool, device), v_pool=device_tensor(v_pool, device),
                 table=device_tensor(np.asarray(table, dtype=np.int32), device), block_size=block_size,
                 max_blocks=max_blocks,
                 bias=None if bias is None else device_tensor(np.asarray(bias, dtype=np.float32), device),
                 lse=None if lse is None else device_tensor(np.asarray(lse, dtype=np.float32), device),
                 cache_lens=None if cache_lens is None else np.asarray(cache_lens, dtype=np.int32))


@dataclass
class Outputs:
    scores: torch.Tensor
    kept: torch.Tensor
    ws: torch.Tensor = None
    k_out: torch.Tensor = None
    v_out: torch.Tensor = None
    freed: torch.Tensor = None
    freed_counts: np.ndarray = field(default=None)


def allocate(b: Batch) -> Outputs:
    sh = b.shape
    dev = b.q.device
    scores = torch.zeros((sh.num_seqs, sh.num_kv_heads, sh.n_max), dtype=torch.float32, device=dev)
    kept = torch.full((sh.num_seqs, sh.num_kv_heads, b.m_max), -1, dtype=torch.int32, device=dev)
    wsb = A.kvc_score_workspace_size(sh, b.kview(), b.lse is not None)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev) if wsb else None
    out = Outputs(scores, kept, ws)
    if b.paged:
        out.freed = torch.full((sh.num_seqs, b.max_blocks), -1, dtype=torch.int32, device=dev)
    else:
        el = b.k.dtype
        out.k_out = torch.zeros((sh.num_seqs, sh.num_kv_heads, b.m_max, sh.head_dim), dtype=el, device=dev)
        out.v_out = torch.zeros_like(out.k_out)
    return out


def run_score(b: Batch, o: Outputs, stream=None) -> None:
    A.kvc_score(b.shape, b.q, b.kview(), b.lse, b.bias, o.scores, o.ws, stream)


def run_select(b: Batch, o: Outputs, stream=None) -> None:
    A.kvc_select_topm(b.shape, o.scores, b.m, b.m_max, o.kept, stream)


def run_compact(b: Batch, o: Outputs, stream=None) -> None:
    if b.paged:
        o.freed_counts = A.kvc_compact_paged(b.shape, b.dtype, b.k_pool, b.v_pool, b.block_size, b.table,
                                             b.max_blocks, o.kept, b.m, b.m_max, o.freed, b.cache_lens, stream)
    else:
        A.kvc_compact_contig(b.shape, b.dtype, b.k, b.v, o.kept, b.m, b.m_max, o.k_out, o.v_out, stream)


def run(b: Batch, o: Outputs, stream=None) -> None:
    """One pass of the hot path over the batch (asynchronous on the stream)."""
    run_score(b, o, stream)
    run_select(b, o, stream)
    run_compact(b, o, stream)


# ------------------------------------------------------------------------ ActKV retention stages

@dataclass
class Retention:
    """Per-entry LRFU state of a batch and the buffers of one retention step."""
    state: torch.Tensor        # float32 [S][H][n_max]
    mass: torch.Tensor         # float32 [S][H][n_max]
    side: torch.Tensor         # float32 [S][H][m_max], the state carried through compaction
    counts: torch.Tensor       # int32 [S][H], critical-set sizes
    top_p: float = 0.9
    decay: float = 2.0 ** -0.5


def allocate_retention(b: Batch, state=None) -> Retention:
    sh = b.shape
    dev = b.q.device
    full = (sh.num_seqs, sh.num_kv_heads, sh.n_max)
    st = torch.zeros(full, dtype=torch.float32, device=dev) if state is None else device_tensor(state, dev)
    return Retention(st, torch.zeros(full, dtype=torch.float32, device=dev),
                     torch.zeros((sh.num_seqs, sh.num_kv_heads, b.m_max), dtype=torch.float32, device=dev),
                     torch.zeros((sh.num_seqs, sh.num_kv_heads), dtype=torch.int32, device=dev))


def run_retention_score(b: Batch, o: Outputs, r: Retention, stream=None) -> None:
    """The attention the proxy (action) rows pay each entry."""
    A.kvc_attention_mass(b.shape, b.q, b.kview(), b.lse, b.bias, r.mass, o.ws, stream)


def run_retention_select(b: Batch, o: Outputs, r: Retention, stream=None) -> None:
    """Action-critical set + LRFU step, then the budget's largest LRFU values."""
    A.kvc_lrfu_update(b.shape, r.mass, r.top_p, r.decay, r.state, r.counts, stream)
    A.kvc_select_topm(b.shape, r.state, b.m, b.m_max, o.kept, stream)


def run_retention_compact(b: Batch, o: Outputs, r: Retention, stream=None) -> None:
    """K/V compaction, with the LRFU state carried along into r.side."""
    run_compact(b, o, stream)
    A.kvc_compact_side(b.shape, b.block_size if b.paged else 0, o.kept, b.m, b.m_max, r.state, r.side, stream)


# ------------------------------------------------------------------------ Attention Matching stage

@dataclass
class Matching:
    """Attention Matching outputs of a batch (bias beta and compact values V_C per kept key) and
    the fit's workspace; K_C is the kept keys, gathered by the compaction stage."""
    beta: torch.Tensor         # float32 [S][H][m_max]
    v_c: torch.Tensor          # float32 [S][H][m_max][d]
    ws: torch.Tensor
    iters_beta: int
    iters_v: int


def _value_view(b: Batch) -> A.KView:
    if b.paged:
        return A.KView(b.v_pool, b.dtype, b.block_size, b.table, b.max_blocks)
    return A.KView(b.v, b.dtype)


def allocate_matching(b: Batch, iters_beta: int, iters_v: int) -> Matching:
    sh = b.shape
    dev = b.q.device
    wsb = A.kvc_am_workspace_size(sh, b.kview(), _value_view(b), b.m, b.lse is not None)
    return Matching(torch.zeros((sh.num_seqs, sh.num_kv_heads, b.m_max), dtype=torch.float32, device=dev),
                    torch.zeros((sh.num_seqs, sh.num_kv_heads, b.m_max, sh.head_dim), dtype=torch.float32,
                                device=dev),
                    torch.empty(max(256, wsb), dtype=torch.uint8, device=dev), iters_beta, iters_v)


def run_matching(b: Batch, o: Outputs, am: Matching, stream=None) -> None:
    """Fit beta and V_C for the kept keys o.kept (before a paged compaction rewrites the pool)."""
    A.kvc_am_fit(b.shape, b.q, b.kview(), _value_view(b), b.lse, o.kept, b.m, b.m_max, am.iters_beta, am.iters_v,
                 am.beta, am.v_c, am.ws, stream)
