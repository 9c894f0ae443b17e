"""Thin ctypes binding of libkvc (include/kvc.h): the same entry points, argument marshalling only.

Tensors are torch tensors on the GPU (torch supplies device memory and the current HIP
stream); host arrays are anything numpy can turn into int32. Every step of the computation
runs in the HIP kernels of libkvc.so; if the library is missing this module raises instead of
falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

KVC_OK, KVC_ERR_INVALID_ARGUMENT, KVC_ERR_UNSUPPORTED, KVC_ERR_WORKSPACE_TOO_SMALL, KVC_ERR_HIP = range(5)
KVC_F32, KVC_BF16 = 0, 1
KVC_NOALLOC_SCRATCH_BYTES = 64 << 20  # the static scratch of kvc_score_noalloc (kvc.h)


class KvcError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: status {status}: {detail}")


class _Shape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("group", ctypes.c_int32),
                ("num_queries", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("n_max", ctypes.c_int32),
                ("seq_lens", ctypes.POINTER(ctypes.c_int32)), ("scale", ctypes.c_float),
                ("seq_starts", ctypes.POINTER(ctypes.c_int32)), ("row_pos", ctypes.c_void_p)]


class _KView(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int), ("block_size", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32), ("slot_map", ctypes.c_void_p),
                ("dead_slot", ctypes.c_int32)]


_lib = None

_SIGS = {
    "kvc_lse_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(_Shape), ctypes.POINTER(_KView)]),
    "kvc_lse": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.c_void_p, ctypes.POINTER(_KView), ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "kvc_score_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(_Shape), ctypes.POINTER(_KView), ctypes.c_int]),
    "kvc_score": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.c_void_p, ctypes.POINTER(_KView), ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p]),
    "kvc_score_noalloc": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.c_void_p, ctypes.POINTER(_KView),
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "kvc_attention_mass": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.c_void_p, ctypes.POINTER(_KView),
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p]),
    "kvc_am_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(_Shape), ctypes.POINTER(_KView), ctypes.POINTER(_KView),
                                                ctypes.POINTER(ctypes.c_int32), ctypes.c_int]),
    "kvc_am_fit": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.c_void_p, ctypes.POINTER(_KView),
                                  ctypes.POINTER(_KView), ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]),
    "kvc_evict_redirect": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32),
                                          ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    "kvc_lrfu_update": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.c_void_p, ctypes.c_double, ctypes.c_float,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "kvc_compact_side": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]),
    "kvc_select_topm": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32),
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]),
    "kvc_compact_contig": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "kvc_compact_paged": (ctypes.c_int, [ctypes.POINTER(_Shape), ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.POINTER(ctypes.c_int32), ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p,
                                         ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p]),
    "kvc_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kvc_last_error": (ctypes.c_char_p, []),
    "kvc_version": (ctypes.c_int, []),
}


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libkvc.so (built by online_compaction_amd.build, or the file named by $KVC_LIB);
    raises if it is not there."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("KVC_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libkvc.so not built at {p}: run `python -m online_compaction_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


@dataclass
class Shape:
    num_seqs: int
    num_kv_heads: int
    group: int
    num_queries: int
    head_dim: int
    n_max: int
    seq_lens: object  # host ints [S]: keys scored per sequence
    scale: float
    seq_starts: object = None  # host ints [S]: cache position of each sequence's first scored key
    row_pos: object = None     # device int32 tensor [S][H*G][q]: causal mask, row sees keys j <= row_pos

    def c(self):
        lens = np.ascontiguousarray(np.asarray(self.seq_lens, dtype=np.int32))
        starts = None
        if self.seq_starts is not None:
            starts = np.ascontiguousarray(np.asarray(self.seq_starts, dtype=np.int32))
        if self.row_pos is not None and not isinstance(self.row_pos, int):
            if str(self.row_pos.dtype) != "torch.int32":
                raise ValueError(f"row_pos: int32 tensor required, got {self.row_pos.dtype}")
            _need(self.row_pos, self.num_seqs * self.num_kv_heads * self.group * self.num_queries * 4, "row_pos")
        rp = _ptr(self.row_pos)
        # the struct of the previous call is reused while every field holds the same values (numpy's
        # ctypes pointers cost a few microseconds per call)
        key = (self.num_seqs, self.num_kv_heads, self.group, self.num_queries, self.head_dim, self.n_max,
               lens.tobytes(), None if starts is None else starts.tobytes(), float(self.scale), rp)
        hit = self.__dict__.get("_c_cached")
        if hit is not None and hit[0] == key:
            return hit[1], hit[2]
        sp = None if starts is None else starts.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        sh = _Shape(self.num_seqs, self.num_kv_heads, self.group, self.num_queries, self.head_dim, self.n_max,
                    lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), float(self.scale), sp, rp)
        keep = (lens, starts)  # keeps the arrays alive while `sh` is used
        self.__dict__["_c_cached"] = (key, sh, keep)
        return sh, keep


@dataclass
class KView:
    data: object          # device tensor
    dtype: int            # KVC_F32 | KVC_BF16
    block_size: int = 0
    block_table: object = None  # device int32 tensor [S][max_blocks] (paged)
    max_blocks: int = 0
    slot_map: object = None     # device int32 tensor [S][H][n_max] (slot pool [slots][H][d])
    dead_slot: int = -1

    def c(self):
        return _KView(_ptr(self.data), int(self.dtype), int(self.block_size), _ptr(self.block_table),
                      int(self.max_blocks), _ptr(self.slot_map), int(self.dead_slot))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("libkvc takes device tensors; got a host tensor")
    if not t.is_contiguous():
        raise ValueError("libkvc takes contiguous tensors")
    return t.data_ptr()


def _need(t, nbytes: int, what: str):
    """Refuse buffers smaller than the layout the call will touch (a kernel cannot check)."""
    if t is None:
        return
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{what}: {have} bytes < {nbytes} required")


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)  # the handle without a Stream object
    if raw is not None:
        return raw(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _host_i32(a):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _check(status: int, func: str):
    if status != KVC_OK:
        raise KvcError(status, func, load().kvc_last_error().decode())


def _elt(dtype: int) -> int:
    return 4 if dtype == KVC_F32 else 2


def _check_kview(shape: Shape, kv: KView):
    S, H, d = shape.num_seqs, shape.num_kv_heads, shape.head_dim
    if kv.slot_map is not None:
        _need(kv.slot_map, S * H * shape.n_max * 4, "slot_map")
    elif kv.block_size == 0:
        _need(kv.data, S * H * shape.n_max * d * _elt(kv.dtype), "k")
    else:
        _need(kv.block_table, S * kv.max_blocks * 4, "block_table")


def kvc_lse_workspace_size(shape: Shape, k: KView) -> int:
    sh, _keep = shape.c()
    kv = k.c()
    return int(load().kvc_lse_workspace_size(ctypes.byref(sh), ctypes.byref(kv)))


def kvc_score_workspace_size(shape: Shape, k: KView, lse_supplied: bool) -> int:
    sh, _keep = shape.c()
    kv = k.c()
    return int(load().kvc_score_workspace_size(ctypes.byref(sh), ctypes.byref(kv), int(bool(lse_supplied))))


def kvc_lse(shape: Shape, q, k: KView, bias, lse_out, ws, stream=None) -> None:
    S, HG, R = shape.num_seqs, shape.num_kv_heads * shape.group, shape.num_queries
    _need(q, S * HG * R * shape.head_dim * _elt(k.dtype), "q")
    _check_kview(shape, k)
    _need(bias, S * shape.n_max * 4, "bias")
    _need(lse_out, S * HG * R * 4, "lse_out")
    sh, _keep = shape.c()
    kv = k.c()
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().kvc_lse(ctypes.byref(sh), _ptr(q), ctypes.byref(kv), _ptr(bias), _ptr(lse_out), _ptr(ws),
                          ws_bytes, _stream(stream)), "kvc_lse")


def kvc_score(shape: Shape, q, k: KView, lse, bias, scores, ws=None, stream=None) -> None:
    S, H, HG, R = shape.num_seqs, shape.num_kv_heads, shape.num_kv_heads * shape.group, shape.num_queries
    _need(q, S * HG * R * shape.head_dim * _elt(k.dtype), "q")
    _check_kview(shape, k)
    _need(lse, S * HG * R * 4, "lse")
    _need(bias, S * shape.n_max * 4, "bias")
    _need(scores, S * H * shape.n_max * 4, "scores")
    sh, _keep = shape.c()
    kv = k.c()
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().kvc_score(ctypes.byref(sh), _ptr(q), ctypes.byref(kv), _ptr(lse), _ptr(bias), _ptr(scores),
                            _ptr(ws), ws_bytes, _stream(stream)), "kvc_score")


def kvc_score_noalloc(shape: Shape, q, k: KView, lse, bias, scores, stream=None) -> None:
    S, H, HG, R = shape.num_seqs, shape.num_kv_heads, shape.num_kv_heads * shape.group, shape.num_queries
    _need(q, S * HG * R * shape.head_dim * _elt(k.dtype), "q")
    _check_kview(shape, k)
    _need(lse, S * HG * R * 4, "lse")
    _need(bias, S * shape.n_max * 4, "bias")
    _need(scores, S * H * shape.n_max * 4, "scores")
    sh, _keep = shape.c()
    kv = k.c()
    _check(load().kvc_score_noalloc(ctypes.byref(sh), _ptr(q), ctypes.byref(kv), _ptr(lse), _ptr(bias),
                                    _ptr(scores), _stream(stream)), "kvc_score_noalloc")


def kvc_attention_mass(shape: Shape, q, k: KView, lse, bias, mass, ws=None, stream=None) -> None:
    S, H, HG, R = shape.num_seqs, shape.num_kv_heads, shape.num_kv_heads * shape.group, shape.num_queries
    _need(q, S * HG * R * shape.head_dim * _elt(k.dtype), "q")
    _check_kview(shape, k)
    _need(lse, S * HG * R * 4, "lse")
    _need(bias, S * shape.n_max * 4, "bias")
    _need(mass, S * H * shape.n_max * 4, "mass")
    sh, _keep = shape.c()
    kv = k.c()
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().kvc_attention_mass(ctypes.byref(sh), _ptr(q), ctypes.byref(kv), _ptr(lse), _ptr(bias),
                                     _ptr(mass), _ptr(ws), ws_bytes, _stream(stream)), "kvc_attention_mass")


def kvc_am_workspace_size(shape: Shape, k: KView, v: KView, m, lse_supplied: bool) -> int:
    sh, _keep = shape.c()
    kv, vv = k.c(), v.c()
    marr, mp = _host_i32(m)
    return int(load().kvc_am_workspace_size(ctypes.byref(sh), ctypes.byref(kv), ctypes.byref(vv), mp,
                                            int(bool(lse_supplied))))


def kvc_am_fit(shape: Shape, q, k: KView, v: KView, lse, kept, m, m_max: int, iters_beta: int, iters_v: int,
               beta, v_c, ws, stream=None) -> None:
    S, H, HG, R = shape.num_seqs, shape.num_kv_heads, shape.num_kv_heads * shape.group, shape.num_queries
    _need(q, S * HG * R * shape.head_dim * 2, "q")
    _check_kview(shape, k)
    _check_kview(shape, v)
    _need(lse, S * HG * R * 4, "lse")
    _need(kept, S * H * m_max * 4, "kept")
    _need(beta, S * H * m_max * 4, "beta")
    _need(v_c, S * H * m_max * shape.head_dim * 4, "v_c")
    sh, _keep = shape.c()
    kv, vv = k.c(), v.c()
    marr, mp = _host_i32(m)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().kvc_am_fit(ctypes.byref(sh), _ptr(q), ctypes.byref(kv), ctypes.byref(vv), _ptr(lse), _ptr(kept),
                             mp, int(m_max), int(iters_beta), int(iters_v), _ptr(beta), _ptr(v_c), _ptr(ws),
                             ws_bytes, _stream(stream)), "kvc_am_fit")


def kvc_evict_redirect(shape: Shape, kept, m, m_max: int, slot_map, dead_slot: int, stream=None) -> None:
    S, H = shape.num_seqs, shape.num_kv_heads
    _need(kept, S * H * m_max * 4, "kept")
    _need(slot_map, S * H * shape.n_max * 4, "slot_map")
    sh, _keep = shape.c()
    marr, mp = _host_i32(m)
    _check(load().kvc_evict_redirect(ctypes.byref(sh), _ptr(kept), mp, int(m_max), _ptr(slot_map), int(dead_slot),
                                     _stream(stream)), "kvc_evict_redirect")


def kvc_lrfu_update(shape: Shape, mass, top_p: float, decay: float, state, counts=None, stream=None) -> None:
    S, H = shape.num_seqs, shape.num_kv_heads
    _need(mass, S * H * shape.n_max * 4, "mass")
    _need(state, S * H * shape.n_max * 4, "state")
    _need(counts, S * H * 4, "counts")
    sh, _keep = shape.c()
    _check(load().kvc_lrfu_update(ctypes.byref(sh), _ptr(mass), float(top_p), float(decay), _ptr(state),
                                  _ptr(counts), _stream(stream)), "kvc_lrfu_update")


def kvc_compact_side(shape: Shape, block_size: int, kept, m, m_max: int, src, dst, stream=None) -> None:
    S, H = shape.num_seqs, shape.num_kv_heads
    _need(kept, S * H * m_max * 4, "kept")
    _need(src, S * H * shape.n_max * 4, "src")
    _need(dst, S * H * m_max * 4, "dst")
    sh, _keep = shape.c()
    marr, mp = _host_i32(m)
    _check(load().kvc_compact_side(ctypes.byref(sh), int(block_size), _ptr(kept), mp, int(m_max), _ptr(src),
                                   _ptr(dst), _stream(stream)), "kvc_compact_side")


def kvc_select_topm(shape: Shape, scores, m, m_max: int, kept, stream=None) -> None:
    S, H = shape.num_seqs, shape.num_kv_heads
    _need(scores, S * H * shape.n_max * 4, "scores")
    _need(kept, S * H * m_max * 4, "kept")
    sh, _keep = shape.c()
    marr, mp = _host_i32(m)
    _check(load().kvc_select_topm(ctypes.byref(sh), _ptr(scores), mp, int(m_max), _ptr(kept), _stream(stream)),
           "kvc_select_topm")


def kvc_compact_contig(shape: Shape, dtype: int, k, v, kept, m, m_max: int, k_out, v_out, stream=None) -> None:
    S, H, d = shape.num_seqs, shape.num_kv_heads, shape.head_dim
    for t, nm in ((k, "k"), (v, "v")):
        _need(t, S * H * shape.n_max * d * _elt(dtype), nm)
    for t, nm in ((k_out, "k_out"), (v_out, "v_out")):
        _need(t, S * H * m_max * d * _elt(dtype), nm)
    _need(kept, S * H * m_max * 4, "kept")
    sh, _keep = shape.c()
    marr, mp = _host_i32(m)
    _check(load().kvc_compact_contig(ctypes.byref(sh), int(dtype), _ptr(k), _ptr(v), _ptr(kept), mp, int(m_max),
                                     _ptr(k_out), _ptr(v_out), _stream(stream)), "kvc_compact_contig")


def kvc_compact_paged(shape: Shape, dtype: int, k_pool, v_pool, block_size: int, block_table, max_blocks: int,
                      kept, m, m_max: int, freed_blocks, cache_lens=None, stream=None) -> np.ndarray:
    """Returns freed_counts (host int32 [S])."""
    S, H = shape.num_seqs, shape.num_kv_heads
    _need(block_table, S * max_blocks * 4, "block_table")
    _need(freed_blocks, S * max_blocks * 4, "freed_blocks")
    _need(kept, S * H * m_max * 4, "kept")
    sh, _keep = shape.c()
    marr, mp = _host_i32(m)
    carr, cp = (None, None) if cache_lens is None else _host_i32(cache_lens)
    counts = np.zeros(S, dtype=np.int32)
    _check(load().kvc_compact_paged(ctypes.byref(sh), int(dtype), _ptr(k_pool), _ptr(v_pool), int(block_size),
                                    _ptr(block_table), int(max_blocks), _ptr(kept), mp, int(m_max), cp,
                                    _ptr(freed_blocks), counts.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                    _stream(stream)), "kvc_compact_paged")
    return counts


def kvc_version() -> int:
    return int(load().kvc_version())


def kvc_status_string(status: int) -> str:
    return load().kvc_status_string(int(status)).decode()
