"""Proxy-query Token Eviction (score -> select -> compact) on AMD Instinct MI355X.

The work runs in libkvc.so (hand-written HIP kernels for gfx950 behind the C ABI of
include/kvc.h); this package only binds it (``_abi``) and builds it (``build``).
"""
from ._abi import (  # noqa: F401
    KVC_BF16,
    KVC_F32,
    KvcError,
    KView,
    Shape,
    kvc_am_fit,
    kvc_am_workspace_size,
    kvc_attention_mass,
    kvc_compact_contig,
    kvc_compact_paged,
    kvc_compact_side,
    kvc_evict_redirect,
    kvc_lse,
    kvc_lrfu_update,
    kvc_lse_workspace_size,
    kvc_score,
    kvc_score_noalloc,
    kvc_score_workspace_size,
    kvc_select_topm,
    kvc_status_string,
    kvc_version,
    load,
)
