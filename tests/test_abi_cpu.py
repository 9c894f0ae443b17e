"""The C-ABI library on the CPU: it loads, exports every declared entry point, sizes workspaces,
and rejects bad arguments before anything is enqueued (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import online_compaction_amd as oc
from online_compaction_amd import _abi as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")

FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(A.LIB_PATH):
        pytest.fail("libkvc.so is not built (run __graft_entry__.build())")
    return A.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"kvc_score", "kvc_lse", "kvc_select_topm", "kvc_compact_contig", "kvc_compact_paged"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(A._SIGS), "binding and header disagree"


def test_version_and_status_strings(lib):
    assert oc.kvc_version() == 300
    assert oc.kvc_status_string(0) == "ok"
    assert oc.kvc_status_string(3) == "workspace too small"
    assert oc.kvc_status_string(99) == "unknown status"


def _shape(S=2, H=8, G=4, q=1024, d=128, n=(33000, 20000), n_max=33000, scale=0.088):
    return A.Shape(S, H, G, q, d, n_max, np.array(n, dtype=np.int32), scale)


def test_workspace_sizes():
    kv = A.KView(FAKE, A.KVC_BF16)
    sh = _shape()
    assert oc.kvc_score_workspace_size(sh, kv, True) == 0
    full = oc.kvc_score_workspace_size(sh, kv, False)
    lse_only = oc.kvc_lse_workspace_size(sh, kv)
    assert full > lse_only > 0 and full % 256 == 0
    # computed LSE needs one float per proxy row on top of the partials
    assert full - lse_only >= 2 * 8 * 4 * 1024 * 4
    # VALU path (float32, 32 rows in two blocks of 16): one partial per row and 64-key chunk (the
    # shortest chunk, since even it gives fewer than 4 workgroups per CU)
    kvf = A.KView(FAKE, A.KVC_F32)
    shf = _shape(S=1, H=1, G=1, q=32, n=(4096,), n_max=4096)
    assert oc.kvc_lse_workspace_size(shf, kvf) == 64 * 32 * 8
    # a score call that computes its LSE also keeps the 32 logits of every key, and the LSE itself
    assert oc.kvc_score_workspace_size(shf, kvf, False) == 64 * 32 * 8 + 4096 * 32 * 4 + 256
    # invalid shapes size to 0
    assert oc.kvc_lse_workspace_size(_shape(d=64), kv) == 0


def _raw_status(fn, *args):
    return fn(*args)


def test_score_validation(lib):
    kv = A.KView(FAKE, A.KVC_BF16).c()
    cases = [
        (_shape(d=64), A.KVC_ERR_UNSUPPORTED),
        (_shape(n=(0, 5)), A.KVC_ERR_INVALID_ARGUMENT),
        (_shape(n=(40000, 5)), A.KVC_ERR_INVALID_ARGUMENT),
        (_shape(G=0), A.KVC_ERR_INVALID_ARGUMENT),
    ]
    for shp, want in cases:
        sh, keep = shp.c()
        st = lib.kvc_score(ctypes.byref(sh), FAKE, ctypes.byref(kv), FAKE, None, FAKE, None, 0, None)
        assert st == want, (shp, st, lib.kvc_last_error())
    sh, keep = _shape().c()
    # NULL scores
    assert lib.kvc_score(ctypes.byref(sh), FAKE, ctypes.byref(kv), FAKE, None, None, None, 0, None) == 1
    # LSE to be computed but no workspace
    st = lib.kvc_score(ctypes.byref(sh), FAKE, ctypes.byref(kv), None, None, FAKE, FAKE, 16, None)
    assert st == A.KVC_ERR_WORKSPACE_TOO_SMALL
    assert b"workspace" in lib.kvc_last_error()
    # unsupported page size, missing table, too few table columns
    for view, want in ((A.KView(FAKE, A.KVC_BF16, 32, FAKE, 4096), A.KVC_ERR_UNSUPPORTED),
                       (A.KView(FAKE, A.KVC_BF16, 16, None, 4096), A.KVC_ERR_INVALID_ARGUMENT),
                       (A.KView(FAKE, A.KVC_BF16, 16, FAKE, 100), A.KVC_ERR_INVALID_ARGUMENT),
                       (A.KView(FAKE, 7), A.KVC_ERR_INVALID_ARGUMENT)):
        v = view.c()
        assert lib.kvc_score(ctypes.byref(sh), FAKE, ctypes.byref(v), FAKE, None, FAKE, None, 0, None) == want


def test_select_and_compact_validation(lib):
    sh, keep = _shape().c()
    m_bad = (ctypes.c_int32 * 2)(40000, 10)
    m_ok = (ctypes.c_int32 * 2)(6600, 4000)
    assert lib.kvc_select_topm(ctypes.byref(sh), FAKE, m_bad, 40000, FAKE, None) == A.KVC_ERR_INVALID_ARGUMENT
    assert lib.kvc_select_topm(ctypes.byref(sh), FAKE, m_ok, 100, FAKE, None) == A.KVC_ERR_INVALID_ARGUMENT
    assert lib.kvc_select_topm(ctypes.byref(sh), None, m_ok, 6600, FAKE, None) == A.KVC_ERR_INVALID_ARGUMENT
    m_neg = (ctypes.c_int32 * 2)(-1, 0)
    assert lib.kvc_compact_contig(ctypes.byref(sh), A.KVC_BF16, FAKE, FAKE, FAKE, m_neg, 10, FAKE, FAKE,
                                  None) == A.KVC_ERR_INVALID_ARGUMENT
    assert lib.kvc_compact_contig(ctypes.byref(sh), 5, FAKE, FAKE, FAKE, m_ok, 6600, FAKE, FAKE,
                                  None) == A.KVC_ERR_INVALID_ARGUMENT
    counts = (ctypes.c_int32 * 2)(-7, -7)
    # same pool for K and V, and an unsupported page size: rejected, counts untouched
    assert lib.kvc_compact_paged(ctypes.byref(sh), A.KVC_BF16, FAKE, FAKE, 16, FAKE, 4096, FAKE, m_ok, 6600, None,
                                 FAKE, counts, None) == A.KVC_ERR_INVALID_ARGUMENT
    assert lib.kvc_compact_paged(ctypes.byref(sh), A.KVC_BF16, FAKE, FAKE + 64, 8, FAKE, 4096, FAKE, m_ok, 6600,
                                 None, FAKE, counts, None) == A.KVC_ERR_UNSUPPORTED
    assert list(counts) == [-7, -7]


def test_segment_validation(lib):
    """Segments: paged starts must be block-aligned; a segment followed by more tokens needs
    block-multiple lengths and budgets; contiguous segments must fit the row stride."""
    counts = (ctypes.c_int32 * 1)(-7)
    # paged segment start not a multiple of 16
    sh, keep = _shape(S=1, n=(160,), n_max=160).c()
    sh.seq_starts = (ctypes.c_int32 * 1)(8)
    m = (ctypes.c_int32 * 1)(32)
    st = lib.kvc_compact_paged(ctypes.byref(sh), A.KVC_BF16, FAKE, FAKE + 64, 16, FAKE, 100, FAKE, m, 32, None, FAKE,
                               counts, None)
    assert st == A.KVC_ERR_INVALID_ARGUMENT and b"multiple of the block size" in lib.kvc_last_error()
    # followed by more tokens: m must be a multiple of 16
    sh.seq_starts = (ctypes.c_int32 * 1)(32)
    clen = (ctypes.c_int32 * 1)(400)
    m_bad = (ctypes.c_int32 * 1)(33)
    st = lib.kvc_compact_paged(ctypes.byref(sh), A.KVC_BF16, FAKE, FAKE + 64, 16, FAKE, 100, FAKE, m_bad, 33, clen,
                               FAKE, counts, None)
    assert st == A.KVC_ERR_INVALID_ARGUMENT and b"multiples of 16" in lib.kvc_last_error()
    # cache length shorter than the segment's end
    clen_bad = (ctypes.c_int32 * 1)(100)
    st = lib.kvc_compact_paged(ctypes.byref(sh), A.KVC_BF16, FAKE, FAKE + 64, 16, FAKE, 100, FAKE, m, 32, clen_bad,
                               FAKE, counts, None)
    assert st == A.KVC_ERR_INVALID_ARGUMENT
    assert counts[0] == -7
    # contiguous segment running past n_max
    sh2, keep2 = _shape(S=1, n=(100,), n_max=120).c()
    sh2.seq_starts = (ctypes.c_int32 * 1)(30)
    kv = A.KView(FAKE, A.KVC_BF16).c()
    st = lib.kvc_score(ctypes.byref(sh2), FAKE, ctypes.byref(kv), FAKE, None, FAKE, None, 0, None)
    assert st == A.KVC_ERR_INVALID_ARGUMENT and b"n_max" in lib.kvc_last_error()
    m1 = (ctypes.c_int32 * 1)(20)
    st = lib.kvc_compact_contig(ctypes.byref(sh2), A.KVC_BF16, FAKE, FAKE, FAKE, m1, 20, FAKE, FAKE, None)
    assert st == A.KVC_ERR_INVALID_ARGUMENT
    # a negative start
    sh2.seq_starts = (ctypes.c_int32 * 1)(-1)
    st = lib.kvc_score(ctypes.byref(sh2), FAKE, ctypes.byref(kv), FAKE, None, FAKE, None, 0, None)
    assert st == A.KVC_ERR_INVALID_ARGUMENT


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    t = torch.zeros(4)
    with pytest.raises(ValueError):
        A._ptr(t)


def test_binding_refuses_short_buffers():
    torch = pytest.importorskip("torch")

    class Fake:
        def numel(self):
            return 10

        def element_size(self):
            return 4
    with pytest.raises(ValueError):
        A._need(Fake(), 41, "x")
    A._need(Fake(), 40, "x")


def test_retention_validation(lib):
    """Attention mass, LRFU update and side-array compaction reject bad arguments up front."""
    sh, keep = _shape().c()
    kv = A.KView(FAKE, A.KVC_BF16).c()
    assert lib.kvc_attention_mass(ctypes.byref(sh), FAKE, ctypes.byref(kv), FAKE, None, None, None, 0,
                                  None) == A.KVC_ERR_INVALID_ARGUMENT
    st = lib.kvc_attention_mass(ctypes.byref(sh), FAKE, ctypes.byref(kv), None, None, FAKE, FAKE, 16, None)
    assert st == A.KVC_ERR_WORKSPACE_TOO_SMALL and b"mass needs" in lib.kvc_last_error()
    for top_p, decay in ((0.0, 0.5), (1.5, 0.5), (float("nan"), 0.5), (0.9, -0.1), (0.9, 1.5), (0.9, float("nan"))):
        st = lib.kvc_lrfu_update(ctypes.byref(sh), FAKE, top_p, decay, FAKE, None, None)
        assert st == A.KVC_ERR_INVALID_ARGUMENT, (top_p, decay)
    assert lib.kvc_lrfu_update(ctypes.byref(sh), None, 0.9, 0.7, FAKE, None, None) == A.KVC_ERR_INVALID_ARGUMENT
    m_ok = (ctypes.c_int32 * 2)(6600, 4000)
    assert lib.kvc_compact_side(ctypes.byref(sh), 16, FAKE, m_ok, 6600, FAKE, FAKE, None) == A.KVC_ERR_INVALID_ARGUMENT
    assert b"distinct" in lib.kvc_last_error()
    assert lib.kvc_compact_side(ctypes.byref(sh), -1, FAKE, m_ok, 6600, FAKE, FAKE + 64, None) == \
        A.KVC_ERR_INVALID_ARGUMENT
    assert lib.kvc_compact_side(ctypes.byref(sh), 0, FAKE, m_ok, 100, FAKE, FAKE + 64, None) == \
        A.KVC_ERR_INVALID_ARGUMENT


def test_slot_map_validation(lib):
    """Slot-map key views and the dead-slot redirect reject bad arguments up front."""
    sh, keep = _shape().c()
    bad_dead = A.KView(FAKE, A.KVC_BF16, 0, None, 0, FAKE, -2).c()
    assert lib.kvc_score(ctypes.byref(sh), FAKE, ctypes.byref(bad_dead), FAKE, None, FAKE, None, 0, None) == \
        A.KVC_ERR_INVALID_ARGUMENT
    ok_view = A.KView(FAKE, A.KVC_BF16, 0, None, 0, FAKE, 7).c()
    assert oc.kvc_score_workspace_size(_shape(), A.KView(FAKE, A.KVC_BF16, 0, None, 0, FAKE, 7), True) == 0
    sh2, keep2 = _shape(S=1, n=(100,), n_max=120).c()
    sh2.seq_starts = (ctypes.c_int32 * 1)(30)
    assert lib.kvc_score(ctypes.byref(sh2), FAKE, ctypes.byref(ok_view), FAKE, None, FAKE, None, 0, None) == \
        A.KVC_ERR_INVALID_ARGUMENT  # the slot map row is n_max long
    m_ok = (ctypes.c_int32 * 2)(6600, 4000)
    m_bad = (ctypes.c_int32 * 2)(40000, 4000)
    assert lib.kvc_evict_redirect(ctypes.byref(sh), FAKE, m_ok, 6600, None, 5, None) == A.KVC_ERR_INVALID_ARGUMENT
    assert lib.kvc_evict_redirect(ctypes.byref(sh), FAKE, m_ok, 6600, FAKE, -1, None) == A.KVC_ERR_INVALID_ARGUMENT
    assert lib.kvc_evict_redirect(ctypes.byref(sh), FAKE, m_bad, 40000, FAKE, 5, None) == A.KVC_ERR_INVALID_ARGUMENT


def test_attention_matching_validation(lib):
    """kvc_am_fit rejects unsupported views, budgets and iteration counts up front."""
    sh = _shape()
    kv = A.KView(FAKE, A.KVC_BF16)
    m = [6600, 4000]
    # the kept exponentials E are materialised ([H][R][m rounded up to 64] floats per sequence), the
    # full attention weights are not
    ws = oc.kvc_am_workspace_size(sh, kv, kv, m, True)
    assert 4 * 8 * 4096 * (6656 + 4032) < ws < 4 * 8 * 4096 * (6600 + 33000)
    assert oc.kvc_am_workspace_size(sh, kv, kv, m, False) > oc.kvc_am_workspace_size(sh, kv, kv, m, True)
    assert oc.kvc_am_workspace_size(sh, A.KView(FAKE, A.KVC_F32), kv, m, True) == 0
    assert oc.kvc_am_workspace_size(_shape(G=1, q=8), kv, kv, m, True) == 0  # too few rows for MFMA
    s, keep = sh.c()
    k_, v_ = kv.c(), kv.c()
    mp = (ctypes.c_int32 * 2)(6600, 4000)
    f = lib.kvc_am_fit
    assert f(ctypes.byref(s), FAKE, ctypes.byref(k_), ctypes.byref(v_), FAKE, FAKE, mp, 6600, -1, 5, FAKE, FAKE, FAKE,
             1 << 40, None) == A.KVC_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(s), FAKE, ctypes.byref(k_), ctypes.byref(v_), FAKE, FAKE, mp, 6600, 5, 5, None, FAKE, FAKE,
             1 << 40, None) == A.KVC_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(s), FAKE, ctypes.byref(k_), ctypes.byref(v_), FAKE, FAKE, mp, 6600, 5, 5, FAKE, FAKE, FAKE,
             16, None) == A.KVC_ERR_WORKSPACE_TOO_SMALL
    sl = A.KView(FAKE, A.KVC_BF16, 0, None, 0, FAKE, 3).c()
    assert f(ctypes.byref(s), FAKE, ctypes.byref(sl), ctypes.byref(v_), FAKE, FAKE, mp, 6600, 5, 5, FAKE, FAKE, FAKE,
             1 << 40, None) == A.KVC_ERR_UNSUPPORTED


def test_causal_rows_validation(lib):
    """A causal mask can only grow the workspace (its LSE pass may use shorter key chunks),
    attention matching rejects it, and the binding refuses a row_pos tensor that is not int32 or
    too short."""
    torch = pytest.importorskip("torch")
    kv = A.KView(FAKE, A.KVC_BF16)
    sh = _shape()
    cz = _shape()
    cz.row_pos = FAKE
    assert oc.kvc_score_workspace_size(cz, kv, False) >= oc.kvc_score_workspace_size(sh, kv, False) > 0
    assert oc.kvc_lse_workspace_size(cz, kv) >= oc.kvc_lse_workspace_size(sh, kv) > 0
    assert oc.kvc_score_workspace_size(cz, kv, True) == 0
    assert oc.kvc_am_workspace_size(cz, kv, kv, [6600, 4000], True) == 0
    s, keep = cz.c()
    k_, v_ = kv.c(), kv.c()
    mp = (ctypes.c_int32 * 2)(6600, 4000)
    assert lib.kvc_am_fit(ctypes.byref(s), FAKE, ctypes.byref(k_), ctypes.byref(v_), FAKE, FAKE, mp, 6600, 5, 5,
                          FAKE, FAKE, FAKE, 1 << 40, None) == A.KVC_ERR_UNSUPPORTED
    assert b"row_pos" in lib.kvc_last_error()
    bad = _shape()
    bad.row_pos = torch.zeros((2, 32, 1024), dtype=torch.int64)
    with pytest.raises(ValueError):
        bad.c()
    bad.row_pos = torch.zeros((2, 32, 1000), dtype=torch.int32)
    with pytest.raises(ValueError):
        bad.c()


def test_oversized_launches_rejected_before_any_launch(lib):
    """Work-item counts are summed in 64 bits per launch slice (128 sequences) during validation:
    a request whose later slice would exceed 2^31 - 1 work items fails as unsupported before the
    first slice is launched, and a paged compaction then leaves its host outputs untouched."""
    S, n = 130, 1 << 16
    lens = np.full(S, n, dtype=np.int32)
    sh, keep = A.Shape(S, 1 << 20, 1, 1, 128, n, lens, 0.088).c()
    m = (ctypes.c_int32 * S)(*([0] * 128 + [n, n]))  # nothing to do in the first slice
    counts = (ctypes.c_int32 * S)(*([-7] * S))
    st = lib.kvc_compact_paged(ctypes.byref(sh), A.KVC_BF16, FAKE, FAKE + 64, 16, FAKE, n // 16, FAKE, m, n, None,
                               FAKE, counts, None)
    assert st == A.KVC_ERR_UNSUPPORTED, lib.kvc_last_error()
    assert b"work items" in lib.kvc_last_error()
    assert list(counts) == [-7] * S
    st = lib.kvc_compact_contig(ctypes.byref(sh), A.KVC_BF16, FAKE, FAKE, FAKE, m, n, FAKE, FAKE, None)
    assert st == A.KVC_ERR_UNSUPPORTED
    # one work item per (sequence, head): 128 sequences x 2^25 heads
    sh2, keep2 = A.Shape(128, 1 << 25, 1, 1, 128, 64, np.full(128, 64, dtype=np.int32), 0.088).c()
    m2 = (ctypes.c_int32 * 128)(*([1] * 128))
    assert lib.kvc_select_topm(ctypes.byref(sh2), FAKE, m2, 1, FAKE, None) == A.KVC_ERR_UNSUPPORTED
    # the score kernel's key tiles are checked before the LSE pass would launch
    kv = A.KView(FAKE, A.KVC_BF16).c()
    sh3, keep3 = A.Shape(2, 1 << 24, 1, 16, 128, 1 << 16, np.full(2, 1 << 16, dtype=np.int32), 0.088).c()
    st = lib.kvc_score(ctypes.byref(sh3), FAKE, ctypes.byref(kv), None, None, FAKE, FAKE, 1 << 62, None)
    assert st == A.KVC_ERR_UNSUPPORTED, lib.kvc_last_error()


def test_noalloc_scratch_limit_and_validation(lib):
    """kvc_score_noalloc: the binding's scratch size is the header's; bad shapes are invalid
    arguments; a shape whose computed LSE needs more scratch than the static array holds is
    rejected as unsupported before any device call (the same shape the GPU test uses)."""
    text = open(HEADER).read()
    m = re.search(r"#define KVC_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == A.KVC_NOALLOC_SCRATCH_BYTES
    kv = A.KView(FAKE, A.KVC_BF16).c()
    sh, keep = _shape(d=64).c()
    assert lib.kvc_score_noalloc(ctypes.byref(sh), FAKE, ctypes.byref(kv), None, None, FAKE, None) == \
        A.KVC_ERR_UNSUPPORTED
    sh, keep = _shape(n=(0, 5)).c()
    assert lib.kvc_score_noalloc(ctypes.byref(sh), FAKE, ctypes.byref(kv), None, None, FAKE, None) == \
        A.KVC_ERR_INVALID_ARGUMENT
    S, H, G, q, n = 64, 4, 8, 256, 131072
    shape = A.Shape(S, H, G, q, 128, n, np.full(S, n, dtype=np.int32), 0.088)
    pv = A.KView(FAKE, A.KVC_BF16, 16, FAKE, n // 16)
    assert oc.kvc_score_workspace_size(shape, pv, False) > A.KVC_NOALLOC_SCRATCH_BYTES
    sh, keep = shape.c()
    v = pv.c()
    st = lib.kvc_score_noalloc(ctypes.byref(sh), FAKE, ctypes.byref(v), None, None, FAKE, None)
    assert st == A.KVC_ERR_UNSUPPORTED and b"scratch" in lib.kvc_last_error()
    # the action-token trajectory (8 heads x 1320 rows, 33000 keys) fits
    small = A.Shape(1, 8, 4, 330, 128, 33000, np.array([33000], dtype=np.int32), 0.088)
    assert 0 < oc.kvc_score_workspace_size(small, A.KView(FAKE, A.KVC_BF16, 16, FAKE, 2063), False) \
        <= A.KVC_NOALLOC_SCRATCH_BYTES
