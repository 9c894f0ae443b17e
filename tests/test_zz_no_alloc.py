"""kvc_score_noalloc: the score entry point with its scratch in the library's static device array,
for callers that cannot allocate. Through the C ABI it must give kvc_score's scores bit for bit
(the same kernels; only where the LSE scratch lives differs) and so stay within the oracle's
1e-3 band, on two calls in a row (the second smaller, reusing the array the first left behind),
on the MFMA and VALU paths and with contiguous and paged keys; a supplied LSE needs no scratch;
a shape whose scratch exceeds the array is rejected before anything is enqueued."""
import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from tests.parity import check_scores, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _P():
    from online_compaction_amd import path as P
    return P


def _batch(w):
    P = _P()
    if w.paged:
        data = W.build_paged(w)
        b = P.paged_batch(data["Q"], data["k_pool"], data["v_pool"], data["table"], data["n"], data["m"], w.G,
                          w.logit_scale, w.block_size, n_max=w.n_max, bias=data["bias"])
    else:
        data = W.build_contiguous(w)
        b = P.contiguous_batch(data["Q"], data["K"], data["V"], data["n"], data["m"], w.G, w.logit_scale,
                               bias=data["bias"])
    return data, b


def _oracle_scores(w, data, s, h):
    n = w.n[s]
    keys = (O.paged_unit_keys(data["k_pool"], data["table"][s], n, h, w.block_size) if w.paged
            else data["K"][s, h, :n])
    b = None if data["bias"] is None else data["bias"][s, :n]
    return O.score_unit(O.unit_rows(data["Q"], s, h, w.G), keys, w.dtype, w.logit_scale, b)


def _compare(w, lse=None):
    import online_compaction_amd as oc
    P = _P()
    data, b = _batch(w)
    if lse == "oracle":
        L = np.zeros((w.S, w.H * w.G, w.q), dtype=np.float32)
        for s in range(w.S):
            for h in range(w.H):
                keys = (O.paged_unit_keys(data["k_pool"], data["table"][s], w.n[s], h, w.block_size) if w.paged
                        else data["K"][s, h, :w.n[s]])
                bias = None if data["bias"] is None else data["bias"][s, :w.n[s]]
                L[s, h * w.G:(h + 1) * w.G] = O.lse_unit(O.unit_rows(data["Q"], s, h, w.G), keys, w.dtype,
                                                         w.logit_scale, bias).astype(np.float32).reshape(w.G, w.q)
        b.lse = P.device_tensor(L)
    o = P.allocate(b)
    shape = (w.S, w.H, w.n_max)
    want = torch.full(shape, -3.0, dtype=torch.float32, device="cuda")
    got = torch.full(shape, -3.0, dtype=torch.float32, device="cuda")
    oc.kvc_score(b.shape, b.q, b.kview(), b.lse, b.bias, want, o.ws)
    oc.kvc_score_noalloc(b.shape, b.q, b.kview(), b.lse, b.bias, got)
    torch.cuda.synchronize()
    want, got = P.host_array(want), P.host_array(got)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{w.name}: differs from kvc_score"
    worst = 0.0
    for s in range(w.S):
        for h in range(w.H):
            n = w.n[s]
            if lse == "oracle":
                ref = O.score_unit(O.unit_rows(data["Q"], s, h, w.G),
                                   (O.paged_unit_keys(data["k_pool"], data["table"][s], n, h, w.block_size)
                                    if w.paged else data["K"][s, h, :n]), w.dtype, w.logit_scale,
                                   None if data["bias"] is None else data["bias"][s, :n],
                                   P.host_array(b.lse)[s, h * w.G:(h + 1) * w.G].reshape(-1).astype(np.float64))
            else:
                ref = _oracle_scores(w, data, s, h)
            worst = max(worst, check_scores(got[s, h, :n], ref, f"{w.name} s={s} h={h}"))
            assert np.all(got[s, h, n:] == -3.0), f"{w.name} s={s} h={h}: entries past n written"
    say(f"[ok] {w.name}: noalloc == kvc_score bit for bit; worst rel err vs oracle {worst:.3g}")


def test_noalloc_mfma_contiguous_two_calls():
    # first call: three ragged sequences; second: one shorter sequence (reuses the array)
    _compare(W.custom("na_mfma_a", 301, S=3, H=2, G=4, q=40, n=(700, 1500, 2100), dtype="bf16", keys="mixture",
                      queries="cluster"))
    _compare(W.custom("na_mfma_b", 302, S=1, H=2, G=4, q=40, n=(333,), dtype="bf16", keys="mixture",
                      queries="cluster"))


def test_noalloc_valu_two_calls():
    _compare(W.custom("na_valu_a", 303, S=2, H=3, G=2, q=3, n=(1300, 517)))
    _compare(W.custom("na_valu_b", 304, S=1, H=1, G=2, q=3, n=(90,)))


def test_noalloc_paged_bias_two_calls():
    _compare(W.custom("na_paged_a", 305, S=2, H=2, G=2, q=24, n=(1000, 1777), dtype="bf16", keys="mixture",
                      queries="cluster", paged=True, table="permuted", bias_tail=0.5))
    _compare(W.custom("na_paged_b", 306, S=1, H=2, G=2, q=24, n=(250,), dtype="bf16", keys="mixture",
                      queries="cluster", paged=True, table="permuted", bias_tail=0.5))


def test_noalloc_supplied_lse_uses_no_scratch():
    _compare(W.custom("na_lse", 307, S=2, H=2, G=4, q=20, n=(900, 411), dtype="bf16", keys="mixture",
                      queries="cluster"), lse="oracle")


def test_noalloc_rejects_shapes_beyond_the_scratch():
    import online_compaction_amd as oc
    from online_compaction_amd import _abi as A
    # 64 sequences x 4 heads x 2048 rows, 131072 keys each: the LSE partials alone exceed 64 MiB
    S, H, G, q, n = 64, 4, 8, 256, 131072
    shape = A.Shape(S, H, G, q, 128, n, np.full(S, n, dtype=np.int32), 0.088)
    # a one-block pool and an all-zero table: every position of every sequence names that block
    kv = A.KView(torch.zeros((1, 16, H, 128), dtype=torch.bfloat16, device="cuda"), A.KVC_BF16, 16,
                 torch.zeros((S, n // 16), dtype=torch.int32, device="cuda"), n // 16)
    assert oc.kvc_score_workspace_size(shape, kv, False) > A.KVC_NOALLOC_SCRATCH_BYTES
    qd = torch.empty((S, H * G, q, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.full((S, H, n), -3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(A.KvcError) as ei:
        oc.kvc_score_noalloc(shape, qd, kv, None, None, out)
    assert ei.value.status == A.KVC_ERR_UNSUPPORTED and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == -3.0).all()), "a rejected call wrote its output"
