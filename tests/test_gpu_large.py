"""A contiguous cache whose K/V arrays pass 2^31 elements: one agent turn scored, selected and
gathered from the end of each head's 8.45 M-token cache, so that the second head's rows sit on
both sides of element 2^31 of K and V. Every score, the kept set and every gathered row are
checked against the float64 oracle; the LSE entry point is checked on the same segment.

The 8.6 GiB of K/V are drawn on the device by torch's seeded generator (rounded to bfloat16);
the oracle reads the scored segments back to the host."""
import time

import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from tests.parity import (check_gather, check_kept_form, check_scores, check_selection_band,
                          check_selection_exact, say)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

H, G, QN, D = 2, 4, 4, 128
N_MAX = 8_454_145                      # cache rows per head: H * N_MAX * D = 2.16e9 elements
N = 300_007                            # scored segment (one turn), ragged
START = N_MAX - N                      # the turn sits at the end of the cache
M = 60_001
SCALE = D ** -0.5
# float32 LSE over 300 K keys: about 80 chunk partials of <= 4096 keys merged online; the
# accumulated rounding stays near 1e-6 of the sum, i.e. 1e-6 in the log
LSE_TOL = 1e-5


def test_turn_at_the_end_of_a_cache_past_2_31_elements():
    import online_compaction_amd as oc
    from online_compaction_amd import _abi as A
    from online_compaction_amd import path as P

    # the second head's segment crosses element 2^31 of K and V
    first = ((1 * N_MAX + START) * D, (1 * N_MAX + START + N) * D)
    assert first[0] < 2 ** 31 < first[1]
    say(f"[case] large contiguous: H={H} n_max={N_MAX} segment [{START}, {N_MAX}) R={G * QN} m={M}")
    t0 = time.time()
    K = W.device_normal_bf16((1, H, N_MAX, D), seed=2311)
    V = W.device_normal_bf16((1, H, N_MAX, D), seed=2312)
    Qd = W.device_normal_bf16((1, H * G, QN, D), seed=2313)
    torch.cuda.synchronize()
    say(f"[case] inputs on the device in {time.time() - t0:.1f} s")

    shape = A.Shape(1, H, G, QN, D, N_MAX, np.array([N], dtype=np.int32), SCALE, np.array([START], dtype=np.int32))
    b = P.Batch(shape, A.KVC_BF16, Qd, np.array([M], dtype=np.int32), M, k=K, v=V)
    o = P.allocate(b)
    P.run(b, o)
    lse_gpu = torch.zeros((1, H * G, QN), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, oc.kvc_lse_workspace_size(b.shape, b.kview())), dtype=torch.uint8, device="cuda")
    oc.kvc_lse(b.shape, b.q, b.kview(), None, lse_gpu, ws)
    torch.cuda.synchronize()
    say(f"[ok] GPU pass done ({time.time() - t0:.1f} s)")

    scores, kept = P.host_array(o.scores), P.host_array(o.kept)
    k_out, v_out = P.host_array(o.k_out), P.host_array(o.v_out)
    lse_all = lse_gpu.cpu().numpy()
    Qh = P.host_array(Qd)
    for h in range(H):
        tag = f"large h={h}"
        Kh = P.host_array(K[0, h, START:])
        Vh = P.host_array(V[0, h, START:])
        rows = O.widen(O.unit_rows(Qh, 0, h, G), "bf16")
        keys = O.widen(Kh, "bf16")
        lse_ref = O.lse(rows, keys, SCALE)
        np.testing.assert_allclose(lse_all[0, h * G:(h + 1) * G].reshape(-1), lse_ref, rtol=LSE_TOL, atol=LSE_TOL)
        ref = O.te_scores(rows, keys, SCALE, lse_rows=lse_ref)
        del keys
        worst = check_scores(scores[0, h, :N], ref, tag)
        check_kept_form(kept[0, h], M, N, tag)
        check_selection_exact(kept[0, h], scores[0, h, :N], M, tag)
        swaps = check_selection_band(kept[0, h], ref, M, tag)
        check_gather(Kh, kept[0, h], k_out[0, h], M, tag + " K")
        check_gather(Vh, kept[0, h], v_out[0, h], M, tag + " V")
        say(f"[ok] {tag}: worst score rel err {worst:.3g}, {swaps} band swaps, rows gathered exactly "
            f"({time.time() - t0:.1f} s)")
