"""GPU parity of Attention Matching (beta by multiplicative NNLS updates, V_C by Landweber steps)
against the float64 oracle running the same iterations."""
import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from tests.parity import check_am_unit, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _P():
    from online_compaction_amd import path as P
    return P


def _run(w, data, kept, m, iters_beta, iters_v, lse=None):
    P = _P()
    import online_compaction_amd as oc
    if w.paged:
        kv = oc.KView(P.device_tensor(data["k_pool"]), oc.KVC_BF16, w.block_size, P.device_tensor(data["table"]),
                      w.max_blocks)
        vv = oc.KView(P.device_tensor(data["v_pool"]), oc.KVC_BF16, w.block_size, kv.block_table, w.max_blocks)
    else:
        kv = oc.KView(P.device_tensor(data["K"]), oc.KVC_BF16)
        vv = oc.KView(P.device_tensor(data["V"]), oc.KVC_BF16)
    shape = oc.Shape(w.S, w.H, w.G, w.q, w.d, w.n_max, np.array(w.n, dtype=np.int32), w.logit_scale)
    m_max = int(max(m))
    beta = torch.full((w.S, w.H, m_max), 7.0, dtype=torch.float32, device="cuda")
    vc = torch.full((w.S, w.H, m_max, w.d), 7.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, oc.kvc_am_workspace_size(shape, kv, vv, m, lse is not None)), dtype=torch.uint8,
                     device="cuda")
    dl = None if lse is None else P.device_tensor(lse)
    oc.kvc_am_fit(shape, P.device_tensor(data["Q"]), kv, vv, dl, P.device_tensor(kept), m, m_max, iters_beta, iters_v,
                  beta, vc, ws)
    torch.cuda.synchronize()
    return beta.cpu().numpy(), vc.cpu().numpy()


def _keys_values(w, data, s, h):
    n = w.n[s]
    if w.paged:
        return (O.paged_unit_keys(data["k_pool"], data["table"][s], n, h, w.block_size),
                O.paged_unit_keys(data["v_pool"], data["table"][s], n, h, w.block_size))
    return data["K"][s, h, :n], data["V"][s, h, :n]


def _check(w, data, kept, m, beta, vc, iters_beta, iters_v, lse=None, tag=""):
    """Every unit of the batch against the oracle (the criteria of check_am_unit)."""
    worst = {}
    for s in range(w.S):
        for h in range(w.H):
            K, V = _keys_values(w, data, s, h)
            rows = O.unit_rows(data["Q"], s, h, w.G)
            lr = None if lse is None else lse[s, h * w.G:(h + 1) * w.G].reshape(-1).astype(np.float64)
            err = check_am_unit(rows, K, V, lr, kept[s, h, :m[s]], beta[s, h], vc[s, h], w.dtype, w.logit_scale,
                                iters_beta, iters_v, f"{tag} s={s} h={h}")
            for key, val in err.items():
                worst[key] = max(worst.get(key, 0.0), val)
    say(f"[ok] am {tag}: worst " + ", ".join(f"{k} {v:.3g}" for k, v in worst.items()))


def _kept(rng, w, m):
    kept = np.zeros((w.S, w.H, max(m)), dtype=np.int32)
    for s in range(w.S):
        for h in range(w.H):
            kept[s, h, :m[s]] = np.sort(rng.choice(w.n[s], size=m[s], replace=False))
    return kept


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_am_small_matches_oracle(layout):
    w = W.custom(f"am_{layout}", 170, S=2, H=2, G=4, q=8, n=(300, 129), dtype="bf16", keys="mixture",
                 queries="cluster", paged=layout == "paged", table="permuted", block_size=16)
    data = W.build_paged(w) if w.paged else W.build_contiguous(w)
    m = [60, 40]
    kept = _kept(np.random.default_rng(3), w, m)
    say(f"[case] am {layout}: n={list(w.n)} m={m} R={w.R}")
    beta, vc = _run(w, data, kept, m, 8, 8)
    _check(w, data, kept, m, beta, vc, 8, 8, tag=layout)


def test_am_zero_iterations_is_plain_eviction():
    w = W.custom("am_zero", 171, S=1, H=2, G=4, q=4, n=(200,), dtype="bf16", keys="mixture", queries="cluster")
    data = W.build_contiguous(w)
    m = [50]
    kept = _kept(np.random.default_rng(4), w, m)
    beta, vc = _run(w, data, kept, m, 0, 0)
    # w = 1 is held as exp(ME - Mz) in scaled units: beta = 0 up to one float32 exp/log round trip
    assert np.all(np.abs(beta[:, :, :50]) <= 1e-4)
    for h in range(w.H):
        assert np.array_equal(vc[0, h, :50], W.bf16_bits_to_f32(data["V"][0, h, kept[0, h, :50]]))


def test_am_supplied_lse_and_many_tiles():
    """2048 proxy rows (32 row tiles), 4096 keys, 819 kept (13 key tiles), 16 + 16 iterations,
    LSE supplied by the oracle."""
    w = W.custom("am_big", 172, S=1, H=2, G=4, q=512, n=(4096,), dtype="bf16", keys="mixture", queries="cluster")
    data = W.build_contiguous(w)
    m = [819]
    kept = _kept(np.random.default_rng(5), w, m)
    lse = np.zeros((w.S, w.H * w.G, w.q), dtype=np.float32)
    for h in range(w.H):
        L = O.lse_unit(O.unit_rows(data["Q"], 0, h, w.G), data["K"][0, h, :w.n[0]], w.dtype, w.logit_scale)
        lse[0, h * w.G:(h + 1) * w.G] = L.astype(np.float32).reshape(w.G, w.q)
    say(f"[case] am big: R={w.R} n={w.n[0]} m={m[0]}")
    beta, vc = _run(w, data, kept, m, 16, 16, lse)
    _check(w, data, kept, m, beta, vc, 16, 16, lse, tag="big")


@pytest.mark.parametrize("iters_v", [1, 2, 3, 9])
def test_am_value_iteration_on_either_side(iters_v):
    """The value steps run on the smaller side of P_C: 128 proxy rows against 60 kept keys (the
    keys side) and 200 kept keys (the rows side) in one call; one step is the direct product,
    two or more go through the Gram matrix, an odd and an even count end in either buffer."""
    w = W.custom("am_sides", 173, S=2, H=2, G=4, q=32, n=(400, 257), dtype="bf16", keys="mixture",
                 queries="cluster")
    data = W.build_contiguous(w)
    m = [60, 200]
    kept = _kept(np.random.default_rng(6 + iters_v), w, m)
    say(f"[case] am sides: R={w.R} n={list(w.n)} m={m} iterations 4 + {iters_v}")
    beta, vc = _run(w, data, kept, m, 4, iters_v)
    _check(w, data, kept, m, beta, vc, 4, iters_v, tag=f"sides v{iters_v}")


def test_am_target_key_splits_with_a_ragged_tail():
    """2048 proxy rows over 4000 keys (63 chunks of 64, the last one partial): the target's keys
    are split eight ways (seven runs of 8 chunks, one of 7), and the partial targets are added in
    order by the first value product; 12 + 12 iterations."""
    w = W.custom("am_ragged", 174, S=1, H=1, G=4, q=512, n=(4000,), dtype="bf16", keys="mixture",
                 queries="cluster")
    data = W.build_contiguous(w)
    m = [801]
    kept = _kept(np.random.default_rng(9), w, m)
    say(f"[case] am ragged splits: R={w.R} n={w.n[0]} m={m[0]}")
    beta, vc = _run(w, data, kept, m, 12, 12)
    _check(w, data, kept, m, beta, vc, 12, 12, tag="ragged")


def test_am_on_a_segment_of_a_longer_cache():
    """The fit over one turn inside a longer contiguous cache (seq_starts): keys, values and
    kept positions are the segment's, [start, start + n); the oracle runs on the sliced rows."""
    P = _P()
    import online_compaction_amd as oc
    w = W.custom("am_segment", 175, S=2, H=2, G=4, q=8, n=(600, 600), dtype="bf16", keys="mixture",
                 queries="cluster")
    data = W.build_contiguous(w)
    starts, lens, m = [150, 40], [300, 129], [60, 31]
    kept = np.zeros((w.S, w.H, max(m)), dtype=np.int32)
    rng = np.random.default_rng(11)
    for s in range(w.S):
        for h in range(w.H):
            kept[s, h, :m[s]] = np.sort(rng.choice(lens[s], size=m[s], replace=False))
    kv = oc.KView(P.device_tensor(data["K"]), oc.KVC_BF16)
    vv = oc.KView(P.device_tensor(data["V"]), oc.KVC_BF16)
    shape = oc.Shape(w.S, w.H, w.G, w.q, w.d, w.n_max, np.array(lens, dtype=np.int32), w.logit_scale,
                     seq_starts=np.array(starts, dtype=np.int32))
    m_max = max(m)
    beta = torch.full((w.S, w.H, m_max), 7.0, dtype=torch.float32, device="cuda")
    vc = torch.full((w.S, w.H, m_max, w.d), 7.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, oc.kvc_am_workspace_size(shape, kv, vv, m, False)), dtype=torch.uint8, device="cuda")
    say(f"[case] am segment: starts={starts} n={lens} m={m} R={w.R}")
    oc.kvc_am_fit(shape, P.device_tensor(data["Q"]), kv, vv, None, P.device_tensor(kept), m, m_max, 8, 8, beta, vc, ws)
    torch.cuda.synchronize()
    beta, vc = beta.cpu().numpy(), vc.cpu().numpy()
    for s in range(w.S):
        a, n = starts[s], lens[s]
        for h in range(w.H):
            err = check_am_unit(O.unit_rows(data["Q"], s, h, w.G), data["K"][s, h, a:a + n], data["V"][s, h, a:a + n],
                                None, kept[s, h, :m[s]], beta[s, h], vc[s, h], w.dtype, w.logit_scale, 8, 8,
                                f"segment s={s} h={h}")
            say(f"[ok] am segment s={s} h={h}: " + ", ".join(f"{k} {v:.3g}" for k, v in err.items()))
