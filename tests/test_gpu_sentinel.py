"""GPU parity of layout-preserving eviction: the dead-slot redirect, and scoring, attention mass
and the LSE read through a slot map whose dead slot acts as a logit mask."""
import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from tests.parity import (check_kept_form, check_scores, check_selection_band, check_selection_exact, say,
                          slot_setup)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _P():
    from online_compaction_amd import path as P
    return P


def _oc():
    import online_compaction_amd as oc
    return oc


@pytest.mark.parametrize("case", ["mfma_bf16", "valu_f32", "mfma_bias_all_dead_unit"])
def test_scores_and_mass_through_slot_map(case):
    P, oc = _P(), _oc()
    if case == "valu_f32":
        w = W.custom("slot_valu", 160, S=2, H=2, G=1, q=6, n=(700, 333), paged=True, table="permuted",
                     block_size=16)
    else:
        w = W.custom("slot_mfma", 161, S=2, H=2, G=4, q=20, n=(2500, 900), dtype="bf16", keys="mixture",
                     queries="cluster", paged=True, table="permuted", block_size=16,
                     bias_tail=0.5 if "bias" in case else 0.0)
    rng = np.random.default_rng(7)
    data = W.build_paged(w)
    pool, smap, live, dead = slot_setup(w, data, 0.45, rng)
    if "all_dead" in case:
        smap[1, 0, :w.n[1]] = dead
        live[1, 0, :] = False
    say(f"[case] slot map {case}: n={list(w.n)} dead share ~0.45, dead slot {dead}")
    dq = P.device_tensor(data["Q"])
    kv = oc.KView(P.device_tensor(pool), oc.KVC_BF16 if w.dtype == "bf16" else oc.KVC_F32, 0, None, 0,
                  P.device_tensor(smap), dead)
    shape = oc.Shape(w.S, w.H, w.G, w.q, w.d, w.n_max, np.array(w.n, dtype=np.int32), w.logit_scale)
    bias = None if data["bias"] is None else P.device_tensor(data["bias"].astype(np.float32))
    ws = torch.empty(max(256, oc.kvc_score_workspace_size(shape, kv, False)), dtype=torch.uint8, device="cuda")
    scores = torch.full((w.S, w.H, w.n_max), -1.0, dtype=torch.float32, device="cuda")
    mass = torch.full_like(scores, -1.0)
    oc.kvc_score(shape, dq, kv, None, bias, scores, ws)
    oc.kvc_attention_mass(shape, dq, kv, None, bias, mass, ws)
    torch.cuda.synchronize()
    sc, ma = scores.cpu().numpy(), mass.cpu().numpy()
    for s in range(w.S):
        n = w.n[s]
        b = None if data["bias"] is None else data["bias"][s, :n]
        for h in range(w.H):
            keys = O.slot_unit_keys(pool, smap[s, h], n, h)
            rows = O.unit_rows(data["Q"], s, h, w.G)
            lv = live[s, h, :n]
            ref = O.score_unit_live(rows, keys, lv, w.dtype, w.logit_scale, b)
            mref = O.score_unit_live(rows, keys, lv, w.dtype, w.logit_scale, b, power=1)
            assert np.all(sc[s, h, :n][~lv] == 0) and np.all(ma[s, h, :n][~lv] == 0), "dead positions score 0"
            assert np.all(np.isfinite(sc[s, h, :n])) and np.all(np.isfinite(ma[s, h, :n]))
            check_scores(sc[s, h, :n], ref, f"slot score s={s} h={h}")
            check_scores(ma[s, h, :n], mref, f"slot mass s={s} h={h}")
            if lv.any():
                assert abs(float(ma[s, h, :n].astype(np.float64).sum()) - 1.0) < 1e-4
            assert np.all(sc[s, h, n:] == -1.0), "past n untouched"
    say(f"[ok] slot map {case}")


def test_redirect_matches_oracle():
    P, oc = _P(), _oc()
    rng = np.random.default_rng(31)
    S, H, n_max = 3, 2, 4000
    lens, m = [4000, 1234, 17], [800, 0, 17]
    starts = [0, 100, 3000]
    kept = np.zeros((S, H, max(m)), dtype=np.int32)
    for s in range(S):
        for h in range(H):
            kept[s, h, :m[s]] = np.sort(rng.choice(lens[s], size=m[s], replace=False))
    smap = rng.integers(0, 10 ** 6, size=(S, H, n_max)).astype(np.int32)
    dead = 4242
    shape = oc.Shape(S, H, 1, 1, 128, n_max, np.array(lens, dtype=np.int32), 1.0, np.array(starts, dtype=np.int32))
    dmap = P.device_tensor(smap)
    oc.kvc_evict_redirect(shape, P.device_tensor(kept), m, max(m), dmap, dead)
    torch.cuda.synchronize()
    got = dmap.cpu().numpy()
    for s in range(S):
        a = starts[s]
        for h in range(H):
            want = smap[s, h].copy()
            want[a:a + lens[s]] = O.evict_redirect(smap[s, h, a:a + lens[s]], kept[s, h, :m[s]], lens[s], dead)
            assert np.array_equal(got[s, h], want), f"s={s} h={h}"
    say("[ok] redirect")


def test_evict_then_rescore_end_to_end():
    """Score, keep the top m, redirect the rest to the dead slot, score again through the map:
    evicted positions score 0 and the kept ones are scored as if the others were gone; a second,
    smaller selection picks only among them."""
    P, oc = _P(), _oc()
    w = W.custom("slot_e2e", 162, S=2, H=2, G=4, q=16, n=(3000, 1500), dtype="bf16", keys="mixture",
                 queries="cluster", paged=True, table="permuted", block_size=16)
    data = W.build_paged(w)
    pool, smap, live, dead = slot_setup(w, data, 0.0, np.random.default_rng(1))
    dq = P.device_tensor(data["Q"])
    dmap = P.device_tensor(smap)
    kv = oc.KView(P.device_tensor(pool), oc.KVC_BF16, 0, None, 0, dmap, dead)
    shape = oc.Shape(w.S, w.H, w.G, w.q, w.d, w.n_max, np.array(w.n, dtype=np.int32), w.logit_scale)
    ws = torch.empty(max(256, oc.kvc_score_workspace_size(shape, kv, False)), dtype=torch.uint8, device="cuda")
    m = np.array(w.m, dtype=np.int32)
    scores = torch.zeros((w.S, w.H, w.n_max), dtype=torch.float32, device="cuda")
    kept = torch.zeros((w.S, w.H, int(m.max())), dtype=torch.int32, device="cuda")
    oc.kvc_score(shape, dq, kv, None, None, scores, ws)
    oc.kvc_select_topm(shape, scores, m, int(m.max()), kept)
    oc.kvc_evict_redirect(shape, kept, m, int(m.max()), dmap, dead)
    oc.kvc_score(shape, dq, kv, None, None, scores, ws)
    m2 = m // 2
    kept2 = torch.zeros((w.S, w.H, int(m2.max())), dtype=torch.int32, device="cuda")
    oc.kvc_select_topm(shape, scores, m2, int(m2.max()), kept2)
    torch.cuda.synchronize()
    k1, sc2, k2, mp = P.host_array(kept), P.host_array(scores), P.host_array(kept2), P.host_array(dmap)
    for s in range(w.S):
        n = w.n[s]
        for h in range(w.H):
            tag = f"e2e s={s} h={h}"
            lv = np.zeros(n, dtype=bool)
            lv[k1[s, h, :m[s]]] = True
            assert np.array_equal(mp[s, h, :n] != dead, lv), f"{tag}: map after redirect"
            ref = O.score_unit_live(O.unit_rows(data["Q"], s, h, w.G), O.slot_unit_keys(pool, smap[s, h], n, h), lv,
                                    w.dtype, w.logit_scale)
            check_scores(sc2[s, h, :n], ref, tag)
            check_kept_form(k2[s, h], m2[s], n, tag)
            check_selection_exact(k2[s, h], sc2[s, h, :n], m2[s], tag)
            check_selection_band(k2[s, h], ref, m2[s], tag)
            assert lv[k2[s, h, :m2[s]]].all(), f"{tag}: second selection picked an evicted position"
    say("[ok] evict -> rescore -> select")
