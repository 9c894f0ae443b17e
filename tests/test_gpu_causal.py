"""GPU parity of causal proxy rows (row r of a unit sees only the keys j <= row_pos[r], the
in-trajectory action tokens of ActKV): scores, attention mass and the LSE on the MFMA and VALU
paths, contiguous, paged and through a slot map, against the oracle; the mask that hides
nothing against the unmasked kernels bit for bit; and the whole score -> select -> compact
path with the mask."""
import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from tests.parity import (check_gather, check_kept_form, check_scores, check_selection_band,
                          check_selection_exact, say, slot_setup)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _P():
    from online_compaction_amd import path as P
    return P


def _oc():
    import online_compaction_amd as oc
    return oc


def _workload(case):
    if case == "mfma_action_bias":      # the action tokens' own positions, biased tail
        return W.custom("causal_act", 170, S=1, H=2, G=4, q=40, n=(3000,), dtype="bf16", keys="mixture",
                        queries="action", bias_tail=0.5), "action"
    if case == "mfma_two_row_blocks":   # R = 600: two LSE row blocks, ten score stages, ragged tails
        return W.custom("causal_rb", 171, S=2, H=2, G=4, q=150, n=(2100, 700), dtype="bf16", keys="mixture",
                        queries="cluster"), "spread"
    if case == "mfma_paged":
        return W.custom("causal_pg", 172, S=2, H=2, G=2, q=24, n=(1000, 1333), dtype="bf16", keys="mixture",
                        queries="cluster", paged=True, table="permuted", block_size=16), "spread"
    if case == "valu_f32":
        return W.custom("causal_vf", 173, S=1, H=3, G=1, q=7, n=(900,)), "spread"
    if case == "valu_bf16":             # R = 8 < 16 rows: bf16 on the VALU path
        return W.custom("causal_vb", 174, S=1, H=2, G=1, q=8, n=(1500,), dtype="bf16", keys="mixture",
                        queries="cluster"), "spread"
    if case == "supplied_lse":
        return W.custom("causal_lse", 175, S=1, H=2, G=4, q=20, n=(1500,), dtype="bf16", keys="mixture",
                        queries="cluster"), "spread"
    raise ValueError(case)


def _batch(w, data, lse=None):
    P = _P()
    if w.paged:
        return P.paged_batch(data["Q"], data["k_pool"], data["v_pool"], data["table"], data["n"], data["m"], w.G,
                             w.logit_scale, w.block_size, n_max=w.n_max, bias=data["bias"], lse=lse)
    return P.contiguous_batch(data["Q"], data["K"], data["V"], data["n"], data["m"], w.G, w.logit_scale,
                              bias=data["bias"], lse=lse)


def _keys(w, data, s, h):
    n = w.n[s]
    return (O.paged_unit_keys(data["k_pool"], data["table"][s], n, h, w.block_size) if w.paged
            else data["K"][s, h, :n])


def _run_all(oc, b, w, with_lse=True):
    """Scores, masses and (optionally) the LSE of a batch; outputs past each n start at -1."""
    scores = torch.full((w.S, w.H, w.n_max), -1.0, dtype=torch.float32, device="cuda")
    mass = torch.full_like(scores, -1.0)
    ws = torch.empty(max(256, oc.kvc_score_workspace_size(b.shape, b.kview(), False)), dtype=torch.uint8,
                     device="cuda")
    oc.kvc_score(b.shape, b.q, b.kview(), b.lse, b.bias, scores, ws)
    oc.kvc_attention_mass(b.shape, b.q, b.kview(), b.lse, b.bias, mass, ws)
    lse = None
    if with_lse:
        lse = torch.zeros((w.S, w.H * w.G, w.q), dtype=torch.float32, device="cuda")
        oc.kvc_lse(b.shape, b.q, b.kview(), b.bias, lse, ws)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), mass.cpu().numpy(), None if lse is None else lse.cpu().numpy()


@pytest.mark.parametrize("case", ["mfma_action_bias", "mfma_two_row_blocks", "mfma_paged", "valu_f32", "valu_bf16",
                                  "supplied_lse"])
def test_causal_scores_mass_and_lse_match_oracle(case):
    P, oc = _P(), _oc()
    w, kind = _workload(case)
    rp = W.row_positions(w, kind)
    say(f"[case] causal {case}: S={w.S} H={w.H} R={w.R} n={list(w.n)} {w.dtype} positions {kind}")
    data = W.build_paged(w) if w.paged else W.build_contiguous(w)
    lse_in = None
    if case == "supplied_lse":
        lse_in = np.zeros((w.S, w.H * w.G, w.q), dtype=np.float32)
        for h in range(w.H):
            _, L = O.causal_unit(O.unit_rows(data["Q"], 0, h, w.G), data["K"][0, h, :w.n[0]],
                                 rp[0, h * w.G:(h + 1) * w.G].reshape(-1), w.dtype, w.logit_scale)
            lse_in[0, h * w.G:(h + 1) * w.G] = (L + 0.25).astype(np.float32).reshape(w.G, w.q)  # a superset's LSE
    b = _batch(w, data, lse_in)
    b.shape.row_pos = P.device_tensor(rp)
    sc, ma, lse = _run_all(oc, b, w, with_lse=lse_in is None)
    for s in range(w.S):
        n = w.n[s]
        bias = None if data["bias"] is None else data["bias"][s, :n]
        for h in range(w.H):
            tag = f"causal {case} s={s} h={h}"
            rows = O.unit_rows(data["Q"], s, h, w.G)
            pos = rp[s, h * w.G:(h + 1) * w.G].reshape(-1)
            lrows = None if lse_in is None else lse_in[s, h * w.G:(h + 1) * w.G].reshape(-1).astype(np.float64)
            keys = _keys(w, data, s, h)
            ref, L = O.causal_unit(rows, keys, pos, w.dtype, w.logit_scale, bias, lrows)
            mref, _ = O.causal_unit(rows, keys, pos, w.dtype, w.logit_scale, bias, lrows, power=1)
            check_scores(sc[s, h, :n], ref, tag + " score")
            check_scores(ma[s, h, :n], mref, tag + " mass")
            assert np.all(sc[s, h, n:] == -1.0) and np.all(ma[s, h, n:] == -1.0), f"{tag}: past n touched"
            if lse is not None:
                got = lse[s, h * w.G:(h + 1) * w.G].reshape(-1)
                sees = pos >= 0
                assert np.all(got[~sees] == -np.inf), f"{tag}: a row that sees no key has LSE -inf"
                np.testing.assert_allclose(got[sees], L[sees], rtol=2e-6, atol=2e-6, err_msg=tag)
                # each row that sees a key spreads a weight of 1 over what it sees
                assert abs(float(ma[s, h, :n].astype(np.float64).sum()) - sees.mean()) < 1e-4, tag
    say(f"[ok] causal {case}")


def test_causal_through_slot_map_with_dead_slots():
    P, oc = _P(), _oc()
    w = W.custom("causal_slot", 176, S=2, H=2, G=4, q=20, n=(2500, 900), dtype="bf16", keys="mixture",
                 queries="cluster", paged=True, table="permuted", block_size=16, bias_tail=0.5)
    data = W.build_paged(w)
    pool, smap, live, dead = slot_setup(w, data, 0.45, np.random.default_rng(8))
    rp = W.row_positions(w, "spread")
    say(f"[case] causal slot map: n={list(w.n)} dead share ~0.45")
    kv = oc.KView(P.device_tensor(pool), oc.KVC_BF16, 0, None, 0, P.device_tensor(smap), dead)
    shape = oc.Shape(w.S, w.H, w.G, w.q, w.d, w.n_max, np.array(w.n, dtype=np.int32), w.logit_scale,
                     row_pos=P.device_tensor(rp))
    dq = P.device_tensor(data["Q"])
    bias = P.device_tensor(data["bias"].astype(np.float32))
    ws = torch.empty(max(256, oc.kvc_score_workspace_size(shape, kv, False)), dtype=torch.uint8, device="cuda")
    scores = torch.full((w.S, w.H, w.n_max), -1.0, dtype=torch.float32, device="cuda")
    mass = torch.full_like(scores, -1.0)
    lse = torch.zeros((w.S, w.H * w.G, w.q), dtype=torch.float32, device="cuda")
    oc.kvc_score(shape, dq, kv, None, bias, scores, ws)
    oc.kvc_attention_mass(shape, dq, kv, None, bias, mass, ws)
    oc.kvc_lse(shape, dq, kv, bias, lse, ws)
    torch.cuda.synchronize()
    sc, ma, lg = scores.cpu().numpy(), mass.cpu().numpy(), lse.cpu().numpy()
    for s in range(w.S):
        n = w.n[s]
        for h in range(w.H):
            tag = f"causal slot s={s} h={h}"
            rows = O.unit_rows(data["Q"], s, h, w.G)
            keys = O.slot_unit_keys(pool, smap[s, h], n, h)
            pos = rp[s, h * w.G:(h + 1) * w.G].reshape(-1)
            lv = live[s, h, :n]
            ref, L = O.causal_unit_live(rows, keys, lv, pos, w.dtype, w.logit_scale, data["bias"][s, :n])
            mref, _ = O.causal_unit_live(rows, keys, lv, pos, w.dtype, w.logit_scale, data["bias"][s, :n], power=1)
            assert np.all(sc[s, h, :n][~lv] == 0) and np.all(ma[s, h, :n][~lv] == 0), f"{tag}: dead positions"
            check_scores(sc[s, h, :n], ref, tag + " score")
            check_scores(ma[s, h, :n], mref, tag + " mass")
            got = lg[s, h * w.G:(h + 1) * w.G].reshape(-1)
            fin = np.isfinite(L)
            assert np.all(got[~fin] == -np.inf), f"{tag}: rows without a visible live key"
            np.testing.assert_allclose(got[fin], L[fin], rtol=2e-6, atol=2e-6, err_msg=tag)
    say("[ok] causal slot map")


@pytest.mark.parametrize("case", ["mfma_one_head", "mfma_action_bias", "mfma_paged", "valu_f32"])
def test_mask_that_hides_nothing(case):
    """row_pos >= n - 1 everywhere takes the unmasked code only. On the VALU path every output
    equals the run without a mask bit for bit. The MFMA path takes causal rows query-major and
    splits the LSE pass into shorter key chunks, so there the same sums come in another order:
    equal to float32 rounding."""
    P, oc = _P(), _oc()
    if case == "mfma_one_head":
        w = W.custom("causal_g1", 178, S=2, H=2, G=1, q=40, n=(2100, 700), dtype="bf16", keys="mixture",
                     queries="cluster", bias_tail=0.5)
    else:
        w, _ = _workload(case)
    data = W.build_paged(w) if w.paged else W.build_contiguous(w)
    b = _batch(w, data)
    base = _run_all(oc, b, w)
    exact = w.dtype == "f32"
    for extra in (0, 7):
        b.shape.row_pos = P.device_tensor(W.row_positions(w, "all") + extra)
        got = _run_all(oc, b, w)
        for x, y, what in zip(base, got, ("scores", "mass", "lse")):
            if exact:
                assert np.array_equal(x, y), f"{case} +{extra}: {what} differ from the unmasked run"
            else:
                np.testing.assert_allclose(y, x, rtol=1e-5, atol=1e-30 if what != "lse" else 1e-5,
                                           err_msg=f"{case} +{extra}: {what}")
    say(f"[ok] causal nothing hidden {case}")


@pytest.mark.parametrize("case", ["mfma_two_row_blocks", "valu_f32"])
def test_mask_that_hides_everything(case):
    """No row sees a key: every score and mass is 0 and every LSE -inf."""
    P, oc = _P(), _oc()
    w, _ = _workload(case)
    data = W.build_contiguous(w)
    b = _batch(w, data)
    b.shape.row_pos = P.device_tensor(W.row_positions(w, "none"))
    sc, ma, lse = _run_all(oc, b, w)
    for s in range(w.S):
        n = w.n[s]
        assert np.all(sc[s, :, :n] == 0.0) and np.all(ma[s, :, :n] == 0.0)
    assert np.all(lse == -np.inf)
    say(f"[ok] causal everything hidden {case}")


def test_causal_score_select_compact_path():
    """The whole path with action-token rows: scores, exact top-m of them, the oracle's band,
    and the gathered K/V bit for bit."""
    P = _P()
    w = W.custom("causal_path", 177, S=2, H=2, G=4, q=40, n=(2600, 1100), dtype="bf16", keys="mixture",
                 queries="action")
    data = W.build_contiguous(w)
    rp = W.row_positions(w, "action")
    b = _batch(w, data)
    b.shape.row_pos = P.device_tensor(rp)
    o = P.allocate(b)
    P.run(b, o)
    torch.cuda.synchronize()
    scores, kept = P.host_array(o.scores), P.host_array(o.kept)
    k_out, v_out = P.host_array(o.k_out), P.host_array(o.v_out)
    for s in range(w.S):
        n, m = w.n[s], int(w.m[s])
        for h in range(w.H):
            tag = f"causal path s={s} h={h}"
            ref, _ = O.causal_unit(O.unit_rows(data["Q"], s, h, w.G), data["K"][s, h, :n],
                                   rp[s, h * w.G:(h + 1) * w.G].reshape(-1), w.dtype, w.logit_scale)
            check_scores(scores[s, h, :n], ref, tag)
            check_kept_form(kept[s, h], m, n, tag)
            check_selection_exact(kept[s, h], scores[s, h, :n], m, tag)
            check_selection_band(kept[s, h], ref, m, tag)
            check_gather(data["K"][s, h, :n], kept[s, h], k_out[s, h], m, tag + " K")
            check_gather(data["V"][s, h, :n], kept[s, h], v_out[s, h], m, tag + " V")
    say("[ok] causal path")
