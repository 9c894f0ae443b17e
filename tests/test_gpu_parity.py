"""GPU parity: the HIP path (through the C ABI) against the float64 oracle, element by element.

Small and medium cases span several key tiles, row tiles and LDS stages with ragged tails, both
scoring paths (MFMA and VALU), supplied and computed LSE, the per-key bias, contiguous and
paged layouts, and the degenerate budgets m = 0 and m = n.
"""
import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from tests.parity import (check_gather, check_kept_form, check_scores, check_selection_band,
                          check_selection_exact, say)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _P():
    from online_compaction_amd import path as P
    return P


def _lse_for(w, data, paged=False):
    """Oracle LSE for every unit, rounded to float32 [S][H*G][q] (a supplied input)."""
    out = np.zeros((w.S, w.H * w.G, w.q), dtype=np.float32)
    for s in range(w.S):
        b = None if data.get("bias") is None else data["bias"][s, :w.n[s]]
        for h in range(w.H):
            if paged:
                keys = O.paged_unit_keys(data["k_pool"], data["table"][s], w.n[s], h, w.block_size)
            else:
                keys = data["K"][s, h, :w.n[s]]
            L = O.lse_unit(O.unit_rows(data["Q"], s, h, w.G), keys, w.dtype, w.logit_scale, b)
            out[s, h * w.G:(h + 1) * w.G] = L.astype(np.float32).reshape(w.G, w.q)
    return out


def run_contig_case(w, supply_lse=False):
    P = _P()
    say(f"[case] contiguous {w}")
    data = W.build_contiguous(w)
    lse = _lse_for(w, data) if supply_lse else None
    ref = O.run_contiguous(data, w.G, w.dtype, w.logit_scale, lse_all=lse)
    b = P.contiguous_batch(data["Q"], data["K"], data["V"], data["n"], data["m"], w.G, w.logit_scale,
                           bias=data["bias"], lse=lse)
    o = P.allocate(b)
    P.run(b, o)
    torch.cuda.synchronize()
    scores, kept = P.host_array(o.scores), P.host_array(o.kept)
    k_out, v_out = P.host_array(o.k_out), P.host_array(o.v_out)
    worst, swaps = 0.0, 0
    for (s, h), r in ref.items():
        n, m = w.n[s], w.m[s]
        tag = f"{w.name} s={s} h={h}"
        worst = max(worst, check_scores(scores[s, h, :n], r["scores"], tag))
        check_kept_form(kept[s, h], m, n, tag)
        check_selection_exact(kept[s, h], scores[s, h, :n], m, tag)
        swaps += check_selection_band(kept[s, h], r["scores"], m, tag)
        check_gather(data["K"][s, h, :n], kept[s, h], k_out[s, h], m, tag + " K")
        check_gather(data["V"][s, h, :n], kept[s, h], v_out[s, h], m, tag + " V")
    say(f"[ok] {w.name}: worst score rel err {worst:.3g}, tie-band swaps {swaps}")
    return scores, kept


def expected_paged(data, w, kept_gpu):
    """Oracle plan + copy + table update applied to the GPU's kept sets (stage-wise check)."""
    k_pool = data["k_pool"].copy()
    v_pool = data["v_pool"].copy()
    table = data["table"].copy()
    freed = {}
    for s in range(w.S):
        n, m = w.n[s], w.m[s]
        plans = [O.paged_plan(n, m, w.block_size, kept_gpu[s, h, :m]) for h in range(w.H)]
        for h in range(w.H):
            O.apply_paged_copy(k_pool, v_pool, table[s], h, plans[h])
        table[s], freed[s] = O.table_update(table[s], n, m, w.block_size)
    return k_pool, v_pool, table, freed


def run_paged_case(w, supply_lse=False):
    P = _P()
    say(f"[case] paged {w}")
    data = W.build_paged(w)
    lse = _lse_for(w, data, paged=True) if supply_lse else None
    ref = O.run_paged(data, w.G, w.dtype, w.logit_scale, w.block_size, lse_all=lse)
    b = P.paged_batch(data["Q"], data["k_pool"], data["v_pool"], data["table"], data["n"], data["m"], w.G,
                      w.logit_scale, w.block_size, n_max=w.n_max, bias=data["bias"], lse=lse)
    o = P.allocate(b)
    P.run(b, o)
    torch.cuda.synchronize()
    scores, kept = P.host_array(o.scores), P.host_array(o.kept)
    worst = 0.0
    for (s, h), r in ref["units"].items():
        n, m = w.n[s], w.m[s]
        tag = f"{w.name} s={s} h={h}"
        worst = max(worst, check_scores(scores[s, h, :n], r["scores"], tag))
        check_kept_form(kept[s, h], m, n, tag)
        check_selection_exact(kept[s, h], scores[s, h, :n], m, tag)
        check_selection_band(kept[s, h], r["scores"], m, tag)
    ek, ev, et, ef = expected_paged(data, w, kept)
    assert np.array_equal(P.host_array(b.k_pool).view(np.uint8), ek.view(np.uint8)), "K pool differs"
    assert np.array_equal(P.host_array(b.v_pool).view(np.uint8), ev.view(np.uint8)), "V pool differs"
    assert np.array_equal(P.host_array(b.table), et), "block table differs"
    freed = P.host_array(o.freed)
    for s in range(w.S):
        F = len(ef[s])
        assert o.freed_counts[s] == F
        assert np.array_equal(freed[s, :F], ef[s]) and np.all(freed[s, F:] == -1), f"freed list of seq {s}"
    # end to end: where the GPU kept set equals the oracle's, the pools equal the oracle's too
    same = all(np.array_equal(kept[s, h, :w.m[s]], ref["units"][(s, h)]["kept"]) for (s, h) in ref["units"])
    if same:
        assert np.array_equal(P.host_array(b.k_pool).view(np.uint8), ref["k_pool"].view(np.uint8))
        assert np.array_equal(P.host_array(b.table), ref["table"])
    say(f"[ok] {w.name}: worst score rel err {worst:.3g}, end-to-end identical: {same}")


# ------------------------------------------------------------------------------------- contiguous

def test_c1_single_head_f32():
    run_contig_case(W.spec("c1"))


def test_f32_ragged_multi_seq_valu():
    run_contig_case(W.custom("f32_ragged", 101, S=3, H=2, G=2, q=5, n=(1, 300, 777)))


def test_bf16_small_rows_valu():
    run_contig_case(W.custom("bf16_r4", 102, S=2, H=3, G=1, q=4, n=(1000, 513), dtype="bf16", keys="mixture"))


def test_bf16_mfma_ragged_rows_and_keys():
    run_contig_case(W.custom("bf16_r21", 103, S=2, H=2, G=3, q=7, n=(1500, 517), dtype="bf16", keys="mixture",
                             queries="cluster"))


def test_bf16_mfma_many_row_stages():
    run_contig_case(W.custom("bf16_r600", 104, S=1, H=1, G=4, q=150, n=(2100,), dtype="bf16", keys="mixture",
                             queries="cluster"))


def test_bf16_mfma_lse_blocks_and_chunks():
    # R = 1100 spans three 512-row blocks; n = 5000 spans several key chunks
    run_contig_case(W.custom("bf16_r1100", 105, S=1, H=2, G=2, q=550, n=(5000,), dtype="bf16", keys="mixture",
                             queries="cluster"))


def test_bias_internal_lse_mfma_and_valu():
    run_contig_case(W.custom("bias_mfma", 106, S=2, H=2, G=2, q=20, n=(900, 1234), dtype="bf16",
                             keys="mixture", queries="cluster", bias_tail=0.5))
    run_contig_case(W.custom("bias_valu", 107, S=2, H=1, G=1, q=3, n=(700, 64), bias_tail=-1.25))


def test_supplied_lse_mfma_and_valu():
    run_contig_case(W.custom("lse_mfma", 108, S=2, H=2, G=4, q=33, n=(1800, 601), dtype="bf16", keys="mixture",
                             queries="cluster"), supply_lse=True)
    run_contig_case(W.custom("lse_valu", 109, S=1, H=2, G=1, q=6, n=(999,)), supply_lse=True)


def test_degenerate_budgets_contig():
    w = W.custom("budgets", 110, S=4, H=2, G=2, q=9, n=(50, 50, 1, 700), m=(0, 50, 1, 350), dtype="bf16",
                 keys="mixture", queries="cluster")
    run_contig_case(w)


def test_exact_ties_go_to_lower_position():
    P = _P()
    w = W.custom("ties", 111, S=1, H=1, G=2, q=8, n=(600,), m=(37,), dtype="bf16", keys="normal")
    data = W.build_contiguous(w)
    K = data["K"]
    # every key j >= 300 duplicates key j - 300, so scores tie exactly in pairs
    K[0, 0, 300:600] = K[0, 0, 0:300]
    b = P.contiguous_batch(data["Q"], K, data["V"], data["n"], data["m"], w.G, w.logit_scale)
    o = P.allocate(b)
    P.run(b, o)
    torch.cuda.synchronize()
    sc = P.host_array(o.scores)[0, 0]
    kept = P.host_array(o.kept)[0, 0]
    assert np.array_equal(sc[300:600].view(np.uint32), sc[0:300].view(np.uint32)), "duplicate keys score apart"
    check_selection_exact(kept, sc, 37, "ties")
    ks = set(kept.tolist())
    hi = [j for j in ks if j >= 300]
    assert all(j - 300 in ks for j in hi), "a duplicate at the higher position was kept over its twin"
    assert len(ks) - 2 * len(hi) == 1  # m is odd: exactly one twin pair is split, keeping the lower one


def test_deterministic_bits():
    P = _P()
    w = W.custom("det", 112, S=2, H=2, G=4, q=40, n=(3000, 1777), dtype="bf16", keys="mixture", queries="cluster")
    data = W.build_contiguous(w)
    b = P.contiguous_batch(data["Q"], data["K"], data["V"], data["n"], data["m"], w.G, w.logit_scale)
    o1, o2 = P.allocate(b), P.allocate(b)
    P.run(b, o1)
    P.run(b, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1.scores, o2.scores) and torch.equal(o1.kept, o2.kept)


def test_lse_entry_point():
    import online_compaction_amd as oc
    P = _P()
    for w in (W.custom("lse_ep_mfma", 113, S=2, H=2, G=2, q=70, n=(3000, 100), dtype="bf16", keys="mixture",
                       queries="cluster", bias_tail=0.25),
              W.custom("lse_ep_valu", 114, S=1, H=3, G=1, q=5, n=(1000,))):
        data = W.build_contiguous(w)
        b = P.contiguous_batch(data["Q"], data["K"], data["V"], data["n"], data["m"], w.G, w.logit_scale,
                               bias=data["bias"])
        out = torch.zeros((w.S, w.H * w.G, w.q), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(256, oc.kvc_lse_workspace_size(b.shape, b.kview())), dtype=torch.uint8, device="cuda")
        oc.kvc_lse(b.shape, b.q, b.kview(), b.bias, out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = _lse_for(w, data)
        np.testing.assert_allclose(got, ref, rtol=2e-6, atol=2e-6)
        say(f"[ok] lse {w.name}: max abs err {np.abs(got - ref).max():.3g}")


def _wide_range_inputs(seed, n, q, rising):
    """One unit whose logits span hundreds of nats: the first coordinate of key j follows a
    staircase (each 256-key step adds 400, so the running maximum jumps by ~35 nats per step when
    the query's first coordinate is positive and falls when it is negative) with isolated spikes;
    the other coordinates are small noise. bf16 bit patterns, [1][1][n][128] / [1][1][q][128]."""
    rng = np.random.default_rng(seed)
    d = 128
    K = rng.standard_normal((n, d)).astype(np.float32) * 0.5
    step = (np.arange(n) // 256).astype(np.float32)
    K[:, 0] = (-2000.0 + 400.0 * step) if rising else (2000.0 - 400.0 * step)
    spikes = rng.choice(n, size=max(1, n // 500), replace=False)
    K[spikes, 0] += 3000.0
    Q = rng.standard_normal((q, d)).astype(np.float32) * 0.5
    Q[:, 0] = rng.choice([-3.0, -1.0, 0.0, 0.5, 1.0, 3.0], size=q)
    return W.f32_to_bf16_bits(Q)[None, None], W.f32_to_bf16_bits(K)[None, None]


@pytest.mark.parametrize("rising", [True, False])
def test_lse_and_scores_wide_logit_ranges(rising):
    """Logits from about -700 to +1100 nats with jumps far beyond the float32 exponent range
    between tiles, chunks and rows: the LSE pass must follow every rise of the maximum."""
    import online_compaction_amd as oc
    P = _P()
    n, q = 5000, 48
    Q, K = _wide_range_inputs(201 if rising else 202, n, q, rising)
    V = np.zeros_like(K)
    scale = 1.0 / np.sqrt(128.0)
    say(f"[case] wide logit ranges, rising={rising}: n={n} rows={q}")
    b = P.contiguous_batch(Q, K, V, [n], [n // 5], 1, scale)
    out = torch.zeros((1, 1, q), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, oc.kvc_lse_workspace_size(b.shape, b.kview())), dtype=torch.uint8, device="cuda")
    oc.kvc_lse(b.shape, b.q, b.kview(), None, out, ws)
    o = P.allocate(b)
    P.run(b, o)
    torch.cuda.synchronize()
    rows = O.unit_rows(Q, 0, 0, 1)
    ref_lse = O.lse_unit(rows, K[0, 0], "bf16", scale)
    got = out.cpu().numpy().reshape(-1)
    np.testing.assert_allclose(got, ref_lse, rtol=2e-6, atol=2e-5)
    ref = O.score_unit(rows, K[0, 0], "bf16", scale)
    worst = check_scores(P.host_array(o.scores)[0, 0, :n], ref, "wide range")
    check_selection_band(P.host_array(o.kept)[0, 0], ref, n // 5, "wide range")
    say(f"[ok] wide logit ranges: LSE span {ref_lse.min():.0f}..{ref_lse.max():.0f}, "
        f"max LSE err {np.abs(got - ref_lse).max():.3g}, worst score rel err {worst:.3g}")


# ------------------------------------------------------------------------------------- paged

def test_paged_bf16_mfma_permuted():
    run_paged_case(W.custom("paged_mfma", 120, S=3, H=2, G=2, q=10, n=(100, 530, 1031), dtype="bf16",
                            keys="mixture", queries="cluster", paged=True, table="permuted", block_size=16))


def test_paged_f32_valu_bias():
    run_paged_case(W.custom("paged_valu", 121, S=2, H=3, G=1, q=4, n=(77, 400), paged=True, table="permuted",
                            block_size=16, bias_tail=0.5))


def test_paged_degenerate_budgets():
    run_paged_case(W.custom("paged_budgets", 122, S=4, H=2, G=2, q=8, n=(40, 40, 16, 333), m=(0, 40, 16, 1),
                            dtype="bf16", keys="mixture", queries="cluster", paged=True, table="permuted",
                            block_size=16))


def test_paged_supplied_lse():
    run_paged_case(W.custom("paged_lse", 123, S=2, H=2, G=4, q=12, n=(260, 1500), dtype="bf16", keys="mixture",
                            queries="cluster", paged=True, table="identity", block_size=16), supply_lse=True)


@pytest.mark.parametrize("case", ["subtiles9_contig", "subtiles9_paged_bias", "subtiles8_contig"])
def test_score_key_tile_variants(case):
    """The score kernel holds 4, 8 or 9 key subtiles per wave, picked from the workgroup count.
    Small cases run 4; these full-length trajectories with 16 proxy rows run the other two."""
    from tests.parity import score_key_subtiles
    if case == "subtiles9_contig":
        w = W.custom("kt9c", 121, S=1, H=8, G=4, q=4, n=(33000,), dtype="bf16", keys="mixture", queries="cluster")
    elif case == "subtiles9_paged_bias":
        w = W.custom("kt9p", 122, S=1, H=8, G=4, q=4, n=(33000,), dtype="bf16", keys="mixture", queries="cluster",
                     paged=True, table="permuted", block_size=16, bias_tail=0.5)
    else:
        w = W.custom("kt8c", 123, S=4, H=8, G=4, q=4, n=(33000,) * 4, dtype="bf16", keys="mixture",
                     queries="cluster")
    want = int(case[8])
    assert score_key_subtiles(list(w.n), w.H) == want, "the case no longer selects the variant it names"
    if w.paged:
        run_paged_case(w)
    else:
        run_contig_case(w)



@pytest.mark.parametrize("path", ["mfma_contig", "valu_contig", "mfma_paged"])
def test_more_sequences_than_one_launch_describes(path):
    """300 ragged sequences: every entry point splits them over several launches (one launch's
    argument table describes at most 128 sequences), with per-sequence offsets into the
    workspace, the outputs and the paged pool carried across the launches."""
    rng = np.random.default_rng(77)
    lens = tuple(int(x) for x in rng.integers(1, 400, size=300))
    if path == "valu_contig":
        w = W.custom("many_valu", 124, S=300, H=2, G=1, q=3, n=lens)
    else:
        w = W.custom(f"many_{path}", 125, S=300, H=2, G=4, q=4, n=lens, dtype="bf16", keys="mixture",
                     queries="cluster", paged=path == "mfma_paged", table="permuted", block_size=16)
    if w.paged:
        run_paged_case(w)
    else:
        run_contig_case(w)
