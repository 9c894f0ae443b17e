"""GPU parity of ActKV's retention path: attention mass, the action-critical set with the LRFU
step, side arrays carried through compaction, and a whole policy session mirrored by the oracle."""
import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from tests.parity import check_kept_form, check_scores, check_selection_exact, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DECAY = 2.0 ** -0.5


def _P():
    from online_compaction_amd import path as P
    return P


def _oc():
    import online_compaction_amd as oc
    return oc


# ------------------------------------------------------------------------- attention mass

@pytest.mark.parametrize("case", ["mfma_bias", "mfma_paged", "valu_f32", "supplied_lse"])
def test_attention_mass_matches_oracle(case):
    P, oc = _P(), _oc()
    if case == "mfma_bias":
        w = W.custom("mass_mfma", 140, S=2, H=2, G=4, q=40, n=(2100, 700), dtype="bf16", keys="mixture",
                     queries="cluster", bias_tail=0.5)
    elif case == "mfma_paged":
        w = W.custom("mass_paged", 141, S=2, H=2, G=2, q=24, n=(1000, 1333), dtype="bf16", keys="mixture",
                     queries="cluster", paged=True, table="permuted", block_size=16)
    elif case == "valu_f32":
        w = W.custom("mass_valu", 142, S=1, H=3, G=1, q=7, n=(900,))
    else:
        w = W.custom("mass_lse", 143, S=1, H=2, G=4, q=20, n=(1500,), dtype="bf16", keys="mixture",
                     queries="cluster")
    say(f"[case] attention mass {case}: S={w.S} H={w.H} R={w.R} n={list(w.n)} {w.dtype}")
    data = W.build_paged(w) if w.paged else W.build_contiguous(w)
    lse = None
    if case == "supplied_lse":
        lse = np.zeros((w.S, w.H * w.G, w.q), dtype=np.float32)
        for h in range(w.H):
            L = O.lse_unit(O.unit_rows(data["Q"], 0, h, w.G), data["K"][0, h, :w.n[0]], w.dtype, w.logit_scale)
            lse[0, h * w.G:(h + 1) * w.G] = (L + 0.25).astype(np.float32).reshape(w.G, w.q)  # a superset's LSE
    if w.paged:
        b = P.paged_batch(data["Q"], data["k_pool"], data["v_pool"], data["table"], data["n"], data["m"], w.G,
                          w.logit_scale, w.block_size, n_max=w.n_max, bias=data["bias"])
    else:
        b = P.contiguous_batch(data["Q"], data["K"], data["V"], data["n"], data["m"], w.G, w.logit_scale,
                               bias=data["bias"], lse=lse)
    mass = torch.zeros((w.S, w.H, w.n_max), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(256, oc.kvc_score_workspace_size(b.shape, b.kview(), False)), dtype=torch.uint8,
                     device="cuda")
    oc.kvc_attention_mass(b.shape, b.q, b.kview(), b.lse, b.bias, mass, ws)
    torch.cuda.synchronize()
    got = mass.cpu().numpy()
    for s in range(w.S):
        n = w.n[s]
        bias = None if data["bias"] is None else data["bias"][s, :n]
        for h in range(w.H):
            keys = (O.paged_unit_keys(data["k_pool"], data["table"][s], n, h, w.block_size) if w.paged
                    else data["K"][s, h, :n])
            lrows = None if lse is None else lse[s, h * w.G:(h + 1) * w.G].reshape(-1).astype(np.float64)
            ref = O.mass_unit(O.unit_rows(data["Q"], s, h, w.G), keys, w.dtype, w.logit_scale, bias, lrows)
            worst = check_scores(got[s, h, :n], ref, f"mass {case} s={s} h={h}")
            want_sum = 1.0 if lse is None else float(ref.sum())
            assert abs(float(got[s, h, :n].astype(np.float64).sum()) - want_sum) < 1e-4
    say(f"[ok] attention mass {case}: worst rel err {worst:.3g}")


# ------------------------------------------------------------------------- LRFU step

def _masses(rng, n, kind):
    if kind == "ties":
        vals = rng.choice(np.array([0.0, 1.0, 2.0, 3.0, 5.0, 8.0]), size=n)
    elif kind == "zero":
        return np.zeros(n, dtype=np.float32)
    elif kind == "peaked":
        vals = rng.exponential(1.0, size=n) ** 6
    else:
        vals = rng.random(n)
    vals = vals / max(vals.sum(), 1e-300)
    return vals.astype(np.float32)


# length sets whose longest sequence selects each kernel variant: 8, 16 and 36 positions per
# thread held in registers, and the global-memory kernel past 36864
LRFU_LENS = [(5000, 777, 3), (16000, 9000, 1), (33000, 20000, 64), (40000, 100, 5)]


@pytest.mark.parametrize("top_p,lens", [(0.9, LRFU_LENS[0]), (0.5, LRFU_LENS[0]), (1.0, LRFU_LENS[0]),
                                        (0.9, LRFU_LENS[1]), (0.5, LRFU_LENS[2]), (0.9, LRFU_LENS[2]),
                                        (0.9, LRFU_LENS[3])])
def test_lrfu_update_critical_set_exact(top_p, lens):
    oc = _oc()
    rng = np.random.default_rng([int(top_p * 100), lens[0]])
    lens = list(lens)
    S, H, n_max = 3, 3, max(lens)
    kinds = [["ties", "uniform", "peaked"], ["zero", "ties", "peaked"], ["uniform", "ties", "zero"]]
    mass = np.zeros((S, H, n_max), dtype=np.float32)
    for s in range(S):
        for h in range(H):
            mass[s, h, :lens[s]] = _masses(rng, lens[s], kinds[s][h])
    state0 = (rng.random((S, H, n_max)) * 3).astype(np.float32)
    say(f"[case] lrfu update top_p={top_p}: lens {lens}")
    shape = oc.Shape(S, H, 1, 1, 128, n_max, np.array(lens, dtype=np.int32), 1.0)
    dm = torch.from_numpy(mass).cuda()
    st = torch.from_numpy(state0).cuda()
    zero = torch.zeros_like(st)
    counts = torch.zeros((S, H), dtype=torch.int32, device="cuda")
    oc.kvc_lrfu_update(shape, dm, top_p, DECAY, st, counts)
    oc.kvc_lrfu_update(shape, dm, top_p, DECAY, zero)
    torch.cuda.synchronize()
    st, zero, counts = st.cpu().numpy(), zero.cpu().numpy(), counts.cpu().numpy()
    for s in range(S):
        n = lens[s]
        for h in range(H):
            want = O.action_critical(mass[s, h, :n], top_p)
            assert np.array_equal(zero[s, h, :n], want.astype(np.float32)), f"critical set s={s} h={h}"
            assert counts[s, h] == want.sum()
            ref = O.lrfu_step(state0[s, h, :n], want, DECAY)
            np.testing.assert_allclose(st[s, h, :n], ref, rtol=2e-7, atol=0)
            assert np.array_equal(st[s, h, n:], state0[s, h, n:]), "entries past n_s must stay untouched"
    say(f"[ok] lrfu update top_p={top_p}: critical sizes {counts.tolist()}")


# ------------------------------------------------------------------------- side arrays

@pytest.mark.parametrize("B", [0, 16])
def test_compact_side_follows_the_compaction(B):
    oc = _oc()
    rng = np.random.default_rng(50 + B)
    S, H, n_max = 2, 3, 3000
    lens, m = [2900, 1000], [700, 1000]
    starts = [37, 60] if B == 0 else None
    if B == 0:
        n_max = 3000
    else:
        m = [700, 333]
    m_max = max(m)
    kept = np.zeros((S, H, m_max), dtype=np.int32)
    for s in range(S):
        for h in range(H):
            kept[s, h, :m[s]] = np.sort(rng.choice(lens[s], size=m[s], replace=False))
    src = rng.random((S, H, n_max)).astype(np.float32)
    say(f"[case] compact side B={B}: lens {lens} m {m}")
    shape = oc.Shape(S, H, 1, 1, 128, n_max, np.array(lens, dtype=np.int32), 1.0,
                     None if starts is None else np.array(starts, dtype=np.int32))
    dst = torch.full((S, H, m_max), -1.0, dtype=torch.float32, device="cuda")
    oc.kvc_compact_side(shape, B, torch.from_numpy(kept).cuda(), m, m_max, torch.from_numpy(src).cuda(), dst)
    torch.cuda.synchronize()
    dst = dst.cpu().numpy()
    for s in range(S):
        a = 0 if starts is None else starts[s]
        for h in range(H):
            order = O.side_order(lens[s], m[s], B, kept[s, h, :m[s]])
            assert np.array_equal(dst[s, h, :m[s]], src[s, h, a + np.array(order, dtype=np.int64)])
            assert np.all(dst[s, h, m[s]:] == -1.0)
    say(f"[ok] compact side B={B}")


# ------------------------------------------------------------------------- whole policy

def test_actkv_policy_session_mirror():
    """Eight policy steps on a paged cache with a small ratchet (64 x 1.75, cap 300): every
    step's mass, critical set, LRFU state, eviction, pools, table and carried state match the
    oracle replaying the same steps on the host (stage-wise on the GPU's own masses)."""
    P = _P()
    from online_compaction_amd.actkv import ActKVRetention, BudgetRatchet
    B, H, G, d, q = 16, 2, 2, 128, 12
    nblocks, max_blocks = 96, 64
    rng = np.random.default_rng(21)
    scale = 1.0 / np.sqrt(d)
    k_pool = np.zeros((nblocks, B, H, d), dtype=np.uint16)
    v_pool = np.zeros_like(k_pool)
    table = np.full((1, max_blocks), -1, dtype=np.int32)
    dk, dv, dt = P.device_tensor(k_pool), P.device_tensor(v_pool), P.device_tensor(table)
    pol = ActKVRetention(dk, dv, dt, B, H, G, scale, ratchet=BudgetRatchet(initial=64, factor=1.75, cap=300))
    fresh = list(range(nblocks))
    state = np.zeros((H, max_blocks * B), dtype=np.float64)
    L = 0
    for t in range(8):
        n_new = int(rng.integers(40, 130))
        while -(-(L + n_new) // B) > int(np.count_nonzero(table[0] >= 0)):
            blk = pol.free_blocks.pop(0) if pol.free_blocks else fresh.pop(0)
            table[0, int(np.count_nonzero(table[0] >= 0))] = blk
        kv = W.f32_to_bf16_bits(rng.standard_normal((2, n_new, H, d), dtype=np.float32))
        for i in range(n_new):
            p = L + i
            k_pool[table[0, p // B], p % B] = kv[0, i]
            v_pool[table[0, p // B], p % B] = kv[1, i]
        dk.copy_(P.device_tensor(k_pool))
        dv.copy_(P.device_tensor(v_pool))
        dt.copy_(P.device_tensor(table))
        L += n_new
        # action rows attend to a few recent spans
        qf = rng.standard_normal((H * G, q, d), dtype=np.float32) * 0.5
        for hq in range(H * G):
            for r in range(q):
                p = int(rng.integers(max(0, L - 150), L))
                qf[hq, r] += W.bf16_bits_to_f32(k_pool[table[0, p // B], p % B, hq // G])
        qb = W.f32_to_bf16_bits(qf)
        out = pol.update(n_new, P.device_tensor(qb), expand=t in (2, 5))
        torch.cuda.synchronize()
        mass = P.host_array(out["mass"])[0]
        crit = P.host_array(out["critical"])[0]
        for h in range(H):
            keys = O.paged_unit_keys(k_pool, table[0], L, h, B)
            ref = O.mass_unit(O.unit_rows(qb[None], 0, h, G), keys, "bf16", scale)
            check_scores(mass[h, :L], ref, f"step {t} mass h={h}")
            hit = O.action_critical(mass[h, :L], 0.9)
            assert crit[h] == hit.sum()
            state[h, :L] = O.lrfu_step(state[h, :L], hit, 2.0 ** -0.5)
        pre = P.host_array(pol.state)[0]
        np.testing.assert_allclose(pre[:, :L], state[:, :L], rtol=1e-6)
        assert np.all(pre[:, L:] == 0)
        state[:, :L] = pre[:, :L]  # continue from the GPU's float32 state (stage-wise)
        ev = pol.evict()
        torch.cuda.synchronize()
        if ev["evicted"]:
            m = out["budget"]
            kept = P.host_array(ev["kept"])[0]
            plans = []
            for h in range(H):
                check_kept_form(kept[h], m, L, f"step {t} h={h}")
                check_selection_exact(kept[h], pre[h, :L], m, f"step {t} h={h}")
                plans.append(O.paged_plan(L, m, B, kept[h, :m]))
                state[h, :m] = pre[h, np.array(O.side_order(L, m, B, kept[h, :m]), dtype=np.int64)]
                state[h, m:] = 0.0
            for h in range(H):
                O.apply_paged_copy(k_pool, v_pool, table[0], h, plans[h])
            table[0], freed = O.table_update(table[0], L, m, B)
            assert ev["freed"] == len(freed)
            L = m
            assert np.array_equal(P.host_array(dt), table), f"table after step {t}"
            for lb in range(-(-L // B)):
                blk = table[0, lb]
                assert np.array_equal(P.host_array(dk[blk]), k_pool[blk]), f"K block {blk} after step {t}"
                assert np.array_equal(P.host_array(dv[blk]), v_pool[blk]), f"V block {blk} after step {t}"
            post = P.host_array(pol.state)[0]
            assert np.array_equal(post[:, :L], state[:, :L].astype(np.float32)), "carried state"
            assert np.all(post[:, L:] == 0)
        assert pol.length == L
        say(f"[ok] step {t}: n={out['n']} budget {out['budget']} critical {crit.tolist()} "
            f"{'evicted to ' + str(L) if ev['evicted'] else 'kept all'}")
    assert pol.ratchet.expansions == 2
