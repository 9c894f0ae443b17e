"""GPU parity of segment compaction: scoring, selecting and compacting one turn inside a longer
cache (contiguous and paged), and the delayed future-turn schedule that drives it."""
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


@pytest.mark.parametrize("dtype,keys", [("bf16", "mixture"), ("f32", "normal")])
def test_contiguous_segments(dtype, keys):
    P = _P()
    w = W.custom(f"seg_contig_{dtype}", 130, S=2, H=2, G=2, q=(40 if dtype == "bf16" else 3), n=(1500, 1500),
                 dtype=dtype, keys=keys, queries="cluster" if keys == "mixture" else "normal")
    data = W.build_contiguous(w)
    starts, lens = np.array([100, 37]), np.array([800, 1200])
    m = np.array([160, 240])
    say(f"[case] contiguous segments {dtype}: starts {starts.tolist()} lengths {lens.tolist()} m {m.tolist()}")
    b = P.contiguous_batch(data["Q"], data["K"], data["V"], lens, m, w.G, w.logit_scale, starts=starts)
    o = P.allocate(b)
    P.run(b, o)
    torch.cuda.synchronize()
    scores, kept = P.host_array(o.scores), P.host_array(o.kept)
    k_out, v_out = P.host_array(o.k_out), P.host_array(o.v_out)
    for s in range(w.S):
        a, n = int(starts[s]), int(lens[s])
        for h in range(w.H):
            tag = f"seg s={s} h={h}"
            seg = data["K"][s, h, a:a + n]
            ref = O.score_unit(O.unit_rows(data["Q"], s, h, w.G), seg, w.dtype, w.logit_scale)
            check_scores(scores[s, h, :n], ref, tag)
            check_kept_form(kept[s, h], int(m[s]), n, tag)
            check_selection_exact(kept[s, h], scores[s, h, :n], int(m[s]), tag)
            check_selection_band(kept[s, h], ref, int(m[s]), tag)
            check_gather(seg, kept[s, h], k_out[s, h], int(m[s]), tag + " K")
            check_gather(data["V"][s, h, a:a + n], kept[s, h], v_out[s, h], int(m[s]), tag + " V")
    say("[ok] contiguous segments")


def test_paged_segments_middle_and_tail():
    """Sequence 0 compacts a middle turn (320 tokens at 96, 184 tokens after it, m = 64);
    sequence 1 compacts its last turn (340 tokens at 160, m = 70)."""
    P = _P()
    w = W.custom("seg_paged", 131, S=2, H=2, G=2, q=24, n=(600, 500), dtype="bf16", keys="mixture",
                 queries="cluster", paged=True, table="permuted", block_size=16)
    data = W.build_paged(w)
    starts, lens, m, clen = np.array([96, 160]), np.array([320, 340]), np.array([64, 70]), np.array([600, 500])
    b = P.paged_batch(data["Q"], data["k_pool"], data["v_pool"], data["table"], lens, m, w.G, w.logit_scale, 16,
                      n_max=int(lens.max()), starts=starts, cache_lens=clen)
    o = P.allocate(b)
    P.run(b, o)
    torch.cuda.synchronize()
    scores, kept = P.host_array(o.scores), P.host_array(o.kept)
    kp, vp, table = data["k_pool"].copy(), data["v_pool"].copy(), data["table"].copy()
    for s in range(w.S):
        a, n, ms, L = int(starts[s]), int(lens[s]), int(m[s]), int(clen[s])
        plans = []
        for h in range(w.H):
            tag = f"paged seg s={s} h={h}"
            keys = O.paged_unit_keys(data["k_pool"], data["table"][s], L, h, 16)[a:a + n]
            ref = O.score_unit(O.unit_rows(data["Q"], s, h, w.G), keys, w.dtype, w.logit_scale)
            check_scores(scores[s, h, :n], ref, tag)
            check_selection_exact(kept[s, h], scores[s, h, :n], ms, tag)
            check_selection_band(kept[s, h], ref, ms, tag)
            plans.append(O.paged_plan(n, ms, 16, kept[s, h, :ms]))
        for h in range(w.H):
            O.apply_paged_copy(kp, vp, table[s], h, plans[h], offset=a)
        table[s], freed = O.table_update_segment(table[s], a, n, L, ms, 16)
        F = len(freed)
        assert o.freed_counts[s] == F
        assert np.array_equal(P.host_array(o.freed)[s, :F], freed)
    assert np.array_equal(P.host_array(b.k_pool), kp) and np.array_equal(P.host_array(b.v_pool), vp)
    assert np.array_equal(P.host_array(b.table), table)
    say(f"[ok] paged segments: freed {o.freed_counts.tolist()} blocks")


def test_delayed_turn_compaction_session():
    """A 9-turn session, delay 1: at the end of each turn the previous one is compacted with this
    turn's queries. The mirror below replays the same schedule on the host with the oracle (its
    own bookkeeping, stage-wise on the GPU's kept sets) and must hold identical bytes."""
    P = _P()
    from online_compaction_amd.schedule import DelayedCompactor
    B, H, G, d = 16, 2, 2, 128
    nblocks, max_blocks = 160, 160
    rng = np.random.default_rng(7)
    lens = [int(x) for x in rng.integers(40, 300, size=9)]
    qs = [int(x) for x in rng.integers(6, 20, size=9)]
    scale = 1.0 / np.sqrt(d)
    k_pool = np.zeros((nblocks, B, H, d), dtype=np.uint16)
    v_pool = np.zeros_like(k_pool)
    table = np.full((1, max_blocks), -1, dtype=np.int32)
    dev_k, dev_v, dev_t = P.device_tensor(k_pool), P.device_tensor(v_pool), P.device_tensor(table)
    comp = DelayedCompactor(dev_k, dev_v, dev_t, B, H, G, scale, delay=1, ratio=0.2)
    fresh = list(range(nblocks))
    mirror_turns = []  # [start, length]
    L = 0
    for t, (n_t, q_t) in enumerate(zip(lens, qs)):
        # the engine appends the turn: new blocks from the free list, K/V rows written in place
        while -(-(L + n_t) // B) > int(np.count_nonzero(table[0] >= 0)):
            blk = comp.free_blocks.pop(0) if comp.free_blocks else fresh.pop(0)
            table[0, int(np.count_nonzero(table[0] >= 0))] = blk
        kv = W.f32_to_bf16_bits(rng.standard_normal((2, n_t, H, d), dtype=np.float32))
        for i in range(n_t):
            p = L + i
            k_pool[table[0, p // B], p % B] = kv[0, i]
            v_pool[table[0, p // B], p % B] = kv[1, i]
        # proxy rows of this turn look back at random earlier tokens
        base = rng.integers(0, max(L, 1), size=q_t)
        q = rng.standard_normal((H * G, q_t, d), dtype=np.float32) * 0.5
        for hq in range(H * G):
            h = hq // G
            for r in range(q_t):
                p = int(base[r])
                if L:
                    q[hq, r] += W.bf16_bits_to_f32(k_pool[table[0, p // B], p % B, h])
        qb = W.f32_to_bf16_bits(q)
        dev_k.copy_(P.device_tensor(k_pool))
        dev_v.copy_(P.device_tensor(v_pool))
        dev_t.copy_(P.device_tensor(table))
        mirror_turns.append([L, n_t, qb])
        L += n_t
        done = comp.append_turn(n_t, P.device_tensor(qb))
        torch.cuda.synchronize()
        # mirror: the turn one back is compacted over its whole inner blocks with this turn's rows
        if t >= 1:
            st, ln, _ = mirror_turns[t - 1]
            a, e = -(-st // B) * B, (st + ln) // B * B
            n = e - a
            if n > 0:
                m = min(n, -(-int(np.floor(0.2 * n + 0.5)) // B) * B)
                assert len(done) == 1 and (done[0].start, done[0].n, done[0].m) == (a, n, m)
                kept = P.host_array(done[0].kept)
                sc = P.host_array(done[0].scores)
                plans = []
                for h in range(H):
                    keys = O.paged_unit_keys(k_pool, table[0], L, h, B)[a:a + n]
                    rows = O.unit_rows(qb[None], 0, h, G)
                    ref = O.score_unit(rows, keys, "bf16", scale)
                    check_scores(sc[0, h, :n], ref, f"turn {t - 1} h={h}")
                    check_selection_exact(kept[0, h], sc[0, h, :n], m, f"turn {t - 1} h={h}")
                    check_selection_band(kept[0, h], ref, m, f"turn {t - 1} h={h}")
                    plans.append(O.paged_plan(n, m, B, kept[0, h]))
                for h in range(H):
                    O.apply_paged_copy(k_pool, v_pool, table[0], h, plans[h], offset=a)
                table[0], freed = O.table_update_segment(table[0], a, n, L, m, B)
                assert done[0].freed == freed.tolist()
                shift = len(freed) * B
                mirror_turns[t - 1][1] -= shift
                mirror_turns[t][0] -= shift
                L -= shift
            else:
                assert not done
        assert comp.length == L
        assert np.array_equal(P.host_array(dev_t), table), f"block table after turn {t}"
        live = -(-L // B)
        for lb in range(live):
            blk = table[0, lb]
            assert np.array_equal(P.host_array(dev_k[blk]), k_pool[blk]), f"K block {blk} after turn {t}"
            assert np.array_equal(P.host_array(dev_v[blk]), v_pool[blk]), f"V block {blk} after turn {t}"
    say(f"[ok] session of {len(lens)} turns: cache {sum(lens)} -> {L} tokens, {len(comp.free_blocks)} blocks free")
