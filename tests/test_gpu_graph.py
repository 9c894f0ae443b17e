"""The hot path inside a captured HIP graph. The library allocates, clears and synchronises
nothing, so score -> select -> compact can be captured once and replayed; every replay must give
the eager result bit for bit, with eager work and synchronisations between the replays."""
import numpy as np
import pytest

import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _P():
    from online_compaction_amd import path as P
    return P


def _outputs(P, o, w, paged):
    """What the path writes: scores of positions < n_s, kept entries < m_s (and the gathers)."""
    sc, kp = P.host_array(o.scores), P.host_array(o.kept)
    out = [np.concatenate([sc[s, :, :w.n[s]].reshape(-1) for s in range(w.S)]),
           np.concatenate([kp[s, :, :w.m[s]].reshape(-1) for s in range(w.S)])]
    if not paged:
        out += [P.host_array(o.k_out), P.host_array(o.v_out)]
    return out


@pytest.mark.parametrize("layout", ["contiguous", "paged"])
def test_captured_pipeline_replays_equal_eager(layout):
    P = _P()
    paged = layout == "paged"
    w = W.custom(f"graph_{layout}", 190, S=2, H=2, G=4, q=24, n=(2100, 1337), dtype="bf16", keys="mixture",
                 queries="cluster", bias_tail=0.5, paged=paged, table="permuted" if paged else "identity",
                 block_size=16)
    print(f"[case] graph {layout}: S={w.S} H={w.H} R={w.R} n={list(w.n)}", flush=True)
    data = W.build_paged(w) if paged else W.build_contiguous(w)
    if paged:
        b = P.paged_batch(data["Q"], data["k_pool"], data["v_pool"], data["table"], data["n"], data["m"], w.G,
                          w.logit_scale, w.block_size, n_max=w.n_max, bias=data["bias"])
        pristine = (b.k_pool.clone(), b.v_pool.clone(), b.table.clone())
    else:
        b = P.contiguous_batch(data["Q"], data["K"], data["V"], data["n"], data["m"], w.G, w.logit_scale,
                               bias=data["bias"])
    o = P.allocate(b)

    def restore():
        if paged:
            b.k_pool.copy_(pristine[0])
            b.v_pool.copy_(pristine[1])
            b.table.copy_(pristine[2])

    # eager reference (after a warm-up call)
    P.run(b, o)
    restore()
    torch.cuda.synchronize()
    P.run(b, o)
    torch.cuda.synchronize()
    want = _outputs(P, o, w, paged)
    if paged:
        want += [P.host_array(b.k_pool), P.host_array(b.v_pool), P.host_array(b.table)]

    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            P.run(b, o)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work between the replays: clobber the outputs (and put the pool back); positions
        # past each n_s and m_s are not the path's to write
        o.scores.fill_(-7.0)
        o.kept.fill_(-7)
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(P, o, w, paged)
        if paged:
            got += [P.host_array(b.k_pool), P.host_array(b.v_pool), P.host_array(b.table)]
        names = ["scores", "kept", "k_out", "v_out"] if not paged else ["scores", "kept", "k_pool", "v_pool", "table"]
        for nm, a, e in zip(names, got, want):
            bad = np.flatnonzero(a.reshape(-1) != e.reshape(-1))
            assert bad.size == 0, (f"replay {rep}: {nm} differs from the eager run at {bad.size} entries, e.g. "
                                   f"{a.reshape(-1)[bad[:3]]} vs {e.reshape(-1)[bad[:3]]}")
    print(f"[ok] graph {layout}: 4 replays equal the eager run", flush=True)
