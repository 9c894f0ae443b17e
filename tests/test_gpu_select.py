"""kvc_select_topm on given float32 scores, bit-exact against the oracle's top-m.

The scores are inputs here (seeded rows from workloads.score_rows), so selection is compared
exactly: the oracle orders the same float32 values widened to float64. Launches are shaped so
that their longest sequence falls in every size class of the register-resident kernel and past
it (the global-memory kernel), with mixed lengths, exact ties, zeros, subnormals, one-binade
rows and the budget edge cases m = 0, 1, n/5, n - 1, n."""
import numpy as np
import pytest

import workloads as W
from oracle import oracle as O
from tests.parity import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LAUNCHES = [
    (1, 64, 1000, 8192),        # longest fits 8 per thread
    (8193, 16384),              # 16
    (16385, 24576, 3),          # 24
    (24577, 36864, 33000),      # 36
    (36865, 49152),             # 48
    (49153, 70000, 500),        # global-memory kernel
]
KINDS = ["uniform", "levels", "zeros", "tiny", "narrow"]


def _budget(n: int, pick: int) -> int:
    return (0, 1, (n + 2) // 5, n - 1, n)[pick % 5] if n > 1 else pick % 2


@pytest.mark.parametrize("kind", KINDS)
def test_select_matches_oracle_exactly(kind):
    from online_compaction_amd import _abi as A
    from online_compaction_amd import path as P
    H = 2
    for li, lens in enumerate(LAUNCHES):
        S, n_max = len(lens), max(lens)
        sc = np.stack([W.score_rows(10 * li + h, lens, kind, n_max) for h in range(H)], axis=1)  # [S][H][n_max]
        m = [_budget(n, s + li + KINDS.index(kind)) for s, n in enumerate(lens)]
        m_max = max(1, max(m))
        say(f"[case] select {kind}: lens={lens} m={m}")
        shape = A.Shape(S, H, 1, 1, 128, n_max, list(lens), 1.0)
        scores = P.device_tensor(sc)
        kept = torch.full((S, H, m_max), -7, dtype=torch.int32, device="cuda")
        A.kvc_select_topm(shape, scores, m, m_max, kept)
        torch.cuda.synchronize()
        got = P.host_array(kept)
        for s, n in enumerate(lens):
            for h in range(H):
                ref = O.select_topm(sc[s, h, :n].astype(np.float64), m[s])
                assert np.array_equal(got[s, h, :m[s]], ref), f"{kind} lens={lens} s={s} h={h} m={m[s]}"
                assert np.all(got[s, h, m[s]:] == -7), f"{kind}: rows past m written (s={s} h={h})"
    say(f"[ok] select {kind}: {len(LAUNCHES)} launches exact")
