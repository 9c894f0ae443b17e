"""The seeded input generators: determinism, shapes and the workload constants (CPU only)."""
import numpy as np
import pytest

import workloads as W
from workloads.gen import action_positions, ratio_budget


def test_budgets_match_the_stated_workloads():
    assert W.spec("c1").m == (819,)
    assert W.spec("c2a").m == (3277,) and W.spec("c2b").m == (3277,)
    assert W.spec("c3").m[0] == 6600 and len(W.spec("c3").m) == 36
    assert [W.spec("c4", k).m[0] for k in range(7)] == [512, 896, 1568, 2744, 4802, 8403, 14706]
    assert ratio_budget(5) == 1 and ratio_budget(7) == 1 and ratio_budget(8) == 2


def test_shapes_of_named_workloads():
    c3 = W.spec("c3")
    assert (c3.S, c3.H, c3.G, c3.q, c3.d, c3.R) == (36, 8, 4, 1024, 128, 4096)
    c5 = W.spec("c5")
    assert (c5.S, c5.H, c5.G, c5.q, c5.R) == (64, 4, 8, 256, 2048)
    assert all(8192 <= n <= 131072 for n in c5.n)
    assert c5.max_blocks == 8192 and c5.paged
    c4 = W.spec("c4", 3)
    assert c4.R == 1320 and c4.max_blocks == 2063 and c4.bias_tail == 0.5


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 ties -> 1 + 2^-6
    got = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.015625 and got[3] == -2.5
    assert np.isfinite(got[4])


def test_generation_is_deterministic_and_per_unit():
    w = W.custom(n=(100, 60), S=2, H=2, G=2, q=3, dtype="bf16", keys="mixture", queries="cluster")
    a = W.build_contiguous(w)
    b = W.build_contiguous(w)
    for key in ("K", "V", "Q"):
        np.testing.assert_array_equal(a[key], b[key])
    np.testing.assert_array_equal(a["K"][1, 0, :60], W.unit_keys(w, 1, 0))
    assert not np.array_equal(W.unit_keys(w, 0, 0), W.unit_keys(w, 0, 1))
    assert np.all(a["K"][1, :, 60:] == 0)


def test_parallel_generation_matches_serial():
    w = W.custom(n=(50, 70, 30), S=3, H=2, dtype="bf16", keys="mixture", queries="cluster", G=2, q=2)
    a = W.build_contiguous(w, workers=1)
    b = W.build_contiguous(w, workers=3)
    np.testing.assert_array_equal(a["K"], b["K"])
    np.testing.assert_array_equal(a["Q"], b["Q"])


def test_mixture_sinks_are_scaled():
    w = W.custom(n=(200,), keys="mixture")
    k = W.unit_keys(w, 0, 0)
    norms = np.linalg.norm(k, axis=1)
    assert norms[:4].min() > 3 * np.median(norms[4:])


def test_action_spans_disjoint_and_in_range():
    w = W.spec("c4", 0)
    pos = action_positions(w, 0)
    assert len(pos) == 330 and len(set(pos.tolist())) == 330
    assert pos.min() >= 4 and pos.max() < 33000
    assert np.count_nonzero(np.diff(pos) != 1) == 9  # ten runs


def test_bias_tail():
    b = W.bias_row(W.spec("c4", 0), 0)
    assert b.shape == (33000,) and np.all(b[:24750] == 0) and np.all(b[24750:] == 0.5)
    assert W.bias_row(W.spec("c3"), 0) is None


def test_paged_layout_and_permuted_table():
    w = W.custom(n=(37, 16, 5), S=3, H=3, paged=True, table="permuted", block_size=4, dtype="bf16",
                 keys="mixture")
    d = W.build_paged(w)
    t = d["table"]
    ids = np.concatenate([t[s, :w.blocks_of(s)] for s in range(3)])
    assert sorted(ids.tolist()) == list(range(d["k_pool"].shape[0]))
    for s in range(3):
        for h in range(3):
            k = W.unit_keys(w, s, h)
            for j in (0, w.n[s] - 1):
                np.testing.assert_array_equal(d["k_pool"][t[s, j // 4], j % 4, h], k[j])
        assert np.all(t[s, w.blocks_of(s):] == -1)


def test_c5_lengths_fixed_by_seed():
    assert W.spec("c5").n == W.spec("c5").n
    assert len(W.spec("c5").n) == 64


def test_device_normal_generator_is_seeded():
    """The on-device generator (used for multi-GiB inputs) is a function of its seed: the same
    seed gives the same bfloat16 values, another seed other values, and the values are standard
    normal rounded to bfloat16 (checked here on the CPU device)."""
    torch = pytest.importorskip("torch")
    a = W.device_normal_bf16((3, 1000, 128), seed=7, device="cpu")
    b = W.device_normal_bf16((3, 1000, 128), seed=7, device="cpu")
    c = W.device_normal_bf16((3, 1000, 128), seed=8, device="cpu")
    assert a.dtype == torch.bfloat16 and a.shape == (3, 1000, 128)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not torch.equal(a.view(torch.int16), c.view(torch.int16))
    x = a.float()
    assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1.0) < 0.02
    # every value is a bfloat16 (the low 16 bits of its float32 pattern are zero)
    assert int((x.view(torch.int32) & 0xFFFF).abs().sum()) == 0
