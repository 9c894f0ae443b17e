"""The committed counter summaries of the score kernel parse, and the figures the benchmark
derives from them agree with the raw counts they state (no GPU: reads text files only)."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_summaries_match_the_score_kernel_source(bench):
    for path in (bench.TRAFFIC_FILE, bench.COUNTERS_FILE):
        assert bench._profile_fields(path, check_source=False) is not None, f"{path} is missing"
        if bench._profile_fields(path) is None:
            pytest.skip(f"{os.path.basename(path)} predates the score kernel's source: the benchmark reports null")


def test_serialized_bound_adds_up(bench):
    kv = bench._profile_fields(bench.COUNTERS_FILE, check_source=False)
    sb = bench.serialized_bound_from_profile(float(kv["serialized_bound_ms"]), check_source=False)
    assert sb["frac"] == pytest.approx(1.0)
    assert sb["ms"] == pytest.approx(sb["mfma_ms"] + sb["valu_ms"], rel=1e-3)
    # VALU: one wave64 instruction occupies a SIMD for 4 cycles at 2.4 GHz
    assert sb["valu_ms"] == pytest.approx(float(kv["valu_insts_per_simd"]) * 4 / 2.4e9 * 1e3, rel=1e-3)
    for k in ("mfma_busy", "valu_busy", "mfma_valu_coexec"):
        assert 0.0 < sb[k] < 1.0
    assert sb["mfma_valu_coexec"] <= min(sb["mfma_busy"], sb["valu_busy"])


def test_traffic_is_at_least_the_algorithmic_bytes(bench):
    t = float(bench._profile_fields(bench.TRAFFIC_FILE, check_source=False)["hbm_bytes_per_launch"])
    assert 2.7e9 < t < 6e9
