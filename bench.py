#!/usr/bin/env python3
"""Benchmark of the proxy-query Token Eviction hot path (score -> select -> compact) on one GPU.

Default workload: one 33 000-token agent trajectory across 36 layers x 8 KV heads (32 query
heads, 1024 delayed future-turn proxy queries per query head, d = 128, bf16, keep ratio 0.2,
so m = 6600 per KV head), per-query LSE supplied as float32, contiguous compaction of every
layer in one launch per stage. A step is one pass of kvc_score + kvc_select_topm +
kvc_compact_contig over the whole trajectory; inputs are resident in HBM before timing starts.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import gc
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# vector float32 peak without packed-FP32 instructions (the library is built with them turned
# off): 256 CUs x 4 SIMDs x 16 lanes x 2 flop (one FMA) x 2.4 GHz = 78.6 TFLOP/s; the published
# 157.3 TFLOP/s counts the packed (two-wide) FMA
F32_VALU_PEAK_TFLOPS = 78.6
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_mfma_c3_traffic.txt")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "score_mfma_c3_counters.txt")
# the score kernel's source: its own file and the headers it includes
SCORE_SRCS = [os.path.join(ROOT, "online_compaction_amd", "csrc", f)
              for f in ("score_mfma.hip", "mfma_common.h", "kvc_internal.h")]


def score_source_sha256() -> str:
    h = hashlib.sha256()
    for f in SCORE_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def describe(w) -> str:
    lay = "paged B=%d" % w.block_size if w.paged else "contiguous"
    lse = "supplied LSE" if w.lse_supplied else "computed LSE"
    n = f"n={w.n[0]}" if len(set(w.n)) == 1 else f"n={min(w.n)}..{max(w.n)}"
    if w.seg_len:
        n += f", segment [{w.seg_start}, {w.seg_start + w.seg_len})"
    pol = (", scored by attention mass, kept by LRFU state (ActKV: 90 % action-critical, lambda 0.5)"
           if w.name == "actkv" else
           ", read through a slot map; evicted positions redirected to a dead slot (no data moved)"
           if w.name == "sentinel" else
           ", then beta and V_C fitted for the kept keys by Attention Matching" if w.name == "am" else "")
    causal = ", causal action rows (each sees the keys up to its own position)" if w.causal else ""
    return (f"{w.name}: {w.S} seqs x {w.H} KV heads, G={w.G}, q={w.q}, R={w.R}, {n}, d={w.d}, {w.dtype}, "
            f"{lse}, m={w.m[0] if len(set(w.m)) == 1 else 'round(n/5)'}, {lay}{pol}{causal}")


def trajectory_tokens(w) -> int:
    """Token positions compacted per step: the 36 sequences of the default workload are layers of
    one trajectory, so it counts 33 000 (the segment workload counts its turn once); elsewhere
    sequences are distinct."""
    if w.seg_len:
        return w.seg_len
    if w.name == "c3":
        return w.n[0]
    return int(sum(w.n))


def scored_lens(w):
    return [w.seg_len] * w.S if w.seg_len else list(w.n)


def algorithmic_bytes(w, moved_rows=None) -> dict:
    """Bytes the method must move per step (reads + writes), per stage: every key row and proxy row
    once, the scores written, and a supplied LSE. (How often an implementation reads the keys is
    not counted: the MFMA path reads them once for the LSE and once for the scores, the few-row
    paths once plus R logits per key.)"""
    el = 2 if w.dtype == "bf16" else 4
    row = w.d * el
    entries = sum(scored_lens(w)) * w.H
    kept = sum(w.m) * w.H
    rows_q = w.S * w.H * w.R
    score = entries * row + rows_q * row + entries * 4 + (rows_q * 4 if w.lse_supplied else 0)
    select = entries * 4 + kept * 4
    if w.name == "sentinel":  # slot map read by both passes; redirect writes the evicted entries
        score += entries * 4 * 2
        return dict(score=score, select=select, compact=kept * 4 + (entries - kept) * 4,
                    total=score + select + kept * 4 + (entries - kept) * 4)
    if w.name == "actkv":
        select += entries * 12  # LRFU step: mass read, state read and written
        kept_side = kept * 8    # the state carried through compaction (read + write)
    else:
        kept_side = 0
    if w.paged:
        moved = kept if moved_rows is None else moved_rows
        compact = kept * 4 + moved * 2 * row * 2 + kept_side
    else:
        compact = kept * 4 + kept * 2 * row * 2 + kept_side
    out = dict(score=score, select=select, compact=compact, total=score + select + compact)
    if w.name == "am":  # the fit reads Q, every key and value, the kept indices; writes beta and V_C
        out["am_fit"] = rows_q * row + entries * 2 * row + kept * 4 + kept * 4 * (1 + w.d)
        out["total"] += out["am_fit"]
    return out


def score_flops(w) -> float:
    """QK^T multiply-adds the scores need: every logit (R x n per unit), or with causal rows only
    the logits a row sees (min(position + 1, n) keys per row)."""
    passes = 1 if w.lse_supplied else 2
    if w.causal:
        rp = W.row_positions(w, "action").astype(np.int64)
        seen = sum(int(np.clip(rp[s] + 1, 0, scored_lens(w)[s]).sum()) for s in range(w.S))
        return float(passes) * 2.0 * w.d * seen
    return float(passes) * 2.0 * w.R * w.d * sum(scored_lens(w)) * w.H


def am_work(w, iters_beta: int, iters_v: int) -> dict:
    """The work one Attention Matching fit does, by the units that do it, and the time it takes
    at their peaks (the bound the fit is priced against):
      bf16     MFMA FLOP on stored bf16 rows: every pass that re-forms E_ij = exp(c q_i.k_Cj - ME)
               (the kept-logit maximum, E^T z, two per bias update, two for P_C) and the target's
               logits over all n keys (twice when the fit computes the LSE itself);
      split2   the target Y = P V, as two bf16 products (P split into halves, V exact);
      split3   the value products on split float32 operands, three bf16 products each:
               Z_0 = P_C V_0, the last P_C^T product, the symmetric Gram matrix of the smaller side
               (N (N + 1) L FLOP) and one N x N x d product per further step;
      exp      the exponentials of every re-formed E entry and of the target's weights, at the
               transcendental rate (a quarter of the FMA rate);
      valu     the float32 FMAs beside them (logit scaling and the row / column sums);
      step_hbm the Gram matrix read once per step (float32 split, 4 bytes per entry), which bounds
               those products instead of their MFMA work."""
    bf16 = split2 = split3 = exps = valu = step_s_mfma = step_bytes = 0.0
    for s in range(w.S):
        n, m, R, d = w.n[s], w.m[s], w.R, w.d
        passes = 2 * iters_beta + 5
        bf16 += 2.0 * R * d * (passes * m + n * (1 if w.lse_supplied else 2))
        exps += (passes - 1) * R * m + R * n
        valu += 4.0 * passes * R * m
        split2 += 2.0 * R * n * d
        if iters_v > 0:
            rows_side = -(-R // 64) * 64 <= -(-m // 64) * 64
            N, L = (R, m) if rows_side else (m, R)
            split3 += 2 * 2.0 * R * m * d
            if iters_v > 1:
                split3 += N * (N + 1) * L
                step = 2.0 * N * N * d * (iters_v - 1)
                split3 += step
                step_s_mfma += 3.0 * step / (MFMA_BF16_PEAK_TFLOPS * 1e12)
                step_bytes += 4.0 * N * N * (iters_v - 1)
    H = w.H
    out = {"bf16": bf16 * H, "split2": split2 * H, "split3": split3 * H, "exp": exps * H, "valu": valu * H}
    step_s_mfma *= H
    step_s_hbm = step_bytes * H / (HBM_PEAK_GBPS * 1e9)
    out["bound_s"] = ((out["bf16"] + 2.0 * out["split2"] + 3.0 * out["split3"]) / (MFMA_BF16_PEAK_TFLOPS * 1e12)
                      - step_s_mfma + max(step_s_mfma, step_s_hbm)
                      + out["exp"] / (F32_VALU_PEAK_TFLOPS * 1e12 / 8.0)
                      + out["valu"] / (F32_VALU_PEAK_TFLOPS * 1e12))
    return out


# ---------------------------------------------------------------------------------- CPU baseline

def _oracle_unit(args):
    w, s, h, bias_row, am_iters = args
    from oracle import oracle as O
    from workloads import unit_keys, unit_queries, unit_values
    K = unit_keys(w, s, h)
    V = unit_values(w, s, h)
    if w.seg_len:  # only the turn is scored and compacted
        K, V = K[w.seg_start:w.seg_start + w.seg_len], V[w.seg_start:w.seg_start + w.seg_len]
    Qr = unit_queries(w, s, h)
    lse_rows = None
    if w.lse_supplied:  # the supplied input, prepared outside the timed region
        lse_rows = O.lse_unit(Qr, K, w.dtype, w.logit_scale, bias_row).astype(np.float32).astype(np.float64)
    pos = None
    if w.causal:
        from workloads import row_positions
        pos = row_positions(w, "action")[s, h * w.G:(h + 1) * w.G].reshape(-1)
    t0 = time.perf_counter()
    if w.name == "actkv" and w.causal:
        mass, _ = O.causal_unit(Qr, K, pos, w.dtype, w.logit_scale, bias_row, lse_rows, power=1)
        hit = O.action_critical(mass.astype(np.float32), 0.9)
        st0 = np.random.default_rng([4096, s, h]).random(K.shape[0]) * 3.41
        kept = O.select_topm(O.lrfu_step(st0, hit, 2.0 ** -0.5), w.m[s])
    elif w.name == "actkv":  # attention mass -> action-critical set -> LRFU step -> top-m of the state
        mass = O.mass_unit(Qr, K, w.dtype, w.logit_scale, bias_row, lse_rows)
        hit = O.action_critical(mass.astype(np.float32), 0.9)
        st0 = np.random.default_rng([4096, s, h]).random(K.shape[0]) * 3.41
        kept = O.select_topm(O.lrfu_step(st0, hit, 2.0 ** -0.5), w.m[s])
    elif w.causal:
        sc, _ = O.causal_unit(Qr, K, pos, w.dtype, w.logit_scale, bias_row, lse_rows)
        kept = O.select_topm(sc, w.m[s])
    else:
        sc = O.score_unit(Qr, K, w.dtype, w.logit_scale, bias_row, lse_rows)
        kept = O.select_topm(sc, w.m[s])
    if w.name == "am":  # Attention Matching fit of the kept keys (K_C is their gather)
        O.am_unit(Qr, K, V, kept, w.dtype, w.logit_scale, am_iters[0], am_iters[1], lse_rows)
    if w.name == "sentinel":  # layout-preserving: redirect the evicted positions, move nothing
        O.evict_redirect(np.arange(K.shape[0]), kept, K.shape[0], K.shape[0])
    else:
        O.gather(K, kept)
        O.gather(V, kept)
    return time.perf_counter() - t0


def _oracle_steps(w, am_iters) -> str:
    lse = ("supplied LSE" if w.lse_supplied else "computed LSE") + (", causal rows" if w.causal else "")
    if w.name == "actkv":
        return f"attention mass ({lse}) + action-critical set + LRFU step + top-m + gather"
    if w.name == "sentinel":
        return f"score ({lse}) + top-m + dead-slot redirect"
    if w.name == "am":
        return (f"score ({lse}) + top-m + gather + Attention Matching ({am_iters[0]} bias updates, "
                f"{am_iters[1]} value steps)")
    return f"score ({lse}) + top-m + gather"


SINGLE_CORE_WORKLOADS = ("c1", "c2a", "c2b", "c4")


def single_core_baseline() -> dict:
    """The oracle on ONE core (one BLAS thread, this process) for the small named workloads: one
    unit of each timed and scaled by the workload's unit count (its units cost the same), c4 at
    its largest budget."""
    from threadpoolctl import threadpool_limits
    out = {}
    for name in SINGLE_CORE_WORKLOADS:
        w = W.spec(name, 6) if name == "c4" else W.spec(name)
        with threadpool_limits(1):
            t = _oracle_unit((w, 0, 0, W.bias_row(w, 0), (0, 0)))
        units = w.S * w.H
        out[name] = {"tokens_per_s": trajectory_tokens(w) / (t * units), "step_s": t * units,
                     "sample": f"1 of {units} units timed ({t:.3f} s), scaled by {units}"}
    return out


def cpu_baseline(w, budget_s: float, am_iters=(0, 0), single_core: bool = False) -> dict:
    from concurrent.futures import ProcessPoolExecutor
    import multiprocessing as mp
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = W.gen.default_workers()
    units = [(s, h) for s in range(w.S) for h in range(w.H)]
    # a first unit calibrates how many fit the budget
    ctx = mp.get_context("fork")
    if threadpool_limits:
        threadpool_limits(1)
    t_first = _oracle_unit((w, 0, 0, W.bias_row(w, 0), am_iters))
    per_wave = max(1, int(budget_s / max(t_first, 1e-3)))
    rng = np.random.default_rng(0)
    if len(units) > 1:
        count = max(1, min(len(units) - 1, per_wave * cores))
        pick = [units[i] for i in sorted(rng.choice(np.arange(1, len(units)), size=count, replace=False))]
    else:  # a single unit: time repeats of it
        count = max(1, min(per_wave * cores, 64))
        pick = units * count
    log(f"[cpu] oracle: first unit {t_first:.2f} s; timing {count} more units on {cores} processes")
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=cores, mp_context=ctx) as ex:
        busy = list(ex.map(_oracle_unit, [(w, s, h, W.bias_row(w, s), am_iters) for s, h in pick]))
    wall = time.perf_counter() - t0
    # units of one workload cost about the same, so a step takes units / count times the sample
    step_s = wall * len(units) / count
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    out = {"value": trajectory_tokens(w) / step_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": (f"{count} of {len(units)} (sequence or layer, KV head) units, float64 NumPy oracle "
                      f"{_oracle_steps(w, am_iters)}, one unit per process with 1 BLAS thread; "
                      f"wall {wall:.1f} s (busy {sum(busy):.1f} s) scaled by {len(units)}/{count}"),
           "cpu_model": model}
    if single_core:  # the same oracle on one core, for the small named workloads
        out["single_core"] = single_core_baseline()
    return out


# ---------------------------------------------------------------------------------- roofline

def _profile_fields(path: str, check_source: bool = True):
    """The key = value lines of a committed PMC summary, or None if it is missing or (unless
    check_source is False) the score kernel's source changed since its counters were taken."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if check_source and kv.get("source_sha256") != score_source_sha256():
        return None
    return kv


def traffic_from_profile():
    """HBM bytes per launch of the score kernel from the committed PMC summary, or None."""
    kv = _profile_fields(TRAFFIC_FILE)
    try:
        return float(kv["hbm_bytes_per_launch"]) if kv else None
    except (KeyError, ValueError):
        return None


def serialized_bound_from_profile(launch_ms: float, check_source: bool = True):
    """The score kernel's serialized MFMA + VALU bound from its committed pipe counters: the
    QK^T FLOP at the bf16 spec rate plus every VALU instruction it issues at 4 cycles per wave
    at 2.4 GHz, none of it overlapped, beside the busy fractions the counters read. `frac` is
    that bound over the measured launch (1.0 = the kernel runs no slower than its two pipes
    back to back). None if the summary is missing or stale."""
    kv = _profile_fields(COUNTERS_FILE, check_source)
    if not kv:
        return None
    try:
        b = float(kv["serialized_bound_ms"])
        return {"ms": b, "mfma_ms": float(kv["mfma_only_ms"]), "valu_ms": float(kv["valu_only_ms"]),
                "frac": b / launch_ms, "mfma_busy": float(kv["mfma_busy"]),
                "valu_busy": float(kv["valu_busy"]), "mfma_valu_coexec": float(kv["coexec"])}
    except (KeyError, ValueError):
        return None


def measured_ceilings() -> dict:
    """What the machine reaches outside this library, for context beside the spec peaks: a plain
    1 GiB device-to-device copy (torch; read + write bytes per second) and a square bf16 matrix
    product of 8192 (torch.mm on contiguous operands, float32 accumulation). Timed after the
    benchmark's own timed region, a few repetitions each."""
    import torch
    out = {}
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["copy_gbps"] = 2.0 * (1 << 30) * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16).contiguous()
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16).contiguous()
    c = torch.mm(a, b)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        c = torch.mm(a, b)
    e1.record()
    torch.cuda.synchronize()
    out["bf16_matmul_tflops"] = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3", help="c3 (default) or another named workload, for study")
    ap.add_argument("--k", type=int, default=6, help="budget index for the paged action-token workload")
    ap.add_argument("--causal", action="store_true",
                    help="action-token workloads (c4, actkv, sentinel): each proxy row sees only the keys "
                         "up to its own position")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="approximate CPU baseline budget")
    ap.add_argument("--am-iters", type=int, nargs=2, default=(32, 32), metavar=("BETA", "V"),
                    help="Attention Matching: multiplicative bias updates and Landweber value steps")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the copy / matmul ceiling measurement after the timed region")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this size (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (units never interact, so "
              f"more GPUs would each run this same benchmark on their own share)", file=sys.stderr)
        sys.exit(2)

    w = W.spec(args.workload, args.k) if args.workload == "c4" else W.spec(args.workload)
    if args.causal:
        if w.queries != "action":
            print(f"--causal needs an action-token workload (c4, actkv, sentinel), not {w.name}", file=sys.stderr)
            sys.exit(2)
        w = dataclasses.replace(w, causal=True)
    log(f"[bench] workload {describe(w)}")
    t0 = time.perf_counter()
    workers = W.gen.default_workers()
    data = W.build_paged(w, workers) if w.paged else W.build_contiguous(w, workers)
    log(f"[bench] inputs generated in {time.perf_counter() - t0:.1f} s")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, args.cpu_seconds, args.am_iters, single_core=(w.name == "c3"))
        log(f"[cpu] oracle baseline {cpu['value']:.4g} tokens/s on {cpu['cores']} cores")
        if "single_core" in cpu:
            log("[cpu] one core: " + ", ".join(f"{k} {v['tokens_per_s']:.4g} tokens/s"
                                              for k, v in cpu["single_core"].items()))
        # let the worker processes' exit (and the release of their memory) finish before the
        # GPU is timed: right after a many-core CPU leg some host calls were seen to stall
        gc.collect()
        time.sleep(2.0)

    import torch
    from online_compaction_amd import _abi as A
    from online_compaction_amd import path as P
    A.load()  # fails loudly when libkvc.so is missing

    if w.paged and w.seg_len:
        b = P.paged_batch(data["Q"], data["k_pool"], data["v_pool"], data["table"], [w.seg_len] * w.S, data["m"],
                          w.G, w.logit_scale, w.block_size, n_max=w.seg_len, starts=[w.seg_start] * w.S,
                          cache_lens=data["n"])
        pristine = (b.k_pool.clone(), b.v_pool.clone(), b.table.clone())
    elif w.paged:
        b = P.paged_batch(data["Q"], data["k_pool"], data["v_pool"], data["table"], data["n"], data["m"], w.G,
                          w.logit_scale, w.block_size, n_max=w.n_max, bias=data["bias"])
        pristine = (b.k_pool.clone(), b.v_pool.clone(), b.table.clone())
    else:
        b = P.contiguous_batch(data["Q"], data["K"], data["V"], data["n"], data["m"], w.G, w.logit_scale,
                               bias=data["bias"])
        pristine = None
    del data
    if w.causal:
        b.shape.row_pos = P.device_tensor(W.row_positions(w, "action"))
    if w.lse_supplied:  # the harness computes the supplied LSE with the library's own LSE pass
        lse = torch.empty((w.S, w.H * w.G, w.q), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(256, A.kvc_lse_workspace_size(b.shape, b.kview())), dtype=torch.uint8, device="cuda")
        A.kvc_lse(b.shape, b.q, b.kview(), b.bias, lse, ws)
        b.lse = lse
        del ws
    o = P.allocate(b)
    retention = None
    if w.name == "sentinel":  # slot pool = the paged pool + one sentinel block; slot map from the table
        nb = b.k_pool.shape[0]
        sent = torch.full((1,) + tuple(b.k_pool.shape[1:]), -1.0e4, dtype=b.k_pool.dtype, device="cuda")
        spool = torch.cat([b.k_pool, sent]).reshape(-1, w.H, w.d)
        dead = nb * w.block_size
        pos = torch.arange(w.n_max, device="cuda")
        base = (b.table[0, (pos // w.block_size).clamp(max=b.max_blocks - 1)].long() * w.block_size
                + pos % w.block_size).to(torch.int32)
        smap = base.expand(w.S, w.H, w.n_max).contiguous()
        pristine = (smap.clone(),)
        sview = A.KView(spool, b.dtype, 0, None, 0, smap, dead)

        def sentinel_score():
            A.kvc_score(b.shape, b.q, sview, None, b.bias, o.scores, o.ws)

        def sentinel_redirect():
            A.kvc_evict_redirect(b.shape, o.kept, b.m, b.m_max, smap, dead)
        stages = (sentinel_score, lambda: P.run_select(b, o), sentinel_redirect)
    if w.name == "actkv":  # a warm LRFU state: seeded values in [0, 1 / (1 - 2^-0.5))
        st0 = np.random.default_rng(4096).random((w.S, w.H, w.n_max)).astype(np.float32) * 3.41
        retention = P.allocate_retention(b, st0)
        pristine = pristine + (retention.state.clone(),)
        stages = (lambda: P.run_retention_score(b, o, retention), lambda: P.run_retention_select(b, o, retention),
                  lambda: P.run_retention_compact(b, o, retention))
    elif w.name != "sentinel":
        stages = (lambda: P.run_score(b, o), lambda: P.run_select(b, o), lambda: P.run_compact(b, o))
    names = ("score", "select", "redirect" if w.name == "sentinel" else "compact")
    matching = None
    if w.name == "am":  # the fit reads the pool before a paged compaction would rewrite it
        matching = P.allocate_matching(b, *args.am_iters)
        stages = stages[:2] + (lambda: P.run_matching(b, o, matching),) + stages[2:]
        names = ("score", "select", "am_fit", "compact")
    ns = len(stages)
    torch.cuda.synchronize()
    log("[bench] inputs resident on the GPU")

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")

    def restore():
        if w.name == "sentinel":
            smap.copy_(pristine[0])
        elif pristine is not None:
            b.k_pool.copy_(pristine[0])
            b.v_pool.copy_(pristine[1])
            b.table.copy_(pristine[2])
            if retention is not None:
                retention.state.copy_(pristine[3])

    for _ in range(args.warmup):
        restore()
        for run_stage in stages:
            run_stage()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)] for _ in range(args.steps)]
    stage_ms = np.zeros((args.steps, ns))
    host_ms = np.zeros((args.steps, ns))  # time the host spends enqueueing each stage

    def timed_step(i):
        e = ev[i]
        e[0].record()
        for k in range(ns):
            h0 = time.perf_counter()
            stages[k]()
            host_ms[i, k] = (time.perf_counter() - h0) * 1e3
            e[k + 1].record()

    wall = 0.0
    if pristine is None:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            timed_step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:  # paged: restore the pristine pool before each step, outside the timed region
        for i in range(args.steps):
            restore()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            timed_step(i)
            torch.cuda.synchronize()
            wall += time.perf_counter() - t0
    for i in range(args.steps):
        e = ev[i]
        stage_ms[i] = [e[k].elapsed_time(e[k + 1]) for k in range(ns)]
    ms_step = wall * 1e3 / args.steps
    avg = stage_ms.mean(axis=0)
    havg = host_ms.mean(axis=0)
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step ("
        + ", ".join(f"{nm} {t:.3f}" for nm, t in zip(names, avg)) + " ms; host enqueue "
        + " / ".join(f"{t:.3f}" for t in havg) + " ms)")
    st = dict(zip(names, avg))

    moved = None
    if w.paged and w.name != "sentinel":
        kept = P.host_array(o.kept)
        moved = 0
        for s in range(w.S):
            n, m = (w.seg_len or w.n[s]), w.m[s]
            start = (-(-n // w.block_size) - -(-m // w.block_size)) * w.block_size
            for h in range(w.H):
                k = kept[s, h, :m]
                moved += int(np.count_nonzero((k < start) | (k >= start + m)))
    ab = algorithmic_bytes(w, moved)
    tokens = trajectory_tokens(w)
    flops = score_flops(w)
    score_s = avg[0] * 1e-3
    achieved_tf = flops / score_s / 1e12
    step_s = ms_step * 1e-3
    traffic = traffic_from_profile() if (w.name == "c3") else None
    roof = {
        "kernel": "score_mfma (kvc_attention_mass)" if w.name == "actkv" else "score_mfma (kvc_score)",
        "bound": "mfma",
        "achieved": achieved_tf,
        "peak": MFMA_BF16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": achieved_tf / MFMA_BF16_PEAK_TFLOPS,
        "traffic": traffic,
        "flops_per_launch": flops,
        "launch_ms": avg[0],
    }
    if w.name == "c3":
        roof["serialized_bound"] = serialized_bound_from_profile(avg[0])
    few_kernels = ("valu_lse_pass + valu_score_cached" if w.R <= 32 else "valu_lse_pass + valu_score_keys")
    if w.lse_supplied:
        few_kernels = "valu_score_keys"
    if w.dtype == "f32":  # float32 scoring runs on the vector ALU
        roof.update({"kernel": few_kernels + " (score stage)", "bound": "alu",
                     "achieved": achieved_tf, "peak": F32_VALU_PEAK_TFLOPS,
                     "frac": achieved_tf / F32_VALU_PEAK_TFLOPS})
    elif w.R < 16:  # bf16 with few proxy rows: one pass over K (few-row MFMA kernels), bound by reading it
        gbps = ab["score"] / score_s / 1e9
        small = "small_score_keys" if w.lse_supplied else "small_lse_pass + valu_score_cached"
        roof.update({"kernel": small + " (score stage)", "bound": "hbm", "achieved": gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                     "bytes_per_launch": ab["score"]})
    if w.name == "am":  # the fit dominates: its kernels against the peak of the units they use
        af = am_work(w, *args.am_iters)
        fit_s = st["am_fit"] * 1e-3
        tot = af["bf16"] + af["split2"] + af["split3"] + af["valu"]
        roof = {"kernel": "kvc_am_fit (all of its kernels)", "bound": "mfma", "achieved": tot / fit_s / 1e12,
                "peak": tot / af["bound_s"] / 1e12, "unit": "TFLOP/s", "frac": af["bound_s"] / fit_s,
                "traffic": None, "work_per_launch": af, "launch_ms": st["am_fit"],
                "iters": {"beta": args.am_iters[0], "v": args.am_iters[1]}}
    line = {
        "metric": "compacted KV tokens/sec (score+select+compact) and % of peak HBM GB/s, 1 GPU",
        "value": tokens / step_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded generators shaped like the pages' agent trajectories)",
        "config": {
            "workload": describe(w),
            "tokens_per_step": tokens,
            "kv_entries_per_step": int(sum(scored_lens(w)) * w.H),
            "entries_per_s": sum(scored_lens(w)) * w.H / step_s,
            "stage_ms": st,
            "hbm_algorithmic_bytes_per_step": ab["total"],
            "hbm_algorithmic_gbps": ab["total"] / step_s / 1e9,
            "hbm_frac_of_peak": ab["total"] / step_s / 1e9 / HBM_PEAK_GBPS,
            "select_compact_hbm_gbps": (ab["select"] + ab["compact"]) / ((st["select"] + st[names[-1]]) * 1e-3) / 1e9,
            "mfma_util": achieved_tf / MFMA_BF16_PEAK_TFLOPS,
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if not args.no_ceilings:
        line["ceilings"] = measured_ceilings()
        log(f"[bench] measured ceilings: device copy {line['ceilings']['copy_gbps']:.0f} GB/s, "
            f"bf16 matmul {line['ceilings']['bf16_matmul_tflops']:.0f} TFLOP/s "
            f"(spec {HBM_PEAK_GBPS:.0f} GB/s, {MFMA_BF16_PEAK_TFLOPS:.0f} TFLOP/s)")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
