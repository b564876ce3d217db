#!/usr/bin/env python3
"""LISA layer benchmark on one MI355X.

Prints ONE JSON line.  The headline is the prefill of one Qwen2.5-7B-shaped
LISA layer at 16K context (B=1, n=16384, 28 query / 4 KV heads, d=128,
indexer 4 x 64, M=256, C=64): `value` = tokens/s = n / call time.  The
decode step at 16K context (Qwen2.5-1.5B shapes, B=16, 16384 cached + 1 new
token, M=256) is measured in the same run and reported under "decode".

Inputs are seeded synthetic tensors (the generator in
hybrid_linear_top_amd/inputs.py), resident in HBM before timing starts, and
rotated over several copies so the 256 MB Infinity Cache cannot serve
repeated reads.  Per-kernel durations come from HIP events the library
records around each launch on the caller's stream (lisa_stage_timing), in a
separate pass so the headline timing carries no event overhead.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--decode-steps K2]
                  [--no-cpu-baseline] [--copy-calibration]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LISA layer tokens/s at 16K ctx (decode + prefill); % of HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector (256 CUs, 2.4 GHz), TFLOP/s
PROFILES = os.path.join(ROOT, "profiles")


# ---------------------------------------------------------------------------
# algorithmic work (counts of the method itself, not of any implementation)
def tri(n):
    return n * (n + 1) // 2


def pairs(n, M):
    """sum_{t<n} min(M, t+1): selected (query, key) pairs per group."""
    if n <= M:
        return tri(n)
    return tri(M) + (n - M) * M


def prefill_flops(cfg, n, B=1):
    G, Hq, d, C = cfg.Hkv, cfg.Hq, cfg.d, cfg.chunk
    f = {
        "indexer_topm": 2 * G * cfg.HI * cfg.dI * tri(n),
        "sparse_gate_prefill": 4 * Hq * d * pairs(n, cfg.M),
        "linear_chunk_state": G * 2 * n * d * d,
        "linear_prefix_scan": 0,
        "linear_chunk_output": Hq * (4 * n * C * d + 2 * n * d * d),
    }
    return {k: v * B for k, v in f.items()}


def decode_bytes(cfg, lengths):
    import numpy as np
    L = np.asarray(lengths, dtype=np.int64)
    B, G, Hq, d = len(L), cfg.Hkv, cfg.Hq, cfg.d
    kI = int(L.sum()) * G * cfg.dI * 2
    kv_rows = int(np.minimum(L, cfg.M).sum()) * G * 2 * d * 2
    state = B * Hq * d * d * 4 * 2
    small = B * (2 * Hq * d * 2 + G * cfg.HI * cfg.dI * 2 + G * cfg.HI * 2 + Hq * 2 + 2 * G * d * 2)
    # the score launch streams k_I; the state step (state read and write, the
    # new token's q, k, v) runs in the select launch, beside the selects
    return {
        "decode_score_state": kI + B * (G * cfg.HI * cfg.dI * 2 + G * cfg.HI * 2),
        "decode_select": state + B * (Hq * d * 2 + 2 * G * d * 2),
        "sparse_gate_decode": kv_rows + B * (2 * Hq * d * 2 + Hq * 2),
        "total": kI + kv_rows + state + small,
        "kI": kI, "kv_rows": kv_rows, "state": state, "small": small,
    }


# stage name (as lisa_stage_timing reports it) -> (rocprofv3 kernel-name
# pattern, the sources that kernel is built from)
STAGE_KERNELS = {
    "indexer_topm": (r"indexer_topm_kernel<", ["indexer.hip", "common.hpp", "kernels.hpp"]),
    "indexer_pack": (r"pack_keys_kernel<", ["indexer.hip", "common.hpp", "kernels.hpp"]),
    "sparse_gate_prefill": (r"sparse_prefill_wave_kernel<|sparse_gate_kernel<[^>]*, false,",
                            ["sparse.hip", "common.hpp", "kernels.hpp"]),
    "sparse_gate_decode": (r"sparse_gate_kernel<[^>]*, true,", ["sparse.hip", "common.hpp", "kernels.hpp"]),
    "linear_chunk_state": (r"chunk_state_kernel<", ["linear.hip", "common.hpp", "kernels.hpp"]),
    "linear_prefix_scan": (r"prefix_scan_kernel<", ["linear.hip", "common.hpp", "kernels.hpp"]),
    "linear_chunk_output": (r"chunk_output_kernel<", ["linear.hip", "common.hpp", "kernels.hpp"]),
    "decode_score_state": (r"decode_score_state_kernel<", ["decode.hip", "common.hpp", "kernels.hpp"]),
    "decode_select": (r"decode_topm_kernel<|decode_merge_kernel<", ["decode.hip", "common.hpp", "kernels.hpp"]),
    "bwd_sparse": (r"sparse_bwd_kernel<", ["backward.hip", "common.hpp", "kernels.hpp"]),
    "bwd_sparse_query": (r"sparse_bwd_q_kernel<", ["backward.hip", "common.hpp", "kernels.hpp"]),
    "bwd_sparse_keys": (r"sparse_bwd_walk_kernel<", ["backward.hip", "common.hpp", "kernels.hpp"]),
}


def source_hash(*names):
    h = hashlib.sha256()
    for nm in names:
        with open(os.path.join(ROOT, "hybrid_linear_top_amd", "csrc", nm), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# The benchmark's phases, in the order it runs them.  With --phase-markers a
# tiny calibration copy (probe_copy_kernel on 4 KiB) is launched before each
# phase, so that a rocprofv3 database can be split by phase: the 16K and the
# ragged decode batches launch the same kernels, and the backward launches
# the forward's linear kernels on its own operands.
PHASES = ["prefill_7b_16k", "prefill_1p5b_4k", "decode_1p5b_16k", "decode_7b_ragged", "backward_setup",
          "backward_7b_16k"]
MARKER_KERNEL = "probe_copy_kernel"


def traffic_from_profiles(stage, phase):
    """HBM bytes per launch of a stage in a phase, from the committed rocprofv3
    counter summary; None when absent or when the kernel's sources changed
    since the counters were taken."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get("phases", {}).get(phase, {}).get(stage)
    if not ent or ent.get("source_hash") != source_hash(*STAGE_KERNELS[stage][1]):
        return None
    return ent.get("hbm_bytes_per_launch")


def _db_rows(db, counters=None):
    """(phase, stage, counter, value) per dispatch of a rocprofv3 --pmc
    database written by a run with --phase-markers."""
    import re
    import sqlite3
    cur = sqlite3.connect(db).cursor()
    rows = list(cur.execute("select kernel_name, counter_name, value, dispatch_id from counters_collection"))
    marks = sorted({i for nm, _, _, i in rows if MARKER_KERNEL in nm})
    import bisect
    out = []
    for nm, cn, v, i in rows:
        if counters and cn not in counters:
            continue
        if MARKER_KERNEL in nm or "copyBuffer" in nm:
            out.append(("calibration", nm, cn, v, i))
            continue
        ph = bisect.bisect_left(marks, i) - 1
        phase = PHASES[ph] if 0 <= ph < len(PHASES) else "unmarked"
        for stage, (pat, _) in STAGE_KERNELS.items():
            if re.search(pat, nm):
                out.append((phase, stage, cn, v, i))
                break
    return out


def traffic_summary(fetch_db, write_db, out_json, out_md, command):
    """Turn two rocprofv3 --pmc databases (FETCH_SIZE and WRITE_SIZE, KiB per
    dispatch) into HBM bytes per launch, per phase and stage.  Each counter is
    scaled by what it reads for the 1 GiB device copy that --copy-calibration
    runs first (the copy reads and writes 2^30 bytes)."""

    def per_stage(db, counter):
        rows = _db_rows(db, {counter})
        cal = [v for ph, nm, _, v, _ in rows if ph == "calibration" and "copyBuffer" in nm and v > 1e5]
        if not cal:
            raise SystemExit(f"{db}: no calibration copy found (run bench.py --copy-calibration)")
        factor = (1 << 30) / (sum(cal) / len(cal) * 1024.0)
        acc = {}
        for ph, stage, _, v, _ in rows:
            if ph in ("calibration", "unmarked", "backward_setup"):
                continue
            acc.setdefault((ph, stage), []).append(v)
        return {k: (sum(v) / len(v) * 1024.0 * factor, len(v)) for k, v in acc.items()}, factor

    fetch, ff = per_stage(fetch_db, "FETCH_SIZE")
    write, wf = per_stage(write_db, "WRITE_SIZE")
    phases = {}
    for key in fetch:
        if key not in write:
            continue
        ph, stage = key
        phases.setdefault(ph, {})[stage] = {
            "fetch_bytes": round(fetch[key][0]), "write_bytes": round(write[key][0]),
            "hbm_bytes_per_launch": round(fetch[key][0] + write[key][0]), "dispatches": fetch[key][1],
            "source_hash": source_hash(*STAGE_KERNELS[stage][1])}
    data = {"command": command, "fetch_scale": round(ff, 4), "write_scale": round(wf, 4), "phases": phases}
    with open(out_json, "w") as f:
        json.dump(data, f, indent=1)
    with open(out_md, "w") as f:
        f.write("# HBM traffic per launch: prefill (16K 7B-shaped, 4K 1.5B-shaped), decode (16K 1.5B-shaped, "
                "7B-shaped ragged), backward (16K 7B-shaped)\n\n")
        f.write("rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each in a pass of its own "
                "(REPO is the repository root, OUT any scratch folder); dispatches are split by phase with "
                "the marker copies the run launches between phases:\n\n")
        f.write("```\n" + command + "\n```\n\n")
        f.write(f"Scale factors from the 1 GiB device copy: FETCH_SIZE x {ff:.3f}, "
                f"WRITE_SIZE x {wf:.3f}.\n\n")
        f.write("| phase | stage | dispatches | fetch MB | write MB | HBM MB per launch |\n|---|---|---|---|---|---|\n")
        for ph in PHASES:
            for stage, e in phases.get(ph, {}).items():
                f.write(f"| {ph} | {stage} | {e['dispatches']} | {e['fetch_bytes'] / 1e6:.2f} | "
                        f"{e['write_bytes'] / 1e6:.2f} | {e['hbm_bytes_per_launch'] / 1e6:.2f} |\n")
    return data


# Derived rocprofv3 counters (definitions of the rocprofiler-sdk counter
# table for gfx950), two passes that each stay within one run's hardware
# counter budget: pass 1 MfmaUtil, MfmaFlopsBF16, VALUBusy, TA_BUSY_avr,
# OccupancyPercent, GRBM_GUI_ACTIVE (4 SQ, 1 GRBM, 1 TA counters); pass 2 LDSBankConflict,
# TCC_HIT_sum, TCC_MISS_sum, MemUnitStalled (1 SQ, 1 GRBM, 2 TCC, 1 TCP).
N_XCD = 8  # MI355X: 8 accelerator complex dies, 32 CUs each
COUNTER_PASSES = [["MfmaUtil", "MfmaFlopsBF16", "VALUBusy", "TA_BUSY_avr", "OccupancyPercent", "GRBM_GUI_ACTIVE"],
                  ["LDSBankConflict", "TCC_HIT_sum", "TCC_MISS_sum", "MemUnitStalled"]]
COUNTER_CMD = ("cd /tmp && export TMPDIR=/tmp && "
               "timeout -s KILL 240 rocprofv3 --pmc {counters} -d $OUT/pmc_{tag} -o run -- python3 $REPO/bench.py "
               "--steps 2 --warmup 1 --decode-steps 9 --decode-warmup 1 --bwd-steps 1 --no-cpu-baseline "
               "--no-peaks --phase-markers")


def counter_summary(dbs, out_json, out_md, durations_db=None):
    """Per (phase, stage) averages of the derived counters in COUNTER_PASSES,
    from one rocprofv3 --pmc database per pass; with a --kernel-trace
    database of a run with --phase-markers, also the MFMA rate each stage's
    issued MFMA flops (MfmaFlopsBF16) make over its mean duration."""
    acc = {}
    for db in dbs:
        for ph, stage, cn, v, _ in _db_rows(db):
            if ph in ("calibration", "unmarked", "backward_setup"):
                continue
            acc.setdefault((ph, stage), {}).setdefault(cn, []).append(v)
    durs = {}
    if durations_db:
        import bisect
        import re
        import sqlite3
        cur = sqlite3.connect(durations_db).cursor()
        kr = list(cur.execute("select name, duration, start from kernels order by start"))
        marks = [st for nm, _, st in kr if MARKER_KERNEL in nm]
        for nm, du, st in kr:
            if MARKER_KERNEL in nm:
                continue
            ph = bisect.bisect_left(marks, st) - 1
            if not 0 <= ph < len(PHASES):
                continue
            for stage, (pat, _) in STAGE_KERNELS.items():
                if re.search(pat, nm):
                    durs.setdefault((PHASES[ph], stage), []).append(du)
                    break
    out = {}
    for (ph, stage), cs in acc.items():
        ent = {cn: round(sum(v) / len(v), 4) for cn, v in cs.items()}
        ent["dispatches"] = max(len(v) for v in cs.values())
        ta, gui = ent.get("TA_BUSY_avr"), ent.get("GRBM_GUI_ACTIVE")
        if ta is not None and gui:
            # the raw GRBM_GUI_ACTIVE value is summed over the chip's 8 XCDs
            # (the derived counters take its maximum, one XCD's active cycles)
            ent["TA_busy_pct"] = round(100.0 * ta / (gui / N_XCD), 2)
        h, m = ent.get("TCC_HIT_sum"), ent.get("TCC_MISS_sum")
        if h is not None and m is not None and h + m > 0:
            ent["L2_hit_pct"] = round(100.0 * h / (h + m), 2)
        d = durs.get((ph, stage))
        if d and ent.get("MfmaFlopsBF16"):
            mean_ns = sum(d) / len(d)
            ent["mean_duration_us"] = round(mean_ns / 1e3, 2)
            ent["mfma_issued_tflops"] = round(ent["MfmaFlopsBF16"] / (mean_ns * 1e-9) / 1e12, 1)
            ent["mfma_issued_frac_peak"] = round(ent["mfma_issued_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)
        ent["source_hash"] = source_hash(*STAGE_KERNELS[stage][1])
        out.setdefault(ph, {})[stage] = ent
    cmds = [COUNTER_CMD.format(counters=" ".join(p), tag=f"pass{i + 1}") for i, p in enumerate(COUNTER_PASSES)]
    cmds.append("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace -d $OUT/trace_marked -o run -- "
                "python3 $REPO/bench.py --steps 2 --warmup 1 --decode-steps 9 --decode-warmup 1 --bwd-steps 1 "
                "--no-cpu-baseline --no-peaks --phase-markers")
    cmds.append("cd $REPO && python3 bench.py --counter-summary $OUT/trace_marked/run_results.db "
                "$OUT/pmc_pass1/run_results.db $OUT/pmc_pass2/run_results.db")
    data = {"commands": cmds, "phases": out}
    with open(out_json, "w") as f:
        json.dump(data, f, indent=1)
    cols = [("MfmaUtil", "MFMA busy %"), ("mfma_issued_frac_peak", "MFMA flops / peak"),
            ("VALUBusy", "VALU busy %"), ("TA_busy_pct", "TA busy %"),
            ("MemUnitStalled", "mem unit stalled %"), ("L2_hit_pct", "L2 hit %"),
            ("LDSBankConflict", "LDS bank conflict %"), ("OccupancyPercent", "occupancy %")]
    with open(out_md, "w") as f:
        f.write("# Hardware counters per kernel: prefill, decode and backward phases\n\n")
        f.write("Derived rocprofv3 counters (rocprofiler-sdk definitions for gfx950), averaged over each "
                "stage's dispatches within a phase; each pass is a run of its own (REPO is the repository "
                "root, OUT any scratch folder):\n\n```\n" + "\n".join(cmds) + "\n```\n\n")
        f.write("MfmaUtil = MFMA-busy cycles / (GPU-active cycles x SIMDs); MFMA flops / peak = "
                "MfmaFlopsBF16 (512 x MFMA MOPS) over the stage's mean kernel-trace duration, against "
                "2.5 PFLOP/s; VALUBusy = VALU-active cycles per CU / GPU-active cycles; TA busy % = busy "
                "cycles of the texture-address unit averaged over its instances (TA_BUSY_avr) / one XCD's "
                "GPU-active cycles (GRBM_GUI_ACTIVE, whose raw value sums the 8 XCDs, / 8); L2 hit % = "
                "TCC_HIT / (TCC_HIT + TCC_MISS).\n\n")
        f.write("| phase | stage | dispatches | " + " | ".join(c[1] for c in cols) + " |\n")
        f.write("|---|---|---|" + "---|" * len(cols) + "\n")
        for ph in PHASES:
            for stage, e in out.get(ph, {}).items():
                vals = [e.get(c[0]) for c in cols]
                f.write(f"| {ph} | {stage} | {e['dispatches']} | " +
                        " | ".join("" if v is None else f"{v:g}" for v in vals) + " |\n")
    return data


def kernel_stats_summary(db, out_md):
    """Per-kernel durations from a rocprofv3 --kernel-trace database, one row
    per (kernel, grid size): the 16K and the ragged decode batches launch the
    same kernels with different grids."""
    import sqlite3
    cur = sqlite3.connect(db).cursor()
    rows = list(cur.execute("select name, grid_x, count(*), sum(duration), avg(duration) from kernels "
                            "group by name, grid_x order by sum(duration) desc"))
    total = sum(r[3] for r in rows) or 1
    with open(out_md, "w") as f:
        f.write("# Kernel durations: 16K prefill (Qwen2.5-7B-shaped), 16K decode step (Qwen2.5-1.5B-shaped), "
                "7B-shaped ragged decode step, 16K backward (7B-shaped)\n\n")
        f.write("Command (on one MI355X; REPO is the repository root, OUT any scratch folder):\n\n```\n"
                "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d $OUT/prof_stats "
                "-o run -- python3 $REPO/bench.py\ncd $REPO && python3 bench.py --kernel-stats "
                "$OUT/prof_stats/run_results.db profiles/kernel_stats_prefill16k_decode16k.md\n```\n\n")
        f.write("rocprofv3 kernel-trace durations in microseconds, one row per kernel and launch grid "
                "(grid_x in work-items):\n\n")
        f.write("| kernel | grid_x | calls | total us | average us | % |\n|---|---|---|---|---|---|\n")
        for name, gx, n, tot, avg in rows:
            short = name.replace("lisa::(anonymous namespace)::", "").replace("void ", "")
            f.write(f"| `{short}` | {gx} | {n} | {tot / 1e3:.1f} | {avg / 1e3:.2f} | {100.0 * tot / total:.1f} |\n")


# ---------------------------------------------------------------------------
def timed_loop(fn, steps, warmup, copies):
    import torch
    for i in range(warmup):
        fn(i % copies)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        fn(i % copies)
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def stage_pass(fn, steps, copies):
    import torch
    from hybrid_linear_top_amd import lisa
    lisa.lisa_stage_timing_read(reset=True)
    lisa.lisa_stage_timing(True)
    for i in range(steps):
        fn(i % copies)
    torch.cuda.synchronize()
    lisa.lisa_stage_timing(False)
    return {k: tot / max(cnt, 1) for k, (cnt, tot) in lisa.lisa_stage_timing_read(reset=True).items()}


# peaks measured on this machine by the calibration kernels (measure_peaks)
MEASURED = {}


def roofline_entry(kernel, ms, work, bound, traffic=None):
    measured = None
    if bound == "hbm":
        achieved = work / (ms * 1e-3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
        measured = MEASURED.get("hbm_gbs")
    elif bound == "alu":
        achieved = work / (ms * 1e-3) / 1e12
        peak, unit = FP32_VECTOR_PEAK_TFLOPS, "TFLOP/s"
    else:
        achieved = work / (ms * 1e-3) / 1e12
        peak, unit = MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
        measured = MEASURED.get("mfma_bf16_tflops")
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kernel,
            "avg_launch_ms": round(ms, 5), "algorithmic_per_launch": work,
            "measured_peak": measured, "frac_measured_peak": round(achieved / measured, 4) if measured else None}


def measure_peaks(copy_bytes=1 << 30, mfma_iters=400, reps=5):
    """The achievable peaks of this part, measured with the library's
    calibration kernels: a plain streaming copy (bytes read + written per
    second) and an MFMA loop (bf16 16x16x32, 8 waves per SIMD)."""
    import torch
    from hybrid_linear_top_amd import lisa
    src = torch.ones(copy_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.empty(1 << 21, dtype=torch.float32, device="cuda")

    def best(fn):
        times, work = [], 0.0
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            work = fn()
            e1.record()
            torch.cuda.synchronize()
            if r:
                times.append(e0.elapsed_time(e1))
        return work, sorted(times)[len(times) // 2]

    w, ms = best(lambda: lisa.peak_probe(lisa.LISA_PROBE_COPY, src, dst, copy_bytes))
    copy_gbs = w / (ms * 1e-3) / 1e9
    w, ms = best(lambda: lisa.peak_probe(lisa.LISA_PROBE_READ, src, sink, copy_bytes))
    read_gbs = w / (ms * 1e-3) / 1e9
    MEASURED["hbm_copy_gbs"] = round(copy_gbs, 1)
    MEASURED["hbm_read_gbs"] = round(read_gbs, 1)
    # the better of the two is the achievable HBM rate the fractions use
    MEASURED["hbm_gbs"] = round(max(copy_gbs, read_gbs), 1)
    w, ms = best(lambda: lisa.peak_probe(lisa.LISA_PROBE_MFMA, None, sink, sink.numel() * 4, mfma_iters))
    MEASURED["mfma_bf16_tflops"] = round(w / (ms * 1e-3) / 1e12, 1)
    # random 256-byte row gathers from an 8 MiB table (the K and V rows of one
    # KV group at 16K positions) and from a 1 MiB one (L2-resident)
    for tag, tb in (("gather_8mib_gbs", 8 << 20), ("gather_1mib_gbs", 1 << 20)):
        w, ms = best(lambda: lisa.peak_probe(lisa.LISA_PROBE_GATHER, src, sink, tb, 8))
        MEASURED[tag] = round(w / (ms * 1e-3) / 1e9, 1)
    del src, dst, sink
    torch.cuda.empty_cache()
    return dict(MEASURED, method="median of 5 event-timed launches of lisa_peak_probe: a copy of 1 GiB "
                                 "(2 GiB moved), a read-only stream over 1 GiB (hbm_gbs is the "
                                 "better of the two), an MFMA loop (2048 x 256 threads, 400 x 8 bf16 "
                                 "16x16x32 MFMAs per wave), and random 256-byte row gathers (65536 waves x "
                                 "8 x 16 KB) from an 8 MiB and a 1 MiB table")


_MARK = {}


def phase_marker(i):
    """With --phase-markers: a 4 KiB calibration copy before phase i, which
    splits a profiler database by phase (PHASES)."""
    if not _MARK:
        return
    from hybrid_linear_top_amd import lisa
    lisa.peak_probe(lisa.LISA_PROBE_COPY, _MARK["src"], _MARK["dst"], 4096)


def cores_used():
    n = os.environ.get("OMP_NUM_THREADS")
    if n and n.isdigit():
        return int(n)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


# ---------------------------------------------------------------------------
def bench_prefill(args, small=False):
    """lisa_prefill on the 16K Qwen2.5-7B-shaped workload, or (small) on the
    4K Qwen2.5-1.5B-shaped one, whose inputs are rotated over enough copies
    that the Infinity Cache cannot hold them between repeats."""
    import numpy as np
    import torch
    from hybrid_linear_top_amd import inputs as gen, lisa
    cfg = gen.PREFILL_1P5B_4K if small else gen.PREFILL_7B_16K
    inp = gen.make_prefill_inputs(cfg)
    dims = lisa.dims_from_config(cfg)
    B, n = inp["B"], inp["n"]
    per_copy = sum(inp[k].nbytes for k in ("q", "k", "v", "q_idx", "k_idx", "w_idx", "gate")) + \
        inp["q"].nbytes + B * n * cfg.Hkv * cfg.M * 4
    copies = rotating_copies(per_copy)
    keys = ("q", "k", "v", "q_idx", "k_idx", "w_idx", "gate")
    sets = [{k: lisa.to_device(inp[k]) for k in keys} for _ in range(copies)]
    outs = [torch.empty_like(s["q"]) for s in sets]
    st = torch.empty((B, cfg.Hq, cfg.d, cfg.d), dtype=torch.float32, device="cuda")
    idx = [torch.empty((B, n, cfg.Hkv, cfg.M), dtype=torch.int32, device="cuda") for _ in range(copies)]
    ws = torch.empty(lisa.lisa_prefill_workspace_bytes(dims, B, n), dtype=torch.uint8, device="cuda")

    def step(c):
        s = sets[c]
        lisa.prefill(dims, s["q"], s["k"], s["v"], s["q_idx"], s["k_idx"], s["w_idx"], s["gate"],
                     out=outs[c], state_out=st, topm_out=idx[c], workspace=ws)

    steps = args.steps * 5 if small else args.steps
    ms = timed_loop(step, steps, args.warmup, copies)
    stages = stage_pass(step, max(3, min(steps, 10)), copies)
    flops = prefill_flops(cfg, n, B)
    total_flops = sum(flops.values())
    stage_rows = {}
    for k, v in stages.items():
        f = flops.get(k, 0)
        stage_rows[k] = {"ms": round(v, 5),
                         "tflops": round(f / (v * 1e-3) / 1e12, 3) if f else None,
                         "frac_mfma_peak": round(f / (v * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
                         if f else None}
    # the sparse stage moves K and V rows from L2 by random 256-byte gathers:
    # its rate against the gather probe at the same table size
    if "sparse_gate_prefill" in stage_rows:
        gbytes = B * cfg.Hkv * pairs(n, cfg.M) * 2 * cfg.d * 2
        gbs = gbytes / (stages["sparse_gate_prefill"] * 1e-3) / 1e9
        stage_rows["sparse_gate_prefill"]["gather_bytes"] = gbytes
        stage_rows["sparse_gate_prefill"]["gather_gbs"] = round(gbs, 1)
        if MEASURED.get("gather_8mib_gbs"):
            stage_rows["sparse_gate_prefill"]["frac_measured_gather"] = round(gbs / MEASURED["gather_8mib_gbs"], 4)
    dom = max(stages, key=stages.get)
    phase = "prefill_1p5b_4k" if small else "prefill_7b_16k"
    roof = roofline_entry(dom, stages[dom], flops.get(dom, 0), "mfma", traffic_from_profiles(dom, phase))
    if dom == "sparse_gate_prefill":
        # its MFMA work is light: what bounds it is the random-row gather
        # rate from L2 / Infinity Cache, measured by the gather probe
        sg = stage_rows[dom]
        roof.update({"limiter": "random 256-byte K/V row gathers from L2 and the Infinity Cache",
                     "gather_bytes_per_launch": sg.get("gather_bytes"), "gather_gbs": sg.get("gather_gbs"),
                     "gather_peak_measured_gbs": MEASURED.get("gather_8mib_gbs"),
                     "frac_measured_gather": sg.get("frac_measured_gather")})
    # the indexer, the other large kernel, against the MFMA peak as well
    idx_roof = (roofline_entry("indexer_topm", stages["indexer_topm"], flops["indexer_topm"], "mfma",
                               traffic_from_profiles("indexer_topm", phase))
                if "indexer_topm" in stages and dom != "indexer_topm" else None)
    shape = "qwen2.5-1.5b-shaped" if small else "qwen2.5-7b-shaped"
    res = {
        "workload": f"lisa_prefill {shape} B={B} n={n} Hq={cfg.Hq} Hkv={cfg.Hkv} "
                    f"d={cfg.d} indexer={cfg.HI}x{cfg.dI} M={cfg.M} C={cfg.chunk} bf16",
        "tokens_per_s": B * n / (ms * 1e-3), "ms": ms, "steps": steps, "copies": copies,
        "roofline": roof, "roofline_indexer": idx_roof, "stages": stage_rows,
        "step_roofline": {"bound": "mfma", "algorithmic_flops": total_flops,
                          "achieved_tflops": round(total_flops / (ms * 1e-3) / 1e12, 3),
                          "frac": round(total_flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                          "frac_measured_peak": round(total_flops / (ms * 1e-3) / 1e12 /
                                                      MEASURED["mfma_bf16_tflops"], 4)
                          if MEASURED.get("mfma_bf16_tflops") else None},
        "cfg": cfg, "inp": inp,
    }
    del sets, outs, idx, ws
    torch.cuda.empty_cache()
    return res


def rotating_copies(bytes_per_step):
    """Input copies to rotate over so that the bytes read between repeats of
    a copy add up to at least 3 x the 256 MB Infinity Cache (9 x ~96 MB for
    the 16K decode, 2 x ~427 MB for the ragged batch); at least 2."""
    return max(2, -(-3 * 256 * 2**20 // bytes_per_step))


def bench_decode(args, ragged=False):
    """One decode step: the 16K Qwen2.5-1.5B-shaped batch of 16, or (ragged)
    the Qwen2.5-7B-shaped batch of 32 with contexts U[4096, 32768]."""
    import numpy as np
    import torch
    from hybrid_linear_top_amd import inputs as gen, lisa
    cfg = gen.DECODE_7B_RAGGED if ragged else gen.DECODE_1P5B_16K
    inp = gen.make_decode_inputs(cfg)
    dims = lisa.dims_from_config(cfg)
    B = inp["B"]
    by = decode_bytes(cfg, inp["lengths"])
    copies = rotating_copies(by["total"])
    cu = lisa.to_device(inp["cu_ctx"])
    shared = {k: lisa.to_device(inp[k]) for k in ("q", "q_idx", "w_idx", "gate")}
    per = [{k: lisa.to_device(inp[k]) for k in ("k_cache", "v_cache", "k_idx_cache", "state")}
           for _ in range(copies)]
    out = torch.empty_like(shared["q"])
    idx = torch.empty((B, cfg.Hkv, cfg.M), dtype=torch.int32, device="cuda")
    ws = torch.empty(lisa.lisa_decode_workspace_bytes(dims, B, inp["max_ctx"]), dtype=torch.uint8,
                     device="cuda")

    def step(c):
        p = per[c]
        lisa.decode_step(dims, cu, inp["max_ctx"], shared["q"], p["k_cache"], p["v_cache"],
                         shared["q_idx"], p["k_idx_cache"], shared["w_idx"], shared["gate"],
                         p["state"], out=out, topm_out=idx, workspace=ws)

    ms = timed_loop(step, args.decode_steps, args.decode_warmup, copies)
    stages = stage_pass(step, max(copies, min(args.decode_steps, 45)), copies)
    stage_rows = {}
    for k, v in stages.items():
        b = by.get(k, 0)
        stage_rows[k] = {"ms": round(v, 5),
                         "gbs": round(b / (v * 1e-3) / 1e9, 1) if b else None,
                         "frac_hbm_peak": round(b / (v * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if b else None}
    # the step is bound by its HBM stream: the kernel reported is the one
    # that carries most of the step's algorithmic bytes (the score/state
    # scan); the select and the sparse kernel are short latency chains on
    # B x G work-groups, and the dispatch events of the sparse one read up to
    # 4x its kernel-trace duration, so their event times rank nothing here
    dom = max((k for k in stages if by.get(k)), key=lambda k: by[k])
    roof = roofline_entry(dom, stages[dom], by.get(dom, 0), "hbm",
                          traffic_from_profiles(dom, "decode_7b_ragged" if ragged else "decode_1p5b_16k"))
    L = inp["lengths"]
    ctx = (f"ctx=16384+1" if not ragged else
           f"ragged ctx U[4096,32768]+1 (sum {int(L.sum())}, max {int(L.max())})")
    shape = "qwen2.5-7b-shaped" if ragged else "qwen2.5-1.5b-shaped"
    res = {
        "workload": f"lisa_decode_step {shape} B={B} {ctx} Hq={cfg.Hq} "
                    f"Hkv={cfg.Hkv} d={cfg.d} indexer={cfg.HI}x{cfg.dI} M={cfg.M} bf16",
        "tokens_per_s": B / (ms * 1e-3), "ms": ms, "roofline": roof, "stages": stage_rows,
        "step_roofline": {"bound": "hbm", "algorithmic_bytes": by["total"],
                          "achieved_gbs": round(by["total"] / (ms * 1e-3) / 1e9, 1),
                          "frac": round(by["total"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "frac_measured_peak": round(by["total"] / (ms * 1e-3) / 1e9 / MEASURED["hbm_gbs"], 4)
                          if MEASURED.get("hbm_gbs") else None},
        "cfg": cfg, "inp": inp,
    }
    del per, ws
    torch.cuda.empty_cache()
    return res


def backward_flops(cfg, n, B):
    """Algorithmic flops of the sparse branch's backward per (query head,
    selected key): the logit and d_out.v dots and the dq terms on the query
    side (3 x 2d), the dk and dv terms on the key side (2 x 2d)."""
    ph = B * cfg.Hq * pairs(n, cfg.M)
    return {"bwd_sparse_query": 6 * cfg.d * ph, "bwd_sparse_keys": 4 * cfg.d * ph,
            "bwd_sparse": 10 * cfg.d * ph}


def bench_backward(args, pre):
    import torch
    from hybrid_linear_top_amd import inputs as gen, lisa
    cfg, inp = pre["cfg"], pre["inp"]
    dims = lisa.dims_from_config(cfg)
    B, n = inp["B"], inp["n"]
    binp = gen.make_backward_inputs(cfg)
    x = {k: lisa.to_device(inp[k]) for k in ("q", "k", "v", "q_idx", "k_idx", "w_idx", "gate")}
    s0 = lisa.to_device(binp["state_in"])
    _, _, idx = lisa.prefill(dims, x["q"], x["k"], x["v"], x["q_idx"], x["k_idx"], x["w_idx"], x["gate"],
                             state_in=s0)
    dO, dS = lisa.to_device(binp["d_out"]), lisa.to_device(binp["d_state_out"])
    ws = torch.empty(lisa.lisa_prefill_backward_workspace_bytes(dims, B, n), dtype=torch.uint8,
                     device="cuda")
    phase_marker(PHASES.index("backward_7b_16k"))

    def step(c):
        lisa.prefill_backward(dims, x["q"], x["k"], x["v"], x["gate"], idx, dO, state_in=s0,
                              d_state_out=dS, want_state_grad=True, workspace=ws)

    ms = timed_loop(step, args.bwd_steps, 1, 1)
    stages = stage_pass(step, args.bwd_steps, 1)
    fl = backward_flops(cfg, n, B)
    dom = max(stages, key=stages.get)
    # the query side runs on bf16 MFMA; the key side is fp32 VALU work whose
    # ceiling in practice is the L2 atomic rate
    bound = "mfma" if dom == "bwd_sparse_query" else "alu"
    roof = roofline_entry(dom, stages[dom], fl.get(dom, 0), bound, traffic_from_profiles(dom, "backward_7b_16k"))
    res = {
        "workload": f"lisa_prefill_backward qwen2.5-7b-shaped B={B} n={n} Hq={cfg.Hq} Hkv={cfg.Hkv} "
                    f"d={cfg.d} M={cfg.M} bf16 (sets from the forward; d_state_out and state_in given)",
        "tokens_per_s": B * n / (ms * 1e-3), "ms": ms, "roofline": roof,
        "stages": {k: {"ms": round(v, 5)} for k, v in stages.items()},
    }
    del x, ws, idx
    torch.cuda.empty_cache()
    return res


def cpu_backward(pre, n_sample=1024):
    """The fp64 backward oracle (numpy loops) on the first n_sample positions
    of the same inputs, with the oracle's own sets for them."""
    import numpy as np
    from oracle import oracle as orc, backward as obwd
    from hybrid_linear_top_amd import inputs as gen
    cfg, inp = pre["cfg"], pre["inp"]
    sub = {k: (v[:, :n_sample] if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
    sub["n"] = n_sample
    fwd = orc.prefill(sub, cfg)
    binp = gen.make_backward_inputs(cfg)
    w = lambda key: orc.widen(sub[key], cfg.dtype)  # noqa: E731
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        obwd.prefill_backward(w("q"), w("k"), w("v"), w("gate"), fwd["idx"],
                              orc.widen(binp["d_out"][:, :n_sample], cfg.dtype),
                              state_in=binp["state_in"], d_state_out=binp["d_state_out"])
        secs = time.perf_counter() - t0
    return {"value": round(inp["B"] * n_sample / secs, 3), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"fp64 backward oracle (numpy loops, BLAS held to one thread) on the first "
                      f"{n_sample} positions of the same inputs ({secs:.1f}s)",
            "seconds_measured": round(secs, 2)}


def cpu_prefill(res):
    """The fp64 oracle's full prefill call on the same n=16384 inputs (all rows;
    input widening excluded from the timed region)."""
    from oracle import oracle as orc
    cfg, inp = res["cfg"], res["inp"]
    n = inp["n"]
    secs = orc.prefill(inp, cfg)["seconds"]
    return {"value": round(inp["B"] * n / secs, 3), "unit": "tokens/s", "cores": cores_used(),
            "kind": "oracle",
            "sample": f"one full fp64 oracle prefill call on the same B=1, n={n} inputs "
                      f"({secs:.1f}s); not a sample: the whole call fits the CPU budget",
            "seconds_measured": round(secs, 2)}


def cpu_decode(res, reps=31):
    from oracle import oracle as orc
    cfg, inp = res["cfg"], res["inp"]
    secs = sorted(orc.decode(inp, cfg)["seconds"] for _ in range(reps))
    med = secs[len(secs) // 2]
    return {"value": round(inp["B"] / med, 3), "unit": "tokens/s", "cores": cores_used(),
            "kind": "oracle",
            "sample": f"fp64 oracle decode step on the full batch (B={inp['B']}, 16385 visible "
                      f"tokens each), median of {reps} calls ({med:.3f}s per step)",
            "seconds_measured": round(sum(secs), 2)}


def copy_calibration(nbytes=1 << 30):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE /
    WRITE_SIZE readings (the copy reads and writes nbytes each)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return nbytes


def gather_sweep(mib=(1, 2, 4, 8, 16, 32), reps=5):
    """Random 256-byte row gather rate (GB/s) against the table size, with the
    gather probe of measure_peaks."""
    import torch
    from hybrid_linear_top_amd import lisa
    src = torch.ones((max(mib) << 20) // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty(1 << 21, dtype=torch.float32, device="cuda")
    out = {}
    for m in mib:
        times, work = [], 0.0
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            work = lisa.peak_probe(lisa.LISA_PROBE_GATHER, src, sink, m << 20, 8)
            e1.record()
            torch.cuda.synchronize()
            if r:
                times.append(e0.elapsed_time(e1))
        out[f"{m}_mib_gbs"] = round(work / (sorted(times)[len(times) // 2] * 1e-3) / 1e9, 1)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--decode-warmup", type=int, default=20)
    ap.add_argument("--bwd-steps", type=int, default=3)
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the 7B-shaped ragged decode batch (its kernels share names with the "
                         "16K decode's, so counter runs leave it out)")
    ap.add_argument("--kernel-stats", nargs=2, metavar=("DB", "OUT_MD"),
                    help="write a per-kernel duration table from a rocprofv3 --kernel-trace "
                         "database and exit")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--phase-markers", action="store_true",
                    help="launch a 4 KiB calibration copy before each phase (splits profiler databases)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak calibration")
    ap.add_argument("--gather-sweep", action="store_true",
                    help="print the row-gather probe's rate for tables of 1 to 32 MiB and exit")
    ap.add_argument("--counter-summary", nargs="+", metavar="DB",
                    help="kernel-trace database of a --phase-markers run, then one rocprofv3 --pmc database "
                         "per counter pass: write profiles/counters.json and the table, and exit")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc databases and exit")
    args = ap.parse_args()
    if args.kernel_stats:
        kernel_stats_summary(*args.kernel_stats)
        return
    if args.counter_summary:
        data = counter_summary(args.counter_summary[1:], os.path.join(PROFILES, "counters.json"),
                               os.path.join(PROFILES, "counters_prefill_decode_backward.md"),
                               durations_db=args.counter_summary[0])
        print(json.dumps(data, indent=1))
        return
    if args.traffic_summary:
        cmd = ("cd /tmp && export TMPDIR=/tmp && for c in FETCH_SIZE WRITE_SIZE; do "
               "timeout -s KILL 180 rocprofv3 --pmc $c -d $OUT/pmc_$c -o run -- "
               "python3 $REPO/bench.py --steps 2 --warmup 1 --decode-steps 9 --decode-warmup 1 "
               "--bwd-steps 1 --no-cpu-baseline --no-peaks --copy-calibration --phase-markers; done; "
               "cd $REPO && python3 bench.py "
               "--traffic-summary $OUT/pmc_FETCH_SIZE/run_results.db "
               "$OUT/pmc_WRITE_SIZE/run_results.db")
        data = traffic_summary(*args.traffic_summary, os.path.join(PROFILES, "traffic.json"),
                               os.path.join(PROFILES, "hbm_traffic_prefill16k_decode16k.md"), cmd)
        print(json.dumps(data, indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the LISA layer here is a single-GPU kernel path "
              "(no collectives are built); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    t_start = time.time()
    if args.gather_sweep:
        print(json.dumps({"gather_sweep": gather_sweep()}), flush=True)
        return
    if args.copy_calibration:
        nb = copy_calibration()
        print(json.dumps({"copy_calibration_bytes": nb}), flush=True)
    peaks = None
    if not args.no_peaks:
        peaks = measure_peaks()
        print(f"[bench] measured peaks {peaks}", file=sys.stderr, flush=True)
    if args.phase_markers:
        _MARK["src"] = torch.zeros(1024, dtype=torch.float32, device="cuda")
        _MARK["dst"] = torch.empty_like(_MARK["src"])
    phase_marker(PHASES.index("prefill_7b_16k"))
    pre = bench_prefill(args)
    print(f"[bench] prefill {pre['ms']:.3f} ms/call, stages {pre['stages']}", file=sys.stderr, flush=True)
    phase_marker(PHASES.index("prefill_1p5b_4k"))
    pre_small = bench_prefill(args, small=True)
    print(f"[bench] prefill (4K, 1.5B shapes) {pre_small['ms']:.4f} ms/call, stages {pre_small['stages']}",
          file=sys.stderr, flush=True)
    phase_marker(PHASES.index("decode_1p5b_16k"))
    dec = bench_decode(args)
    print(f"[bench] decode {dec['ms'] * 1e3:.1f} us/step, stages {dec['stages']}", file=sys.stderr, flush=True)
    rag = None
    phase_marker(PHASES.index("decode_7b_ragged"))
    if not args.no_ragged:
        rag = bench_decode(args, ragged=True)
        print(f"[bench] ragged decode {rag['ms'] * 1e3:.1f} us/step, stages {rag['stages']}", file=sys.stderr,
              flush=True)
    bwd = None
    phase_marker(PHASES.index("backward_setup"))
    if not args.no_backward:
        bwd = bench_backward(args, pre)
        print(f"[bench] backward {bwd['ms']:.2f} ms/call, stages {bwd['stages']}", file=sys.stderr, flush=True)
    cpu_p = cpu_d = cpu_b = None
    if not args.no_cpu_baseline:
        cpu_p = cpu_prefill(pre)
        print(f"[bench] cpu prefill baseline {cpu_p}", file=sys.stderr, flush=True)
        cpu_d = cpu_decode(dec)
        print(f"[bench] cpu decode baseline {cpu_d}", file=sys.stderr, flush=True)
        if bwd is not None:
            cpu_b = cpu_backward(pre)
            print(f"[bench] cpu backward baseline {cpu_b}", file=sys.stderr, flush=True)
    line = {
        "metric": METRIC,
        "value": round(pre["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": pre["workload"], "global_batch": 1, "seq_len": 16384,
                   "parallelism": "single-gpu"},
        "roofline": pre["roofline"],
        "cpu_baseline": cpu_p,
        "step_roofline": pre["step_roofline"],
        "stages": pre["stages"],
        "peaks_measured": peaks,
        "prefill_1p5b_4k": {
            "workload": pre_small["workload"], "value": round(pre_small["tokens_per_s"], 1),
            "unit": "tokens/s", "steps": pre_small["steps"], "input_copies": pre_small["copies"],
            "ms_per_step": round(pre_small["ms"], 5), "roofline": pre_small["roofline"],
            "step_roofline": pre_small["step_roofline"], "stages": pre_small["stages"],
        },
        "decode": {
            "workload": dec["workload"], "value": round(dec["tokens_per_s"], 1), "unit": "tokens/s",
            "steps": args.decode_steps, "warmup": args.decode_warmup,
            "ms_per_step": round(dec["ms"], 5), "roofline": dec["roofline"],
            "step_roofline": dec["step_roofline"], "stages": dec["stages"], "cpu_baseline": cpu_d,
        },
        "decode_ragged": None if rag is None else {
            "workload": rag["workload"], "value": round(rag["tokens_per_s"], 1), "unit": "tokens/s",
            "steps": args.decode_steps, "warmup": args.decode_warmup,
            "ms_per_step": round(rag["ms"], 5), "roofline": rag["roofline"],
            "step_roofline": rag["step_roofline"], "stages": rag["stages"],
        },
        "backward": None if bwd is None else {
            "workload": bwd["workload"], "value": round(bwd["tokens_per_s"], 1), "unit": "tokens/s",
            "steps": args.bwd_steps, "ms_per_step": round(bwd["ms"], 4), "roofline": bwd["roofline"],
            "stages": bwd["stages"], "cpu_baseline": cpu_b,
        },
        "wall_s": round(time.time() - t_start, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
