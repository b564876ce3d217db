"""The benchmark's algorithmic work counts and its profile summaries (CPU).

The roofline fractions bench.py prints divide these counts by measured
times, so they are checked here against counts worked out independently:
the causal pair count T(n) and the selected pair count P(n, M) by brute
force, the per-config flop and byte totals of the layer at the sizes the
benchmark runs (16K prefill with Qwen2.5-7B shapes, 16K decode with
Qwen2.5-1.5B shapes).
"""
import os
import sqlite3
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from hybrid_linear_top_amd import inputs as gen  # noqa: E402


@pytest.mark.parametrize("n,M", [(1, 1), (5, 3), (64, 64), (100, 7), (300, 256)])
def test_pair_counts_brute_force(n, M):
    assert bench.tri(n) == sum(t + 1 for t in range(n))
    assert bench.pairs(n, M) == sum(min(M, t + 1) for t in range(n))


def test_prefill_flops_16k_7b():
    cfg = gen.PREFILL_7B_16K
    f = bench.prefill_flops(cfg, cfg.n, 1)
    n, G, Hq, d, M, C = cfg.n, cfg.Hkv, cfg.Hq, cfg.d, cfg.M, cfg.chunk
    # indexer: 2 flops per multiply-add, H_I heads of d_I per (group, causal pair)
    assert f["indexer_topm"] == 2 * G * cfg.HI * cfg.dI * n * (n + 1) // 2
    # sparse: q.k and p.v, 2 flops each per head dim, per head and selected pair
    P = n * M - M * (M - 1) // 2
    assert f["sparse_gate_prefill"] == 4 * Hq * d * P
    # chunked linear: K_c^T V_c per group and chunk; per head the masked
    # intra-chunk Q K^T and A V (2nCd each) and the inter-chunk Q S (2nd^2)
    assert f["linear_chunk_state"] == 2 * G * n * d * d
    assert f["linear_chunk_output"] == Hq * (4 * n * C * d + 2 * n * d * d)
    total = sum(f.values())
    assert abs(total - 3.668e11) / 3.668e11 < 1e-3
    assert abs(f["indexer_topm"] - 2.749e11) / 2.749e11 < 1e-3


def test_decode_bytes_16k_and_ragged():
    cfg = gen.DECODE_1P5B_16K
    L = np.full(16, 16385)
    by = bench.decode_bytes(cfg, L)
    assert by["kI"] == 16 * 16385 * cfg.Hkv * cfg.dI * 2
    assert by["state"] == 16 * cfg.Hq * cfg.d * cfg.d * 4 * 2
    assert by["kv_rows"] == 16 * cfg.Hkv * cfg.M * 2 * cfg.d * 2
    assert by["total"] == by["kI"] + by["kv_rows"] + by["state"] + by["small"]
    assert abs(by["total"] - 96.6e6) / 96.6e6 < 2e-3
    # the ragged batch: K/V rows are min(M, L_b) per sequence and group
    cfg4 = gen.DECODE_7B_RAGGED
    L4 = np.array([100, 600, 5000])
    by4 = bench.decode_bytes(cfg4, L4)
    assert by4["kv_rows"] == (100 + 512 + 512) * cfg4.Hkv * 2 * cfg4.d * 2
    assert by4["kI"] == int(L4.sum()) * cfg4.Hkv * cfg4.dI * 2


def test_backward_flops_per_pair():
    cfg = gen.PREFILL_7B_16K
    fl = bench.backward_flops(cfg, cfg.n, 1)
    P = bench.pairs(cfg.n, cfg.M)
    assert fl["bwd_sparse_query"] == 6 * cfg.d * cfg.Hq * P
    assert fl["bwd_sparse_keys"] == 4 * cfg.d * cfg.Hq * P
    assert fl["bwd_sparse"] == fl["bwd_sparse_query"] + fl["bwd_sparse_keys"]


def test_kernel_stats_rows_per_grid(tmp_path):
    db = tmp_path / "k.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, grid_x integer, duration integer)")
    rows = [("void lisa::(anonymous namespace)::k_a<1>(int)", 1024, 3000),
            ("void lisa::(anonymous namespace)::k_a<1>(int)", 1024, 5000),
            ("void lisa::(anonymous namespace)::k_a<1>(int)", 4096, 10000),
            ("void lisa::(anonymous namespace)::k_b(int)", 64, 2000)]
    con.executemany("insert into kernels values (?, ?, ?)", rows)
    con.commit()
    out = tmp_path / "k.md"
    bench.kernel_stats_summary(str(db), str(out))
    lines = [ln for ln in out.read_text().splitlines() if ln.startswith("| `")]
    assert len(lines) == 3
    # ordered by total time; durations in microseconds; namespace trimmed
    assert lines[0].startswith("| `k_a<1>(int)` | 4096 | 1 | 10.0 | 10.00 |")
    assert lines[1].startswith("| `k_a<1>(int)` | 1024 | 2 | 8.0 | 4.00 |")
    assert lines[2].startswith("| `k_b(int)` | 64 | 1 | 2.0 | 2.00 |")


def test_rotating_copies_exceed_the_infinity_cache():
    # the decode benchmark rotates enough input copies that their bytes read
    # between repeats are at least 3 x 256 MB
    for cfg, expect in ((gen.DECODE_1P5B_16K, 9), (gen.DECODE_7B_RAGGED, 2)):
        total = bench.decode_bytes(cfg, gen.decode_lengths(cfg))["total"]
        copies = bench.rotating_copies(total)
        assert copies * total >= 3 * 256 * 2 ** 20
        assert (copies - 1) * total < 3 * 256 * 2 ** 20 or copies == 2
        assert copies == expect
