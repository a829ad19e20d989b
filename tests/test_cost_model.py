"""bench.py's flop and byte model against the numbers the pages print
(golden fixtures, CPU only)."""
import json
import math
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MIB = 2.0 ** 20


def test_lesson06_traffic_table():
    """'Flash Attention -- five lessons converging into 80 lines', Results
    and Lesson 1: naive (4N^2 + 4Nd) and flash 4Nd fp32 elements, printed in
    MiB ('MB'), and their ratio 1 + N/d, for one head at d = 64."""
    g = json.load(open(os.path.join(GOLDEN, "lesson06_t4_results.json")))
    d, e = g["d"], g["elem_bytes"]
    for row in g["rows"]:
        n = row["N"]
        naive = bench.naive_fwd_bytes(1, 1, n, d, e, e, lse=False)
        flash = bench.fused_fwd_bytes(1, 1, n, d, e, lse=False)
        assert naive / MIB == pytest.approx(row["naive_hbm"], abs=0.05)
        assert flash / MIB == pytest.approx(row["flash_hbm"], abs=0.005)
        assert round(naive / flash) == row["ratio"]
        assert naive / flash == pytest.approx(1 + n / d)


def test_lesson06_speedup_and_throughput():
    """The printed speedups are naive ms / flash ms, and the printed GFLOP/s
    re-derive from 4 N^2 d + 3 N^2 flops per head (the page counts the
    softmax too; the bench credits 4 N^2 d only)."""
    g = json.load(open(os.path.join(GOLDEN, "lesson06_t4_results.json")))
    for row in g["rows"]:
        assert row["naive_ms"] / row["flash_ms"] == pytest.approx(row["speedup"], abs=0.006)
    first, last = g["rows"][0], g["rows"][-1]
    f = lambda n: 4 * n * n * 64 + 3 * n * n  # noqa: E731
    gf = g["gflops"]
    assert f(first["N"]) / (first["naive_ms"] * 1e-3) / 1e9 == pytest.approx(gf["naive_first"], rel=0.005)
    assert f(last["N"]) / (last["naive_ms"] * 1e-3) / 1e9 == pytest.approx(gf["naive_last"], rel=0.005)
    assert f(first["N"]) / (first["flash_ms"] * 1e-3) / 1e9 == pytest.approx(gf["flash_first"], rel=0.005)
    assert f(last["N"]) / (last["flash_ms"] * 1e-3) / 1e9 == pytest.approx(gf["flash_last"], rel=0.005)
    # with the bench's credited count the last flash figure is 4N^2 d / t
    assert bench.fwd_flops(1, 1, 4096, 64, False) / (last["flash_ms"] * 1e-3) / 1e9 == pytest.approx(1733.9, abs=0.1)


def test_essay_sp_traffic_table():
    """'Flash Attention: IO-awareness principle': S + P written twice and read
    twice in fp16 is 8 N^2 bytes, printed to two significant figures."""
    g = json.load(open(os.path.join(GOLDEN, "essay_sp_traffic.json")))
    for row in g["rows"]:
        b = bench.sp_roundtrip_bytes(row["N"], 2)
        assert b == 8 * row["N"] ** 2
        digits = 2 if b < 1e8 else 3 if b < 1e9 else 2
        assert float(f"{b:.{digits}g}") == pytest.approx(row["bytes"], rel=1e-9)


def test_essay_sram_budget():
    """'Flash Attention: IO-awareness principle', Tiling: five 64 x 64 fp16
    tiles are 8 KB each, 40 KB of 192 KB, and N = 1024 splits into 16 x 16
    tiles."""
    g = json.load(open(os.path.join(GOLDEN, "essay_sram_budget.json")))
    tile = g["br"] * g["d"] * g["elem_bytes"]
    assert tile == g["tile_kib"] * 1024
    assert 5 * tile == g["total_kib"] * 1024 < g["sram_kib"] * 1024
    assert math.ceil(g["N"] / g["br"]) == g["tr"] and math.ceil(g["N"] / g["bc"]) == g["tc"]


def test_workload_flop_counts():
    """Credited flops of the workloads (4 B H N^2 d forward, 10 B H N^2 d
    backward, halved for causal)."""
    assert bench.fwd_flops(2, 32, 8192, 128, True) == pytest.approx(1.0995e12, rel=1e-4)
    assert bench.fwd_flops(1, 16, 16384, 64, True) == pytest.approx(549.8e9, rel=1e-4)
    assert bench.fwd_flops(4, 16, 4096, 128, True) == pytest.approx(274.9e9, rel=1e-4)
    assert bench.bwd_flops(4, 16, 4096, 128, True) == pytest.approx(687.2e9, rel=1e-4)
    assert bench.fused_fwd_bytes(2, 32, 8192, 128, 2) == 538968064
    assert bench.fused_fwd_bytes(1, 16, 16384, 64, 2) == 135266304
    assert bench.fused_bwd_bytes(4, 16, 4096, 128, 2) == 741343232
    assert bench.naive_fwd_bytes(1, 16, 16384, 64, 2, 2) == 16 * 4 * 16384 ** 2 * 2 + 135266304
