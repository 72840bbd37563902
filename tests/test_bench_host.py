"""Host logic of the benchmark: FLOP accounting pinned to the pages' table and
the one-GPU contract."""

import json
import os
import subprocess
import sys

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_flop_model_matches_pages_tables():
    g = json.load(open(os.path.join(GOLDEN, "table_flops.json")))
    N, d = 32760, 128  # Wan2.1-1.3B attention shape
    full = g["full_attention"]
    # printed to 2-3 significant digits: agree within the last printed digit
    assert abs(full * bench.pages_flop_fraction(0.05, N, d) - g["sla_softmax_top5"]) < 0.015
    assert abs(full * bench.pages_flop_fraction(0.05, N, d) - g["sla_table1_95pct"]) < 0.015
    assert abs(full * bench.pages_flop_fraction(0.10, N, d) - g["sla_top10"]) < 0.015
    assert abs(full * bench.pages_flop_fraction(0.20, N, d) - g["sla_top20"]) < 0.015
    assert abs(full * bench.pages_flop_fraction(0.0, N, d) - g["linear_only"]) < 0.006


def test_executed_tiles_track_kh():
    B, H, N, d = 1, 12, 32760, 128
    Nb = 512
    F = bench.dense_flops(B, H, N, d)
    assert abs(F - 6.594e12) / 6.594e12 < 1e-3
    t = bench.sparse_tile_flops(B, H, Nb, 25, d)  # n_h = floor(0.05 * 512)
    # whole tiles: 25 of 512 blocks (4.88%) within tile rounding of kh = 5%
    assert 0.047 < t / F < 0.05


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_sla1_roofline_counts_the_output_map():
    B, H, Nb, d = 1, 12, 512, 128
    extra = bench.sparse_kernel_flops(B, H, Nb, 25, d, proj=True) - bench.sparse_kernel_flops(B, H, Nb, 25, d)
    assert extra == 2.0 * B * H * Nb * 64 * d * d  # one d x d map per (tile-rounded) query token


def test_sla1_with_the_8bit_branch_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"),
                        "--config", "5", "--variant", "sla1"], capture_output=True, text=True)
    assert r.returncode == 2 and "8-bit" in r.stderr


def test_soft_topk_halvings_and_peak():
    import numpy as np
    import oracle as orc
    lg = np.random.default_rng(3).standard_normal((20, 512)) * 3
    M, lam = orc.soft_topk(lg, 25, 1e-3)
    h = bench.soft_topk_halvings(orc.compressed_map(lg), lam, 1e-3)
    # a float32 bracket ~0.12 wide halved to the spacing of floats near lambda
    assert ((h >= 20) & (h <= 40)).all()
    assert abs(bench.PEAK_SIGMOID_PER_S - 4.9152e12) < 1e9
