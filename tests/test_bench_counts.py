"""bench.py's algorithmic counts (the denominators of every reported roofline
fraction) against figures derived independently from the problem sizes:
the survey's per-workload table of causal flops F = B H T [Q(Q+1)(N+P) + 4QPN]
and compulsory bytes B_min, and compute_out's byte count.  CPU only."""
import os
import subprocess
import sys

import pytest

import bench
import ssd_synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name,gflop,bmin_mb", [
    ("mamba2_780m", 32.29, 112.7),
    ("mamba2_2p7b", 107.63, 359.7),
    ("long_prefill", 861.0, 2796),
    ("large_state", 224.0, 847.2),
])
def test_path_counts_match_the_table(name, gflop, bmin_mb):
    c = bench.counts(ssd_synth.CONFIGS[name])
    assert abs(c["f_path"] / 1e9 - gflop) <= 0.005 * gflop
    assert abs(c["b_min"] / 1e6 - bmin_mb) <= 0.005 * bmin_mb


def test_compute_out_counts_2p7b():
    c = bench.counts(ssd_synth.CONFIGS["mamba2_2p7b"])
    # 5120 (chunk, head) units of Q(Q+1)(N+P) + 2QPN flops; x read + y written,
    # chunk states, G and dt rows, B and C rows, D
    assert c["units_out"] == 2 * 32 * 80
    assert c["f_out"] == 5120 * (256 * 257 * 192 + 2 * 256 * 64 * 128)
    assert abs(c["b_out"] / 1e6 - 438.3) < 0.05
    assert c["tokens"] == 2 * 8192


def test_decode_bytes():
    p = ssd_synth.Problem(**bench.DECODE_WORKLOADS["decode_2p7b_b128"])
    # fp32 state read + written dominates: 128 x 80 x 64 x 128 x 4 x 2
    assert bench.decode_counts(p) == (2 * 4 * 128 * 80 * 64 * 128 + 2 * 128 * 80 * 64 * 2
                                      + 2 * 128 * 128 * 2 + 4 * 128 * 80 + 8 * 80)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_bwd_counts_2p7b():
    # per (batch, chunk, head): Q(Q+1)/2 causal pairs x (3N + 2P) FMAs for the
    # chunk x chunk products, 5 Q P N for the state products; 2 flops per FMA
    import ssd_synth
    c = bench.bwd_counts(ssd_synth.CONFIGS["mamba2_2p7b"])
    pairs = 256 * 257 // 2
    assert c["per_unit"] == 2 * (pairs * (3 * 128 + 2 * 64) + 5 * 256 * 64 * 128) == 54657024
    assert c["units"] == 2 * 80 * 32
    assert round(c["flops"] / 1e9, 2) == 279.84
    # blended peak: 33.69 MFLOP at 2.5 PFLOP/s plus 20.97 MFLOP at 157.3 TFLOP/s
    assert c["chunk_per_unit"] == 2 * pairs * (3 * 128 + 2 * 64)
    t = c["chunk_per_unit"] / 2.5e15 + c["state_per_unit"] / 157.3e12
    assert abs(c["peak"] - c["per_unit"] / t) < 1.0 and 372e12 < c["peak"] < 373e12
