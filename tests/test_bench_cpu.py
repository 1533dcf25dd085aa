"""Host-side pieces of bench.py that need no GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_spread_percentiles_and_aa_noise():
    # even blocks 10, odd blocks 12: medians 10 and 12, overall median 11
    r = bench.spread([10.0, 12.0] * 5, 10)
    assert r["blocks"] == 10 and r["launches_per_block"] == 10 and r["p50"] == 11.0
    assert r["p10"] == 10.0 and r["p90"] == 12.0
    assert abs(r["aa_noise"] - 2.0 / 11.0) < 1e-4
    assert "aa_noise" not in bench.spread([1.0, 2.0, 3.0], 10)


def test_block_size_leaves_four_blocks_at_short_runs():
    # the driver's short run (20 steps) still yields 4 blocks, so an A/A noise floor exists
    assert bench.block_size(20) == 5 and -(-20 // bench.block_size(20)) == 4
    assert bench.block_size(200) == 10 and bench.block_size(4) == 1 and bench.block_size(1) == 1
    for k in range(1, 300):
        b = bench.block_size(k)
        assert 1 <= b <= 10 and (k < 4 or -(-k // b) >= 4)


def test_encode_kernel_names():
    assert bench.encode_kernel_name(128, 2, True, 2) == "kvq::encode_mx_kernel<128, 2, true, 2>"
    assert bench.encode_kernel_name(128, 3, True, 2) == "kvq::encode_mx_kernel<128, 3, true, 2>"
    assert bench.encode_kernel_name(256, 4, True, 2) == "kvq::encode_mx_kernel<256, 4, true, 2>"
    assert bench.encode_kernel_name(256, 3, True, 2) == "kvq::encode_kernel<256, 3, true, 2>"
    assert bench.encode_kernel_name(64, 2, False, 1) == "kvq::encode_kernel<64, 2, false, 1>"


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert p.returncode == 2 and "one GPU" in p.stderr and p.stdout == ""
