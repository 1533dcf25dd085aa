"""Host-side pieces of bench.py that need no GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_spread_percentiles_and_aa_noise():
    # even blocks 10, odd blocks 12: medians 10 and 12, overall median 11
    r = bench.spread([10.0, 12.0] * 5)
    assert r["blocks"] == 10 and r["p50"] == 11.0
    assert r["p10"] == 10.0 and r["p90"] == 12.0
    assert abs(r["aa_noise"] - 2.0 / 11.0) < 1e-4
    assert "aa_noise" not in bench.spread([1.0, 2.0, 3.0])


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert p.returncode == 2 and "one GPU" in p.stderr and p.stdout == ""
