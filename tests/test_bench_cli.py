"""CPU: bench.py's contract that needs no GPU -- one GPU only, and the peak sanity check."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_sanity_flags_rates_above_peak():
    ok = {"value": 0.9, "roofline": {"achieved": 970.0, "peak": 8000.0, "unit": "GB/s"},
          "split_kernel": {"achieved_gbs": 1600.0},
          "secondary": {"p": {"roofline": {"achieved": 28.0, "peak": 157.3}}}}
    assert bench.sanity(ok) == []
    bad = {"value": 9.0, "roofline": {"achieved": 9000.0, "peak": 8000.0, "unit": "GB/s"},
           "split_kernel": {"achieved_gbs": 8100.0},
           "secondary": {"p": {"roofline": {"achieved": 200.0, "peak": 157.3}}}}
    found = bench.sanity(bad)
    assert len(found) == 4, found
