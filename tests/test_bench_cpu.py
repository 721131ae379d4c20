"""Host-side checks of bench.py's contract (no GPU needed)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "single GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_committed_decode_counters_match_the_sources():
    """The HBM byte count bench.py reports as roofline.traffic is read from the committed
    counter summary, keyed by a hash of the decode sources: it must match the tree."""
    b = bench.decode_traffic()
    assert b is not None, "decode sources changed since the HBM counters were taken"
    algorithmic = 8 * 8 * 131072 * 108
    assert algorithmic <= b < 1.1 * algorithmic
