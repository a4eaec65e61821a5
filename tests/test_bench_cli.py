"""Host-only checks of bench.py's contract that need no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_matches_the_kernel_sources():
    """The committed counter summary is read only while the kernel sources
    hash to the value it records; then it must give a plausible byte count."""
    sys.path.insert(0, ROOT)
    import bench
    t = bench.measured_traffic()
    if t is not None:
        assert 4.0e8 < t < 6.0e8
