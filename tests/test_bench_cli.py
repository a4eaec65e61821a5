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


def test_traffic_digest_covers_every_local_include_of_the_kernel():
    """The digest that guards the counter summary must hash every header the
    decode GEMM's source pulls in (directly or through other local headers),
    or a kernel change in a header would leave a stale summary in use."""
    import re
    sys.path.insert(0, ROOT)
    import bench
    csrc = os.path.join(ROOT, "w4a8_moe_grouped_amd", "csrc")
    seen, todo = set(), ["gemm_skinny.hip"]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        seen.add(name)
        with open(os.path.join(csrc, name)) as f:
            for inc in re.findall(r'^#include "([^"]+)"', f.read(), flags=re.M):
                if os.path.exists(os.path.join(csrc, inc)):
                    todo.append(inc)
    assert seen <= set(bench.TRAFFIC_SOURCES), sorted(seen - set(bench.TRAFFIC_SOURCES))
