"""bench.py's command line on the host: more than one GPU is refused with a
message (this build measures one GPU), and every row named on the command
line exists."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_rows_are_known():
    sys.path.insert(0, ROOT)
    import bench
    assert set(bench.ROWS) == {"xattn", "window", "bigtree", "paged", "commit", "rope"}
