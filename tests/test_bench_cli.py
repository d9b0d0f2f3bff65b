"""bench.py's command line on the CPU: more than one GPU is refused with a
message (the benchmark measures one GPU; the path shards over heads with no
exchange), before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 3
    assert "one GPU" in r.stderr and r.stdout == ""
