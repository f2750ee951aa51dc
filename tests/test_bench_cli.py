"""bench.py's command line on the CPU: more than one GPU is refused with a message."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert p.returncode != 0
    msg = json.loads(p.stdout.strip().splitlines()[-1])
    assert msg["requested_gpus"] == 2 and "one GPU" in msg["error"]
