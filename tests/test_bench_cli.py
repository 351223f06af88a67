"""The benchmark's command line: more than one GPU is refused with a JSON
message and exit status 2, before anything touches a GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, r.stderr
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU only" in msg["error"]
