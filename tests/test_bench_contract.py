"""bench.py's command-line contract on the host: more than one GPU is refused with a JSON
message and exit status 2 (the library runs on one GPU), before anything touches a GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
