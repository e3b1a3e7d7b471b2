"""bench.py's command-line contract that needs no GPU: asked for more than one GPU it prints one
JSON line saying why and exits non-zero, before touching the device."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode != 0
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]
