"""CPU test of bench.py's command line: more than one GPU is refused with a message and exit
status 2 before any GPU work (the path is measured on one GPU)."""
import json
import os
import subprocess
import sys

from tests.conftest import ROOT


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]
