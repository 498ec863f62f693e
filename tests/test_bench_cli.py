"""bench.py's command line on the CPU: the checks that run before any GPU work."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]
    assert "shard" in r.stderr


def test_workload_applies_to_the_verify_op_only():
    r = run("--op", "sample", "--workload", "4")
    assert r.returncode == 2
    assert "verify op only" in r.stderr
