"""bench.py's command line without a GPU: more than one GPU is refused with a
message on stdout and a non-zero exit, and without a GPU the run stops with
a clear message instead of falling back to anything."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_no_gpu_stops_with_a_message():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu")
    assert r.returncode != 0
    assert "needs a GPU" in (r.stdout + r.stderr)
