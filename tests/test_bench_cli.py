"""bench.py's command line on the host: more than one GPU is refused with a
message, and the run stops before touching a device when none is present."""

import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the host without a GPU")
def test_no_gpu_stops_before_any_timing():
    r = run_bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr
    assert '"metric"' not in r.stdout
