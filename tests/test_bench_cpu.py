"""bench.py's command-line contract on the CPU: more than one GPU is refused with a
message (the path is built and measured on one GPU) before any GPU work starts."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "4"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_help_lists_the_options():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--no-cpu-baseline", "--no-model", "--no-other", "--sweep",
                "--ramp-ms"):
        assert opt in r.stdout, opt
