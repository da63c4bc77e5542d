"""bench.py's command-line contract, checked on the host (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = run_bench("--gpus", n)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_help_lists_the_contract_flags():
    r = run_bench("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout

