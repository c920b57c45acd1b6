"""bench.py's command-line contract on the CPU: one GPU only, and no device work before the
argument check (so the refusal works on any machine)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    for n in ("2", "8"):
        r = _bench("--gpus", n, "--steps", "1", "--warmup", "0")
        assert r.returncode == 2, r.stderr
        assert "one GPU only" in r.stderr and r.stdout == ""


def test_help_lists_the_contract_flags():
    r = _bench("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--codes"):
        assert flag in r.stdout
