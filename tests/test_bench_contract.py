"""The benchmark's command-line contract, on the CPU (no GPU is touched)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, cwd=ROOT)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = run("--gpus", n)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_workload_names_and_options():
    r = run("--help")
    assert r.returncode == 0
    for w in ("moe_decode", "moe_decode_routed", "moe_prefill", "moe_stack", "supergroup", "supergroup_a8",
              "gemv", "prerouter"):
        assert w in r.stdout
    for opt in ("--steps", "--warmup", "--batch", "--group", "--params", "--skew", "--tokens"):
        assert opt in r.stdout
