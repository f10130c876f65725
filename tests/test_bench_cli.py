"""bench.py's command line on a host without a GPU: it measures one GPU, so --gpus above 1 (or a
torch.distributed launch with more than one rank) exits with status 2 and says why, before it
imports torch or touches a device."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = _run(["--gpus", str(n)])
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_more_than_one_rank_exits_with_a_message():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr
