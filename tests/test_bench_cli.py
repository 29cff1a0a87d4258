"""bench.py's command line on the CPU: it measures one GPU and refuses any
other count (or a multi-rank launch) with a message and exit status 2,
before it touches torch or the GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, cwd=ROOT, env=env, timeout=60)


@pytest.mark.parametrize("n", ["2", "8", "0"])
def test_bench_refuses_other_gpu_counts(n):
    r = _run(["--gpus", n])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and "--gpus 1" in r.stderr
    assert r.stdout == ""   # no JSON line


def test_bench_refuses_multi_rank_launch():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
