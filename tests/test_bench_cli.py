"""bench.py's command-line contract, checked without a GPU: more than one GPU
is refused with a message, and without a GPU the benchmark fails loudly
instead of falling back to the CPU (no result line is printed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None, timeout=240):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout, env=env)


@pytest.mark.parametrize("mode", [[], ["--layer"], ["--backward"], ["--decode"]])
def test_more_than_one_gpu_is_refused(mode):
    r = _bench("--gpus", "2", *mode)
    assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
    assert "one GPU" in (r.stdout + r.stderr)
    assert not any(line.startswith("{") for line in r.stdout.splitlines())


def test_no_gpu_fails_loudly():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1")
    r = _bench("--steps", "1", "--warmup", "0", "--no-cpu-baseline", env=env)
    assert r.returncode != 0
    assert not any(line.startswith("{") for line in r.stdout.splitlines())
