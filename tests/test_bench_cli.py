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


@pytest.mark.gpu
def test_bench_line_fields():
    """One short run on the 16k workload: the single JSON line carries the
    contract's fields, a roofline of the dominant kernel and a CPU baseline
    of the oracle, and the step's kernels each have warm and cold times."""
    import json
    r = _bench("--workload", "qwen3_1p7b_16k", "--steps", "3", "--warmup", "1", "--no-configs",
               "--no-context", timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in rec, k
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["config"]["workload"] == "qwen3_1p7b_16k"
    assert rec["value"] > 0 and rec["ms_per_step"] > 0
    assert abs(rec["value"] - rec["config"]["tokens"] / (rec["ms_per_step"] * 1e-3)) < 1e-6 * rec["value"]
    roof = rec["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] in ("hbm", "mfma", "alu") and 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    cpu = rec["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    for n in ("gate", "select", "gather", "attention"):
        assert rec["kernels"][n]["ms"] > 0 and rec["kernels"][n]["ms_cold"] > 0
