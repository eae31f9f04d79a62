"""bench.py's output contract on a short run: one JSON line with the metric,
the whole-job value, the roofline of the kernel that streams the cache and the
per-call timings (the GPU run itself is what the driver's bench repeats at
full length)."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    print(f"\n[case] bench.py {' '.join(args)}", flush=True)
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [line for line in out.stdout.splitlines() if line.startswith("{")]
    assert len(lines) == 1, out.stdout[-2000:]
    return json.loads(lines[0])


def test_default_decode_line():
    d = run_bench("--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["config"]["workload"] == "qwen3_8b_37x2304"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["frac"] < 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    # the call (kernel + merge) takes longer than its partition kernel
    assert d["attn_call_us"] >= d["attn_kernel_us"] > 0


def test_verify_line():
    d = run_bench("--op", "verify", "--steps", "2", "--warmup", "1", "--no-cpu-baseline")
    assert d["roofline"]["bound"] == "hbm" and d["value"] > 0

