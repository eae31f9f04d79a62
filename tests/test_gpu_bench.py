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
    # the default is the long-context workload, the largest that fits one GPU
    assert d["config"]["workload"] == "gqa70b_12x131072"
    assert d["config"]["partition_tokens"] == 512
    assert d["value"] > 0 and d["ms_per_step"] > 0
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["frac"] <= 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    # the call (kernel + merge) takes longer than its partition kernel
    assert d["attn_call_us"] >= d["attn_kernel_us"] > 0


@pytest.mark.parametrize("args", [
    ("--workload", "qwen3_8b_37x2304"),
    ("--workload", "shared_prefix_16x8448"),
    ("--workload", "shared_prefix_16x8448", "--cascade"),
    ("--workload", "agentic_fork_64x33281"),
    ("--workload", "agentic_fork_64x33281", "--cascade"),
    ("--workload", "qwen3_8b_37x2304", "--kv", "q8_0"),
])
def test_roofline_never_above_peak(args):
    """The roofline counts the bytes a launch must read (shared blocks once), so no
    workload reaches more than the HBM peak; logical bytes are reported apart."""
    d = run_bench(*args, "--steps", "2", "--warmup", "1", "--no-cpu-baseline")
    r = d["roofline"]
    assert 0 < r["frac"] <= 1, r
    assert d["config"]["workload"] == args[1]
    if "shared_prefix" in args[1] or "fork" in args[1]:
        # sharing sequences: the logical rate counts every sequence's own reads
        assert d["logical_achieved_gbs"] > r["achieved"]


def test_verify_line():
    d = run_bench("--op", "verify", "--steps", "2", "--warmup", "1", "--no-cpu-baseline")
    assert d["roofline"]["bound"] == "hbm" and 0 < d["roofline"]["frac"] <= 1 and d["value"] > 0


@pytest.mark.parametrize("args", [
    ("--op", "prefill", "--kv", "q8_0"),
    ("--op", "verify", "--kv", "q4_0"),
    ("--op", "prefill", "--block-size", "32"),
    ("--op", "verify", "--block-size", "8"),
    ("--workload", "shared_prefix_16x8448", "--cascade", "--kv", "q8_0"),
])
def test_other_storage_and_block_sizes(args):
    """The multi-query lines over quantised pools and other block sizes, and the
    read-once decode over a quantised pool: one JSON line whose config names
    the storage / block size, the roofline within the peak."""
    d = run_bench(*args, "--steps", "2", "--warmup", "1", "--no-cpu-baseline")
    r = d["roofline"]
    assert 0 < r["frac"] <= 1 and d["value"] > 0, r
    if "--kv" in args:
        assert d["config"]["kv_storage"] == args[args.index("--kv") + 1]
    if "--block-size" in args:
        assert d["config"]["block_size"] == int(args[args.index("--block-size") + 1])
