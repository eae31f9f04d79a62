"""CPU checks of bench.py's measurement helpers: the rocprofv3 summaries that
profiles/ holds and the traffic lookup that bench lines report."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("name, short", [
    ("void pagedkv::(anonymous namespace)::attn_mfma_kernel<128, 6, 1, 0>(pagedkv::(anonymous namespace)::sk_args,"
     " int const*, int const*)", "attn_mfma_kernel"),
    ("void pagedkv::(anonymous namespace)::merge_sk_kernel<128>(pagedkv::(anonymous namespace)::sk_args)",
     "merge_sk_kernel"),
    ("__amd_rocclr_copyBuffer", "__amd_rocclr_copyBuffer"),
    ("at::cuda::(anonymous namespace)::spin_kernel(long)", "spin_kernel"),
])
def test_short_kernel_name(name, short):
    assert bench.short_kernel_name(name) == short


def test_counter_mean_per_dispatch(tmp_path):
    d = tmp_path / "run"
    d.mkdir()
    rows = [
        ("void pagedkv::(anonymous namespace)::attn_mfma_kernel<128, 6, 1, 0>(x)", "FETCH_SIZE", 100.0),
        ("void pagedkv::(anonymous namespace)::attn_mfma_kernel<128, 6, 1, 0>(x)", "FETCH_SIZE", 300.0),
        ("void pagedkv::(anonymous namespace)::merge_sk_kernel<128>(x)", "FETCH_SIZE", 7.0),
        ("void pagedkv::(anonymous namespace)::merge_sk_kernel<128>(x)", "WRITE_SIZE", 9.0),
    ]
    with open(d / "run_counter_collection.csv", "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
        for i, (k, c, v) in enumerate(rows):
            f.write(f'{i},"{k}","{c}",{v}\n')
    got = bench.counter_kib_per_dispatch(str(d), "FETCH_SIZE")
    assert got == {"attn_mfma_kernel": (200.0, 2), "merge_sk_kernel": (7.0, 1)}


def test_traffic_lookup_follows_the_kernel_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "pagedattention_decode_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in bench.DECODE_SOURCES:
        (csrc / name).write_text(f"// {name}, version 1\n")
    rec = {"kernel_source_sha256": bench.kernel_source_sha256(bench.DECODE_SOURCES),
           "traffic_bytes_per_launch": 123, "traffic_bytes_per_call": 456, "algorithmic_bytes_per_launch": 100}
    (tmp_path / "profiles" / "hbm_traffic_w.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("w") == 123
    assert bench.measured_traffic("w", key="traffic_bytes_per_call") == 456
    assert bench.measured_traffic("other") is None
    # the ratio comes from the counter run's own algorithmic bytes
    assert bench.traffic_ratio("w") == 1.23
    assert bench.traffic_ratio("w", key="traffic_bytes_per_call") == 4.56
    (csrc / "kernels.hip").write_text("// kernels, version 2\n")  # the counters no longer describe it
    assert bench.measured_traffic("w") is None
    assert bench.traffic_ratio("w") is None
    # a header the device code includes counts as much as the kernel file
    (csrc / "kernels.hip").write_text("// kernels.hip, version 1\n")
    assert bench.measured_traffic("w") == 123
    (csrc / "device_common.h").write_text("// operand loads changed\n")
    assert bench.measured_traffic("w") is None
    assert set(bench.DECODE_SOURCES) >= {"kernels.hip", "device_common.h", "pool_internal.h"}


def test_committed_traffic_summaries_are_consistent():
    """Every committed summary: traffic per call >= per launch, both near or below
    the algorithmic bytes' order, and a source hash of the right form."""
    prof = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(prof) if n.startswith("hbm_traffic_") and n.endswith(".json")]
    assert names
    for n in names:
        with open(os.path.join(prof, n)) as f:
            rec = json.load(f)
        assert len(rec["kernel_source_sha256"]) == 64
        assert rec["traffic_bytes_per_call"] >= rec["traffic_bytes_per_launch"] > 0, n
        assert 1.9 < rec["fetch_scale"] < 2.1 and 0.9 < rec["write_scale"] < 1.1, n


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 2 and "one GPU" in out.stderr
