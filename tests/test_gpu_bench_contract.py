"""bench.py's output contract on the GPU: one JSON line with the metric,
value, unit, step counts, dtype, config, the dominant kernel's roofline
object and the CPU oracle baseline (a short run on the small workload)."""
import json
import os
import subprocess
import sys

import pytest

from gpu_cases import announce

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _reject(name):
    raise AssertionError(f"bench.py printed {name}, which is not JSON")


def test_bench_prints_one_contract_line():
    announce("bench.py contract (bs4, 3 steps)")
    r = subprocess.run([sys.executable, "bench.py", "--workload", "bs4_kv1024_fp8", "--steps", "3",
                        "--warmup", "1", "--no-other-workloads", "--cpu-sample-seqs", "1"],
                       cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0], parse_constant=_reject)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "us/call" and d["higher_is_better"] is False and d["value"] > 0
    assert abs(d["ms_per_step"] * 1e3 - d["value"]) < 0.01 + 1e-3 * d["value"]
    assert d["config"]["workload"] == "bs4_kv1024_fp8"
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    assert rl["achieved"] > 0 and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    # the bs4 cache fits the last-level cache: the cold single launch is reported too
    hot1, cold1 = rl["single_launch_us_hot_cold"]
    assert hot1 > 0 and cold1 > 0 and 0 < rl["frac_cold"] < 1
    assert "resident" in rl["cache_state"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]


def test_bench_default_run_with_other_workloads():
    """The default run (headline plus every other workload, which frees and
    rebuilds the measured case between workloads), at 3 steps."""
    announce("bench.py default run with the other workloads (3 steps)")
    r = subprocess.run([sys.executable, "bench.py", "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline"],
                       cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0], parse_constant=_reject)
    assert d["config"]["workload"] == "bs256_kv8192_fp8" and d["value"] > 0
    assert d["roofline"]["kernel"].startswith("stage1_fp8_kernel<true, false, true>")
    others = d["other_workloads"]
    assert set(others) == {"bs4_kv1024_fp8", "bs32_kv1024_fp8", "bs64_kv8192_fp8",
                           "bs256_kv1024_mxfp4"}
    for name, o in others.items():
        assert o["us_per_call"] > 0 and o["fused_kernel_us"] > 0, name


def test_bench_headline_only_line_is_strict_json():
    """The profiler runs use --headline-only, which skips the cold-cache
    figures: they must read as null, not NaN."""
    announce("bench.py --headline-only contract (bs4, 3 steps)")
    r = subprocess.run([sys.executable, "bench.py", "--workload", "bs4_kv1024_fp8", "--steps", "3",
                        "--warmup", "1", "--headline-only", "--no-cpu-baseline"],
                       cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0], parse_constant=_reject)
    rl = d["roofline"]
    assert rl["frac_cold"] is None and rl["single_launch_us_hot_cold"][1] is None
    assert rl["kernel_us"] > 0 and rl["frac"] > 0
