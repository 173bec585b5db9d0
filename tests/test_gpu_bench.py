"""bench.py end to end on the GPU: one short default run prints one JSON line
with every field of the reporting contract, the roofline and the CPU
baseline, and values that are consistent with each other."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args]
    say("running", " ".join(cmd[2:]))
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=180, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def test_default_bench_line():
    need_gpu()
    d = run_bench("--steps", "4", "--warmup", "1", "--cpu-budget", "0.5")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 4 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["dtype"] == "bf16"
    assert "workload" in d["config"]
    assert d["value"] > 0 and d["ms_per_step"] > 0
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["achieved"] < rf["peak"]
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], abs=1e-4)
    # the step (split + merge) reads the same K/V as the split kernel alone, so it is not faster
    assert d["value"] <= rf["achieved"] * 1.05
    dev = d["device"]
    assert dev["compute_units"] > 0 and dev["max_clock_mhz"] > 0 and dev["bf16_dense_peak_tflops_from_props"] > 0
    vref = d["vendor_attention_reference"]
    if vref["value"] is not None:   # the same attention within the bf16 tolerance
        assert vref["max_abs_diff_from_this_library"] <= 2e-2
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    for part, bound in (("prefill", "mfma"), ("prefill_backward", "mfma")):
        p = d[part]
        assert p["value"] > 0 and p["roofline"]["bound"] == bound
        assert 0 < p["roofline"]["frac"] < 1
    ref = d["prefill"]["matmul_reference"]
    assert ref["unit"] == "TFLOP/s" and ref["value"] > 0 and ref["prefill_over_reference"] > 0
    att = d["prefill"]["vendor_attention_reference"]
    if att["value"] is not None:   # the same attention within the bf16 tolerance
        assert att["max_abs_diff_from_this_library"] <= 2e-2
    batt = d["prefill_backward"]["vendor_attention_reference"]
    if batt["value"] is not None:   # the same gradients, relative to each one's largest magnitude
        assert batt["max_rel_diff_from_this_library"] <= 2e-2


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "4"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_expanded_cache_ab_line():
    """--expanded: the same decode kernel on K/V repeated to Hq heads gives the
    same attention (within the bf16 tolerance of the grouped result) and
    reads g = 4 times the bytes, so its step is several times longer."""
    need_gpu()
    d = run_bench("--steps", "4", "--warmup", "1", "--no-cpu-baseline", "--no-prefill", "--expanded")
    x = d["expanded_ab"]
    say("expanded", x)
    assert x["max_abs_diff_vs_grouped"] <= 2e-2
    assert x["kv_bytes"] == 4 * 1073741824
    assert x["slowdown_vs_grouped"] > 2.0
    assert x["ms_per_step"] > 0 and x["grouped_ms_per_step"] == d["ms_per_step"]
