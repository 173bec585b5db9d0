"""Host-side logic of bench.py (no GPU): the one-GPU guard, the HBM counter
calibration and its staleness check, and the algorithmic byte and FLOP
counts that the roofline fractions divide by."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_record_counters_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "COUNTERS", str(tmp_path / "none.json"))   # no earlier entries
    kib = bench.CALIBRATION_BYTES / 1024
    split = "void gqa::decode_split_bf16<128, false, false>(...)"
    copy = "void at::native::vectorized_elementwise_kernel<4, ...>(...)"
    # FETCH_SIZE reads half the copy's bytes (factor 2), WRITE_SIZE a quarter (factor 4)
    _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", [(split, 100.0), (split, 300.0), (copy, kib / 2)])
    _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", [(split, 10.0), (split, 30.0), (copy, kib / 4)])
    data = bench.record_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "llama3-8b")
    assert data["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert data["calibration"]["write_factor"] == pytest.approx(4.0)
    e = data["kernels"]["decode_split|llama3-8b"]
    assert e["dispatches"] == [2, 2]
    assert e["fetch_bytes"] == 200 * 1024 * 2          # mean over dispatches, then scaled
    assert e["write_bytes"] == 20 * 1024 * 4
    assert e["traffic_bytes"] == e["fetch_bytes"] + e["write_bytes"]
    assert e["source_digest"] == bench.kernel_source_digest("decode_split")


def test_record_counters_needs_the_calibration_copy(tmp_path):
    split = "void gqa::decode_split_bf16<128, false, false>(...)"
    _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", [(split, 100.0)])
    _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", [(split, 10.0)])
    with pytest.raises(SystemExit):
        bench.record_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "llama3-8b")


def test_counters_read_as_null_once_the_sources_change(tmp_path, monkeypatch):
    path = tmp_path / "counters.json"
    entry = {"source_digest": bench.kernel_source_digest("prefill_causal"), "traffic_bytes": 12345}
    path.write_text(json.dumps({"kernels": {"prefill_causal|prefill-4k": entry}}))
    monkeypatch.setattr(bench, "COUNTERS", str(path))
    assert bench.load_counters("prefill_causal", "prefill-4k") == 12345
    assert bench.load_counters("prefill_causal", "other-workload") is None
    entry["source_digest"] = "0" * 16
    path.write_text(json.dumps({"kernels": {"prefill_causal|prefill-4k": entry}}))
    assert bench.load_counters("prefill_causal", "prefill-4k") is None


def test_every_measured_kernel_has_its_sources():
    for kernel, files in bench.KERNEL_SOURCES.items():
        for name in files:
            assert os.path.exists(os.path.join(bench.CSRC, name)), (kernel, name)
        assert len(bench.kernel_source_digest(kernel)) == 16


def test_prefill_flops_count_the_causal_pairs():
    # every (row, key) pair with key <= row costs 2 d FLOPs in Q K^T and 2 d in P V
    for n in (1, 2, 7, 64):
        pairs = int(np.tril(np.ones((n, n), dtype=np.int64)).sum())
        for b, hq, d in ((1, 1, 64), (2, 32, 128)):
            assert bench.prefill_flops(b, hq, n, d) == b * hq * pairs * 4 * d
            assert bench.prefill_backward_flops(b, hq, n, d) == 2.5 * b * hq * pairs * 4 * d


def test_decode_bytes_and_flops_follow_the_lengths():
    lens = np.array([3, 0, 5], dtype=np.int32)
    hq, hkv, d, elem = 8, 2, 64, 2
    kv = sum(2 * t * hkv * d * elem for t in lens.tolist())   # K and V rows each sequence attends
    assert bench.decode_kv_bytes(lens, hkv, d, elem) == kv
    assert bench.decode_split_bytes(lens, hq, hkv, d, elem) == kv + len(lens) * hq * d * elem
    assert bench.decode_flops(lens, hq, d) == sum(4 * hq * d * t for t in lens.tolist())


def test_prefill_bytes_are_the_tensors_it_reads_and_writes():
    b, hq, hkv, n, d = 2, 32, 8, 4096, 128
    q = b * hq * n * d * 2
    kv = 2 * b * hkv * n * d * 2
    out = b * hq * n * d * 4
    assert bench.prefill_bytes(b, hq, hkv, n, d) == q + kv + out == 234_881_024
