"""Host-side checks of the benchmark's contract (no GPU is touched): the single-GPU refusal, and the rule that the
HBM traffic reported beside the roofline comes from counters taken on the kernel source as it stands."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (importing runs nothing: main() is behind the __main__ guard)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_traffic_record_is_used_only_for_its_kernel_source():
    """The counter record of the headline kernel names the attention source it was taken on.  While the tree holds
    that source the benchmark reports the recorded bytes; once the source changes it reports null until new
    counter runs are recorded."""
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)["wan14b-720p/mode2"]
    got = bench.measured_traffic("wan14b-720p", 2, 1.0)
    if rec["kernel_source_sha"] != bench.kernel_source_hash():
        assert got is None
        return
    assert got["total_bytes"] == rec["fetch_bytes"] + rec["write_bytes"]
    # the stored per-launch bytes are the calibrated counter readings: mean KiB per dispatch x factor x 1024 (the
    # file keeps the factor to 5 digits, hence the 1e-5 tolerance)
    cal = rec["copy_calibration"]
    fetch_kib = sum(rec["fetch_kib_per_dispatch"]) / len(rec["fetch_kib_per_dispatch"])
    assert abs(rec["fetch_bytes"] - fetch_kib * 1024 * cal["fetch_factor"]) <= 1e-5 * rec["fetch_bytes"]
    write_kib = sum(rec["write_kib_per_dispatch"]) / len(rec["write_kib_per_dispatch"])
    assert abs(rec["write_bytes"] - write_kib * 1024 * cal["write_factor"]) <= 1e-5 * rec["write_bytes"]


def test_traffic_is_null_for_another_kernel_source_or_workload(monkeypatch):
    assert bench.measured_traffic("tiny", 2, 1.0) is None              # no counter record for that workload
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)  # the kernel changed after the counters
    assert bench.measured_traffic("wan14b-720p", 2, 1.0) is None
