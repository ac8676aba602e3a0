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


def test_record_traffic_reads_counter_runs(tmp_path, monkeypatch):
    """--record-traffic turns four rocprofv3 counter tables (kernel and copy, FETCH_SIZE and WRITE_SIZE) into the
    traffic record: counter values summed per dispatch over their instances, scaled by the copy's calibration."""
    kernel = "void sattn::(anonymous namespace)::attn_pipe_kernel<2, 128, 4, false, false>(sattn::AttnArg)"
    fused = "void sattn::(anonymous namespace)::attn_pipe_kernel<2, 128, 4, false, true>(sattn::AttnArg)"
    header = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"

    def table(run, rows):
        d = tmp_path / run
        d.mkdir()
        (d / "run_counter_collection.csv").write_text(
            header + "".join(f'{i},"{n}",C,{v}\n' for i, n, v in rows))

    # two dispatches of the timed kernel, each counted in two instances; one of the fused kernel (ignored)
    table("pmc_FETCH_SIZE", [(1, fused, 9e9), (2, kernel, 100.0), (2, kernel, 300.0), (3, kernel, 500.0),
                             (3, kernel, 100.0)])
    table("pmc_WRITE_SIZE", [(2, kernel, 40.0), (3, kernel, 60.0)])
    table("copy_FETCH_SIZE", [(1, "fill", 5.0), (2, "__amd_rocclr_copyBuffer", 131072.0)])
    table("copy_WRITE_SIZE", [(2, "__amd_rocclr_copyBuffer", 262144.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.record_traffic(str(tmp_path), "wan14b-720p", 2)
    rec = json.loads(out.read_text())["wan14b-720p/mode2"]
    assert rec["fetch_kib_per_dispatch"] == [400.0, 600.0] and rec["write_kib_per_dispatch"] == [40.0, 60.0]
    assert rec["copy_calibration"]["fetch_factor"] == 2.0 and rec["copy_calibration"]["write_factor"] == 1.0
    assert rec["fetch_bytes"] == 500 * 2 * 1024 and rec["write_bytes"] == 50 * 1024
    assert rec["kernel_source_sha"] == bench.kernel_source_hash()
    # the record it wrote is the one the benchmark then reports
    got = bench.measured_traffic("wan14b-720p", 2, 1.0)
    assert got["total_bytes"] == rec["fetch_bytes"] + rec["write_bytes"]


def test_gpu_sampler_reads_sysfs_files_only(tmp_path, monkeypatch):
    """The clock/power sampler reads hwmon power and the current pp_dpm_sclk level from sysfs, and reports None when
    there is no AMD card to read (as in a container without a GPU)."""
    card = tmp_path / "card0" / "device"
    (card / "hwmon" / "hwmon3").mkdir(parents=True)
    (card / "vendor").write_text("0x1002\n")
    (card / "hwmon" / "hwmon3" / "power1_input").write_text("1288000000\n")
    (card / "hwmon" / "hwmon3" / "power1_cap").write_text("1400000000\n")
    (card / "pp_dpm_sclk").write_text("S: 1973Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    import glob as globmod

    real_glob = globmod.glob
    monkeypatch.setattr(globmod, "glob", lambda p: real_glob(p.replace("/sys/class/drm", str(tmp_path))))
    s = bench.GpuSampler(period_s=0.001).start()
    import time

    time.sleep(0.02)
    out = s.stop()
    assert out["power_cap_w"] == 1400.0 and out["power_w_median"] == 1288.0
    assert out["sclk_mhz_median"] == 1973 and out["samples"] >= 1
    monkeypatch.setattr(globmod, "glob", lambda p: [])
    assert bench.GpuSampler().start().stop() is None
