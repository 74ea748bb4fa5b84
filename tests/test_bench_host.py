"""Host logic of bench.py (CPU): the HBM-traffic summary built from rocprofv3 counter files,
its invalidation when the kernel sources change, and the one-GPU guard.

The counter files are synthetic, in rocprofv3's counter-collection CSV form: per-dispatch
values split over several rows (one per hardware instance) are added, the last device copy
of the run (exactly 1 GiB) calibrates each counter, and the result is the mean scaled bytes
per dispatch of each kernel.
"""

import csv
import json
import os
import subprocess
import sys

import bench

STE = "void qf::k_ste<false, 1>(unsigned short const*, float*, long)"
COPY = "__amd_rocclr_copyBuffer"


def _write(folder, counter, rows):
    os.makedirs(folder)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, k, v in rows:
            w.writerow([d, k, counter, v])


def test_pmc_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    # FETCH_SIZE counts half of the copy's 1 GiB read (scale 2); dispatch 1 comes in two rows
    _write(fetch, "FETCH_SIZE", [(1, STE, 60.0), (1, STE, 40.0), (2, STE, 110.0), (3, COPY, 524288.0)])
    # WRITE_SIZE counts the copy's write exactly (scale 1)
    _write(write, "WRITE_SIZE", [(1, STE, 200.0), (2, STE, 220.0), (3, COPY, 1048576.0)])
    bench.pmc_summary(fetch, write, "w")
    data = json.load(open(tmp_path / "traffic.json"))
    assert abs(data["_calibration"]["FETCH_SIZE"]["scale"] - 2.0) < 1e-12
    assert abs(data["_calibration"]["WRITE_SIZE"]["scale"] - 1.0) < 1e-12
    e = data["w:ste_backward"]
    assert e["kernels"][STE] == {"fetch_bytes": 105 * 1024 * 2, "write_bytes": 210 * 1024}
    assert e["bytes_per_launch"] == 105 * 1024 * 2 + 210 * 1024
    assert e["source_hash"] == bench.kernel_source_hash()
    assert bench.traffic_from_profile("w:ste_backward", 1) == e["bytes_per_launch"]
    # a summary taken under other kernel sources is not reported
    e["source_hash"] = "0" * 16
    json.dump(data, open(tmp_path / "traffic.json", "w"))
    assert bench.traffic_from_profile("w:ste_backward", 1) is None
    assert bench.traffic_from_profile("w:nothing", 1) is None


def test_pmc_summary_needs_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    _write(fetch, "FETCH_SIZE", [(1, STE, 60.0)])
    _write(write, "WRITE_SIZE", [(1, STE, 200.0)])
    try:
        bench.pmc_summary(fetch, write, "w")
    except SystemExit as e:
        assert "calibration" in str(e)
    else:
        raise AssertionError("a run without the calibration copy must be refused")
    assert not (tmp_path / "traffic.json").exists()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
