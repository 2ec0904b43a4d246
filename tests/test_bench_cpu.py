"""Host logic of bench.py (CPU): the one-GPU guard and the traffic figure computed from
rocprofv3 counter files (synthetic csv folders written here)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def _counter_folder(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_pmc_summary_scales_by_the_copy_calibration(tmp_path, capsys):
    cal = bench.CALIBRATION_MIB << 10  # KiB a calibration copy moves each way
    # the copy reads half its bytes through FETCH_SIZE and all of them through WRITE_SIZE
    _counter_folder(tmp_path / "cf", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", cal / 2)] * 4)
    _counter_folder(tmp_path / "cw", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", cal)] * 4)
    _counter_folder(tmp_path / "f", "FETCH_SIZE", [("void moe::ffn_stream_rows_kernel<0, 4>(int)", 1000.0),
                                                   ("void moe::ffn_stream_rows_kernel<0, 4>(int)", 3000.0),
                                                   ("moe::combine_kernel(int)", 99999.0)])
    _counter_folder(tmp_path / "w", "WRITE_SIZE", [("void moe::ffn_stream_rows_kernel<0, 4>(int)", 10.0)])

    class A:
        workload = "decode20b"
        pmc_summary = [str(tmp_path / d) for d in ("cf", "cw", "f", "w")]

    bench.pmc_summary(A, 64)
    line = capsys.readouterr().out.strip()
    kv = dict(t.split("=", 1) for t in line.split()[1:])
    # mean FETCH 2000 KiB x 2 + mean WRITE 10 KiB x 1, in bytes; kernels outside the FFN ignored
    assert int(kv["bytes"]) == (2000 * 2 + 10) * 1024
    assert kv["src"] == bench.kernel_source_hash("decode20b")
    assert "combine" not in kv["kernels"]


def test_stored_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    f = tmp_path / "t.md"
    f.write_text("traffic workload=decode20b T=64 src=%s bytes=123\n"
                 "traffic workload=prefill20b T=4096 src=0000000000000000 bytes=456\n"
                 % bench.kernel_source_hash("decode20b"))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.stored_traffic("decode20b", 64) == 123
    assert bench.stored_traffic("decode20b", 32) is None
    assert bench.stored_traffic("prefill20b", 4096) is None  # another kernel source
