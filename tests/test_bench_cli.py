"""bench.py's contract pieces that need no GPU: the multi-GPU refusal and
the HBM-traffic summary of rocprofv3 counter files."""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"] and msg["n_gpus"] == 2


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_by_the_copy_and_tracks_the_kernel_source(tmp_path):
    calib_kib = bench.CALIB_BYTES / 1024
    # the fetch counter reads half of what the copy moved, the write counter all of it
    _write_counters(tmp_path / "f", "FETCH_SIZE",
                    [("void pkv::attn_kernel<64, 1, 8>(...)", 100.0),
                     ("void pkv::attn_kernel<64, 1, 8>(...)", 300.0),
                     ("pkv::merge_kernel(...)", 999.0),
                     ("at::native::reduce_kernel<512, 1>(...)", calib_kib * 2),
                     ("__amd_rocclr_copyBuffer", calib_kib / 2)])
    _write_counters(tmp_path / "w", "WRITE_SIZE",
                    [("void pkv::attn_kernel<64, 1, 8>(...)", 50.0),
                     ("void pkv::attn_kernel<64, 1, 8>(...)", 50.0),
                     ("at::native::vectorized_elementwise_kernel<4, FillFunctor>", calib_kib * 4),
                     ("__amd_rocclr_copyBuffer", calib_kib)])
    out = tmp_path / "t.json"
    res = bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "c2_trellis")
    assert abs(res["fetch"]["scale"] - 2.0) < 1e-12 and abs(res["write"]["scale"] - 1.0) < 1e-12
    assert abs(res["bytes_per_launch"] - (200.0 * 1024 * 2 + 50.0 * 1024)) < 1e-6
    table = json.loads(out.read_text())
    assert table["c2_trellis"]["kernel_source_sha256"] == bench.kernel_sha256()
    # a second workload is merged into the same table
    bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "c5_verify")
    assert set(json.loads(out.read_text())) == {"c2_trellis", "c5_verify"}


def test_traffic_summary_takes_the_direct_kernel(tmp_path):
    calib_kib = bench.CALIB_BYTES / 1024
    # the library's other kernels (and the flush buffer's fill and reads)
    # must not be taken for the copy
    for sub, counter in (("f", "FETCH_SIZE"), ("w", "WRITE_SIZE")):
        _write_counters(tmp_path / sub, counter,
                        [("void pkv::direct_kernel<64, 8, 2>(...)", 40.0),
                         ("pkv::merge_kernel(...)", calib_kib * 4),
                         ("pkv::append_kernel(...)", calib_kib * 8),
                         ("__amd_rocclr_copyBuffer", calib_kib / 16),
                         ("__amd_rocclr_copyBuffer", calib_kib)])
    res = bench.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "t.json"),
                                "c2_trellis")
    assert res["kernels"] == ["direct_kernel"]
    assert res["fetch"]["attn_dispatches"] == 1 and abs(res["fetch"]["scale"] - 1.0) < 1e-12
    assert abs(res["bytes_per_launch"] - 2 * 40.0 * 1024) < 1e-6
