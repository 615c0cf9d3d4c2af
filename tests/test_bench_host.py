"""Host-side pieces of bench.py (CPU only): the one-GPU guard, the kept-pair
count behind every useful-FLOP figure, the rocprofv3 counter summary that
scales FETCH_SIZE / WRITE_SIZE by the calibration copy's readings, and the
rule that a recorded HBM-traffic figure is reported only for the kernel
source it was taken on."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


@pytest.mark.parametrize("past,sq,window", [(0, 1, -1), (5, 7, -1), (5, 7, 3), (0, 9, 1),
                                            (100, 40, 128), (3, 4, 1000)])
def test_kept_pairs_counts_each_rows_kept_keys(past, sq, window):
    # row i (absolute position past + i) keeps keys k <= past + i and, with a
    # window, k >= past + i - window + 1 (and k >= 0)
    brute = 0
    for i in range(sq):
        pos = past + i
        for k in range(pos + 1):
            if window <= 0 or k >= pos - window + 1:
                brute += 1
    assert bench.kept_pairs(past, sq, window) == brute


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_summary_scales_by_the_calibration_copy(tmp_path):
    full = ("void attn::(anonymous namespace)::attn_pp_kernel<64, 64, 4, false, false, "
            "attn::(anonymous namespace)::F16, unsigned short>(attn::Params)")
    window = ("void attn::(anonymous namespace)::attn_fwd_kernel<64, 32, 2, 2, 3, true, false, "
              "attn::(anonymous namespace)::F16, unsigned short>(attn::Params)")
    copy = "void at::native::elementwise_kernel<128, 4>(int, copy_fn)"
    fetch, write = [], []
    # three full-attention dispatches, each counter read from two instances
    for disp in (10, 11, 12):
        for part in (4000.0, 6000.0):
            fetch.append({"Dispatch_Id": disp, "Kernel_Name": full, "Counter_Name": "FETCH_SIZE",
                          "Counter_Value": part})
        write.append({"Dispatch_Id": disp, "Kernel_Name": full, "Counter_Name": "WRITE_SIZE",
                      "Counter_Value": 4096.0})
    # a window call and a small copy that must not be taken for the calibration
    fetch.append({"Dispatch_Id": 13, "Kernel_Name": window, "Counter_Name": "FETCH_SIZE",
                  "Counter_Value": 999.0})
    fetch.append({"Dispatch_Id": 14, "Kernel_Name": copy, "Counter_Name": "FETCH_SIZE",
                  "Counter_Value": 8.0})
    # the 1 GiB calibration copy: reads counted at half their bytes, writes at all
    fetch.append({"Dispatch_Id": 15, "Kernel_Name": copy, "Counter_Name": "FETCH_SIZE",
                  "Counter_Value": 524288.0})
    write.append({"Dispatch_Id": 15, "Kernel_Name": copy, "Counter_Name": "WRITE_SIZE",
                  "Counter_Value": 1048576.0})
    _counter_csv(os.path.join(tmp_path, "fetch", "x", "p_counter_collection.csv"), fetch)
    _counter_csv(os.path.join(tmp_path, "write", "x", "p_counter_collection.csv"), write)
    res = bench.summarize_counters(os.path.join(tmp_path, "fetch"), os.path.join(tmp_path, "write"))
    assert res["attn_full_launches"] == 3
    assert res["fetch_scale"] == pytest.approx(2.0) and res["write_scale"] == pytest.approx(1.0)
    assert res["attn_full_fetch_kib_raw"] == pytest.approx(10000.0)
    assert res["fetch_bytes_per_launch"] == pytest.approx(10000.0 * 2 * 1024)
    assert res["write_bytes_per_launch"] == pytest.approx(4096.0 * 1024)


def test_recorded_traffic_belongs_to_this_kernel_source():
    # profiles/full_attention_16k_traffic.txt carries the hash of the kernel
    # sources it was measured on; bench.py reports its bytes only while they match
    rec = bench.recorded_traffic()
    assert rec is not None, "the traffic record was taken on another kernel source"
    assert rec > 0
