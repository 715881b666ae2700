"""Host-side logic of bench.py: the HBM-traffic record written from rocprofv3
counter files, and the one-GPU guard.  No GPU work."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEC = "void cg::(anonymous namespace)::k_decode_win<10>(cg::DecodeArgs)"
ENC = "void cg::(anonymous namespace)::k_encode<10>(cg::EncodeArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _counters(path, rows):
    """A counter_collection.csv with the columns bench.py reads; rows are
    (dispatch id, kernel name, value), several rows per dispatch allowed."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, k, v in rows:
            w.writerow([d, k, "X", v])
    return str(path)


def test_record_then_read_traffic(tmp_path):
    # a decoder dispatch split over two rows (summed), an encoder dispatch that
    # must be ignored, a copy that reads half its bytes on FETCH_SIZE
    fetch = _counters(tmp_path / "f.csv", [(5, ENC, 999.0), (7, DEC, 300.0), (7, DEC, 200.0)])
    write = _counters(tmp_path / "w.csv", [(5, ENC, 1.0), (7, DEC, 1500.0)])
    cf = _counters(tmp_path / "cf.csv", [(1, "fill", 3.0), (2, COPY, 524288.0), (3, COPY, 10.0)])
    cw = _counters(tmp_path / "cw.csv", [(2, COPY, 1048576.0)])
    out = tmp_path / "traffic.json"
    bench.record_traffic(str(out), "wl", fetch, write, cf, cw)
    rec = json.load(open(out))
    assert rec["copy_calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["copy_calibration"]["write_scale"] == pytest.approx(1.0)
    assert rec["workloads"]["wl"]["bytes_per_launch"] == 1024 * (500 * 2 + 1500)
    assert bench.decode_traffic(str(out), "wl") == 1024 * 2500
    assert bench.decode_traffic(str(out), "other") is None
    # a second workload joins the same record
    bench.record_traffic(str(out), "wl2", fetch, write, cf, cw)
    assert set(json.load(open(out))["workloads"]) == {"wl", "wl2"}


def test_traffic_is_dropped_when_the_decoder_changes(tmp_path):
    out = tmp_path / "traffic.json"
    json.dump({"kernel": "k_decode", "kernel_source_sha256": "0" * 64,
               "workloads": {"wl": {"bytes_per_launch": 1}}}, open(out, "w"))
    assert bench.decode_traffic(str(out), "wl") is None
    assert bench.decode_traffic(str(tmp_path / "missing.json"), "wl") is None


def test_decoder_kernel_name():
    assert bench.decode_kernel_name((0, 1, 2, 0, 1, 2)) == "k_decode_win"
    assert bench.decode_kernel_name((0,)) == "k_decode_reg"
    assert bench.decode_kernel_name((0, 1, 2)) == "k_decode_reg"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _sq(path, rows):
    """A counter_collection.csv with timestamps: rows are (dispatch id, kernel
    name, counter, value, start ns, end ns)."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for r in rows:
            w.writerow(r)
    return str(path)


def test_record_then_read_valu(tmp_path):
    # 2e8 VALU instructions over 1,024 SIMDs in 8e5 GRBM cycles per XCD (8 XCDs),
    # in a launch of 400 us: busy = 2e8 * 4 / (1024 * 8e5), clock 2 GHz
    sq1 = _sq(tmp_path / "s1.csv", [(3, DEC, "SQ_INSTS_VALU", 2e8, 1000, 401000),
                                    (2, ENC, "SQ_INSTS_VALU", 9e9, 0, 5)])
    sq2 = _sq(tmp_path / "s2.csv", [(3, DEC, "GRBM_GUI_ACTIVE", 6.4e6, 1000, 401000)])
    agent = tmp_path / "agent.csv"
    with open(agent, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Simd_Count", "Num_Xcc", "Max_Engine_Clk_Fcompute"])
        w.writerow([0, 0, 0])          # a CPU agent
        w.writerow([1024, 8, 2400])
    out = tmp_path / "traffic.json"
    bench.record_valu(str(out), "wl", [sq1, sq2], str(agent))
    v = bench.decode_valu(str(out), "wl", 1e7)
    assert v["busy_frac"] == pytest.approx(2e8 * 4 / (1024 * 8e5), abs=1e-4)
    assert v["clock_GHz"] == pytest.approx(2.0)
    assert v["issue_frac_at_peak_clock"] == pytest.approx(2e8 * 4 / (1024 * 2.4 * 4e5), abs=1e-4)
    assert v["insts_per_symbol"] == 20.0
    # a traffic record for the same workload keeps the VALU record beside it
    fetch = _counters(tmp_path / "f.csv", [(7, DEC, 500.0)])
    write = _counters(tmp_path / "w.csv", [(7, DEC, 1500.0)])
    cf = _counters(tmp_path / "cf.csv", [(2, COPY, 524288.0)])
    cw = _counters(tmp_path / "cw.csv", [(2, COPY, 1048576.0)])
    bench.record_traffic(str(out), "wl", fetch, write, cf, cw)
    assert bench.decode_valu(str(out), "wl", 1e7) is not None
    assert bench.decode_traffic(str(out), "wl") == 1024 * 2500


def test_record_modes_do_no_gpu_work(tmp_path):
    # each record mode writes its record and exits before any GPU or input work
    fetch = _counters(tmp_path / "f.csv", [(7, DEC, 500.0)])
    write = _counters(tmp_path / "w.csv", [(7, DEC, 1500.0)])
    cf = _counters(tmp_path / "cf.csv", [(2, COPY, 524288.0)])
    cw = _counters(tmp_path / "cw.csv", [(2, COPY, 1048576.0)])
    out = tmp_path / "t.json"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--traffic-json", str(out), "--record-traffic", fetch, write, cf, cw],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    sq = _sq(tmp_path / "s.csv", [(3, DEC, "SQ_INSTS_VALU", 2e8, 0, 400000),
                                  (3, DEC, "GRBM_GUI_ACTIVE", 6.4e6, 0, 400000)])
    agent = tmp_path / "agent.csv"
    with open(agent, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Simd_Count", "Num_Xcc", "Max_Engine_Clk_Fcompute"])
        w.writerow([1024, 8, 2400])
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--traffic-json", str(out), "--record-valu", sq, str(agent)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    rec = json.load(open(out))["workloads"]["tiny"]
    assert "bytes_per_launch" in rec and "valu" in rec


def test_entropy_of_count_rows():
    import numpy as np
    # a fair coin over four symbols, and a certain symbol: 4 x 1 bit + 0
    assert bench._entropy_bits(np.array([[2, 2, 0, 0], [4, 0, 0, 0]])) == pytest.approx(4.0)
    # three equiprobable symbols, 3 each: 9 log2 3
    assert bench._entropy_bits(np.array([[3, 3, 3]])) == pytest.approx(9 * np.log2(3))
