"""Host-side behaviour of bench.py that needs no GPU: the one-GPU refusal and the HBM traffic
summary arithmetic (counter CSVs of the shape rocprofv3 writes)."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""   # no JSON line


def _counter_csv(path, rows):
    fields = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
              "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
              "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
              "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for i, (name, counter, value) in enumerate(rows):
            w.writerow({k: 0 for k in fields} | {"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                                                 "Counter_Value": value})


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    kname = "void sh::k_head_tile<3, 16, false, 1>(sh::TileArgs)"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    cfetch, cwrite = tmp_path / "cf.csv", tmp_path / "cw.csv"
    # three 1 GiB copies whose FETCH_SIZE reads half of what they move, WRITE_SIZE exact
    _counter_csv(cfetch, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0)] * bench.COPY_LAUNCHES)
    _counter_csv(cwrite, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)] * bench.COPY_LAUNCHES)
    _counter_csv(fetch, [(kname, "FETCH_SIZE", 64000.0), (kname, "FETCH_SIZE", 64200.0),
                         ("void sh::k_head_fin<true>(sh::FinalizeArgs)", "FETCH_SIZE", 900.0)])
    _counter_csv(write, [(kname, "WRITE_SIZE", 384.0), (kname, "WRITE_SIZE", 384.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out))
    bench.traffic_summary([str(fetch), str(write), str(cfetch), str(cwrite)])
    t = json.load(open(out))
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["fetch_kib_per_dispatch"] == 64100.0 and t["write_kib_per_dispatch"] == 384.0
    assert t["hbm_bytes_per_launch"] == (2.0 * 64100.0 + 384.0) * 1024
    assert t["source_sha256"] == bench.sha_of(t["source_files"])
