"""bench.py's host-side logic, on the CPU: the one-GPU guard, the counter
ingestion (copy-probe calibration) and when the traffic figure is reported."""
import csv
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "more than one GPU" in (r.stdout + r.stderr)


def test_ingest_scales_by_the_copy_probe_and_keys_the_workload(tmp_path):
    gib = 2.0 ** 20                                   # KiB per GiB
    names = {p: f"void kd::gemm_nt_kernel<kd::Bf16, 256, 256, 2, 4, 2, kd::{t}, 128>"
             for p, t in bench.PHASE_KERNEL_TAGS.items()}
    copy = "__amd_rocclr_copyBuffer"
    # the probe copy of 2 GiB reads as 1 GiB fetched and 2 GiB written
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, 1 * gib)] + [(n, 3 * gib) for n in names.values()] +
         [(names["gemm_dW"], 5 * gib)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, 2 * gib)] + [(n, 0.5 * gib) for n in names.values()] +
         [(names["gemm_dW"], 0.5 * gib)])
    out = tmp_path / "traffic.json"
    assert bench.ingest_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), out=str(out)) == 0
    rec = json.load(open(out))
    assert rec["copy_scale"] == {"fetch": 2.0, "write": 1.0}
    k = rec["kernels"]["gemm_fwd_lse"]
    assert k["fetch_bytes"] == 6 * 2 ** 30 and k["write_bytes"] == 2 ** 29 and k["dispatches"] == 1
    assert rec["kernels"]["gemm_dW"]["fetch_bytes"] == 8 * 2 ** 30        # mean of 3 and 5 GiB, x2
    key = bench.workload_key(3, 32768, 2048)
    assert rec["workload"] == key
    total, detail = bench.load_traffic("gemm_fwd_lse", key, path=str(out))
    assert total == 6 * 2 ** 30 + 2 ** 29 and detail["copy_scale"]["fetch"] == 2.0
    # another workload, or kernels changed since: no figure
    assert bench.load_traffic("gemm_fwd_lse", bench.workload_key(1, 512, 128), path=str(out)) == (None, None)
    rec["kernel_source_hash"] = "0" * 16
    json.dump(rec, open(out, "w"))
    assert bench.load_traffic("gemm_fwd_lse", key, path=str(out)) == (None, None)
