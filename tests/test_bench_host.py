"""bench.py's host-side logic, without a GPU: the one-GPU refusal, the counter-traffic summary
(FETCH_SIZE / WRITE_SIZE scaled by a calibration copy) and the rule that traffic figures apply
only to the kernel source, workload and key form they were taken on."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import bench
from tests.conftest import ROOT


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_counters(directory, counter, rows):
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, value in rows:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_each_counter_by_the_calibration_copy(tmp_path):
    attn = "void piclink::(anonymous namespace)::link_attention_bf16<128, true, false>(AttnParams)"
    copy = "void at::native::vectorized_elementwise_kernel<4, MulFunctor>(...)"
    # the copy reads and writes 256 MiB; FETCH_SIZE reads half of it, WRITE_SIZE all of it
    _write_counters(tmp_path / "fetch", "FETCH_SIZE", [(attn, 1000.0), (attn, 3000.0), (copy, 131072.0)])
    _write_counters(tmp_path / "write", "WRITE_SIZE", [(attn, 500.0), (copy, 262144.0), ("other", 7.0)])
    out = tmp_path / "traffic.json"
    bench.summarize_traffic(str(tmp_path / "fetch"), str(tmp_path / "write"), 256, "long50k_k32", str(out),
                            "segment_rope")
    t = json.load(open(out))
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["fetch_bytes_per_launch"] == 2000 * 1024 * 2
    assert t["write_bytes_per_launch"] == 500 * 1024
    assert t["hbm_bytes_per_launch"] == 2000 * 1024 * 2 + 500 * 1024
    assert t["key_layout"] == "segment_rope" and t["kernel_source_sha256_16"] == bench.kernel_hash()


def test_traffic_applies_only_to_its_kernel_source_workload_and_key_form(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    base = {"workload": "long50k_k32", "key_layout": "position_free", "kernel_source_sha256_16": bench.kernel_hash(),
            "hbm_bytes_per_launch": 123}
    f.write_text(json.dumps(base))
    assert bench.traffic_from_profiles("long50k_k32") == 123
    assert bench.traffic_from_profiles("batched_k16") is None
    assert bench.traffic_from_profiles("long50k_k32", "segment_rope") is None
    f.write_text(json.dumps(dict(base, kernel_source_sha256_16="0" * 16)))
    assert bench.traffic_from_profiles("long50k_k32") is None



def test_percentiles_of_step_times():
    p = bench.percentiles([float(x) for x in range(1, 12)])
    assert p == {"p10": 2.0, "p50": 6.0, "p90": 10.0}
