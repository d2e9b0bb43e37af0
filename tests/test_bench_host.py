"""Host-side logic of bench.py (no GPU): the one-GPU guard, the counter
summary's source check and the oracle baseline's report."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                      # no JSON line for a run that did not happen


def test_traffic_is_reported_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    import bench
    f = tmp_path / "traffic.json"
    summary = {"workload": "c4_bf16", "kernel_source_hash": bench.kernel_source_hash(),
               "hbm_bytes_per_launch": 1.5e9}
    f.write_text(json.dumps(summary))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("c4_bf16") == 1.5e9
    assert bench.measured_traffic("c3_bf16") is None          # another workload
    summary["kernel_source_hash"] = "0" * 16                   # counters taken on other sources
    f.write_text(json.dumps(summary))
    assert bench.measured_traffic("c4_bf16") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("c4_bf16") is None


def test_committed_traffic_summary_matches_the_current_sources():
    import bench
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    assert t["kernel_source_hash"] == bench.kernel_source_hash(), \
        "profiles/fa_fwd_c4_bf16_traffic.json was taken on other kernel sources: re-take FETCH_SIZE/WRITE_SIZE"
    assert t["hbm_bytes_per_launch"] == t["hbm_fetch_bytes_per_launch"] + t["hbm_write_bytes_per_launch"]


def test_cpu_baseline_reports_the_oracle_on_a_bounded_sample():
    import bench
    from tiled_attention_13_amd.inputs import Workload, make_inputs
    w = Workload("tiny", 1, 2, 512, 32, "bf16", True, 3)
    q, k, v = make_inputs(w)
    r = bench.cpu_baseline(w, q, k, v, budget_s=0.5)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert "query rows" in r["sample"]
    assert np.isfinite(r["seconds"])
