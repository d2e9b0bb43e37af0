"""Host-side logic of bench.py (no GPU): the one-GPU guard, the counter
summary's source check, the counter derivation and the oracle baseline's report."""
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


def test_committed_counters_are_used_only_for_the_source_they_were_taken_on(tmp_path, monkeypatch):
    import bench
    f = tmp_path / "counters.json"
    summary = {"workload": "c4_bf16", "kernel_source_hash": bench.kernel_source_hash(),
               "hbm_bytes_per_launch": 1.5e9, "mfma_busy": 0.5}
    f.write_text(json.dumps(summary))
    monkeypatch.setattr(bench, "counter_file", lambda w: str(f))
    assert bench.committed_counters("c4_bf16")["hbm_bytes_per_launch"] == 1.5e9
    assert bench.committed_counters("c3_bf16") is None         # a summary of another workload
    summary["kernel_source_hash"] = "0" * 16                   # counters taken on other sources
    f.write_text(json.dumps(summary))
    assert bench.committed_counters("c4_bf16") is None
    monkeypatch.setattr(bench, "counter_file", lambda w: str(tmp_path / "missing.json"))
    assert bench.committed_counters("c4_bf16") is None


def _row(dispatch, kernel, counter, value, t0=1000, t1=3000):
    return {"Dispatch_Id": str(dispatch), "Kernel_Name": kernel, "Counter_Name": counter,
            "Counter_Value": str(value), "Start_Timestamp": str(t0), "End_Timestamp": str(t1)}


def test_counter_figures_from_rocprof_rows():
    """Derivation of MFMA busy, conflict share, clock and calibrated HBM bytes from pass rows."""
    import bench
    k = "void fa::(anonymous namespace)::fwd_pp_kernel<128, true, false, 0, false>(KParams)"
    cp = "__amd_rocclr_copyBuffer"
    gui = 8 * 4000                                    # 4000 cycles per XCD in 2000 ns: 2 GHz
    core = []
    for dsp in (1, 2):
        core += [_row(dsp, k, "GRBM_GUI_ACTIVE", gui), _row(dsp, k, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1024 * 4000),
                 _row(dsp, k, "SQ_LDS_BANK_CONFLICT", 10), _row(dsp, k, "SQ_LDS_IDX_ACTIVE", 1000)]
    gib_kib = (1 << 30) / 1024
    fetch = [_row(1, k, "FETCH_SIZE", 1000.0), _row(2, k, "FETCH_SIZE", 3000.0), _row(3, cp, "FETCH_SIZE", gib_kib / 2)]
    write = [_row(1, k, "WRITE_SIZE", 100.0), _row(2, k, "WRITE_SIZE", 100.0), _row(3, cp, "WRITE_SIZE", gib_kib)]
    r = bench.derive_counters({"core": core, "fetch": fetch, "write": write}, "fwd_pp_kernel<128, true, false, 0")
    assert r["mfma_busy"] == 0.5 and r["lds_bank_conflict_share"] == 0.01
    assert r["gui_cycles_per_launch"] == 4000 and r["kernel_ms_under_profiler"] == 0.002 and r["launches"] == 2
    assert r["calibration"]["fetch_factor"] == 2.0 and r["calibration"]["write_factor"] == 1.0
    assert r["hbm_fetch_bytes_per_launch"] == 2000 * 1024 * 2 and r["hbm_write_bytes_per_launch"] == 100 * 1024
    assert r["hbm_bytes_per_launch"] == r["hbm_fetch_bytes_per_launch"] + r["hbm_write_bytes_per_launch"]


def test_committed_counter_summaries_match_the_current_sources():
    import glob
    import bench
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "fa_fwd_*_counters.json")))
    assert bench.counter_file("c4_bf16") in files               # the headline's is always there
    for path in files:
        with open(path) as fh:
            t = json.load(fh)
        assert path == bench.counter_file(t["workload"])
        assert t["kernel_source_hash"] == bench.kernel_source_hash(), \
            f"{os.path.basename(path)} was taken on other kernel sources: re-take it (bench.py --write-profile)"
        assert t["hbm_bytes_per_launch"] == t["hbm_fetch_bytes_per_launch"] + t["hbm_write_bytes_per_launch"]
        assert 0.0 < t["mfma_busy"] < 1.0 and 0.0 <= t["lds_bank_conflict_share"] < 1.0


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
