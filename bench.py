"""Benchmark of the fused attention forward on one MI355X.

One step = one ``fa_fwd`` call over the whole long-sequence workload
(bf16, causal, B=1, H=32, N=16384, d=128; inputs resident in HBM before the
timed region).  Prints ONE JSON line with attention TFLOP/s (4*B*H*N^2*d,
halved for causal), ms per call, the roofline entry of the attention kernel
and the float64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4_bf16]
                    [--no-cpu-baseline] [--no-bwd] [--no-configs] [--headline-only]
                    [--calib-copy-mib M]

The line also carries a ``splitkv`` object: ``fa_fwd`` against
``fa_fwd_splitkv`` (keys split into ranges run as separate workgroups, then
merged by lse) on the workload's per-device share at eight devices (H/8
heads), where one query tile per workgroup no longer fills the device.
A ``blocksparse`` object times ``fa_fwd_blocksparse`` on the same workload
with a sliding-window (16 blocks) plus global (2 blocks) table of 64x64
blocks, TFLOP/s counted over the (query, key) pairs the table and the causal
mask leave visible.
A ``configs`` object times every other forward workload (fp32 128 x 64,
the two d=32 shapes, bf16 4x32x4096x128 causal): median / p10 / p90 ms warm
(back to back) and, for working sets under the 256 MB MALL, cold (a 512 MiB
write before each call, outside the events) with HBM GB/s of the compulsory
bytes; the d=32 shapes also carry a VALU estimate, their binding roof.
It also carries a ``backward`` object: ``fa_bwd`` (dQ, dK, dV for a
seeded upstream gradient) timed the same way on the same bf16 workload,
with TFLOP/s by the usual convention (2.5 x the forward FLOPs) and the
matrix-core FLOPs the kernels actually execute (3.5 x at d = 128: the dK/dV
kernel and the dQ kernel each recompute S, and both compute dP).
A ``power`` object gives the socket power and graphics clock (amdsmi's GPU
metrics) while the headline calls run back to back for two more seconds,
untimed, after the timed region; ``--no-power`` skips it.

Hardware counters: before it touches the GPU, the script runs itself three
times under ``rocprofv3 --pmc`` (one counter pass each, two timed calls after
one warm-up, then a 1 GiB device copy of known traffic) and reports, for the
attention kernel, MFMA busy, the LDS bank-conflict share, the shader clock and
the HBM bytes read and written (FETCH_SIZE / WRITE_SIZE scaled by what the
same counters read for the copy).  ``--no-counters`` skips them;
``--counter-dir D`` keeps the raw rocprofv3 output; ``--write-profile F``
writes the counter summary with the hash of the kernel sources it was taken
on.  ``--calib-copy-mib`` runs, after the timed loop, a plain device copy of
M MiB (what the counter passes use).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import shutil
import subprocess
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS & % MFMA peak (bf16 causal N=16K d=128); ms/call"
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp8pv": 5000.0, "f32": 157.3}   # MI355X dense MFMA peaks
PEAK_HBM_GBPS = 8000.0
# the forward kernel's code: the HBM traffic summary is valid while these are unchanged
KERNEL_SOURCES = [os.path.join(ROOT, "tiled_attention_13_amd", "csrc", f)
                  for f in ("fa_fwd.hip", "fa_device.h", "fa_internal.h")]
def counter_file(workload: str) -> str:
    """The committed counter summary of a workload's attention kernel."""
    return os.path.join(ROOT, "profiles", f"fa_fwd_{workload}_counters.json")
# rocprofv3 counter passes (each within one run's hardware limits: at most 8 SQ,
# 2 GRBM and 4 TCC counters; FETCH_SIZE takes 3 TCC counters, WRITE_SIZE 2)
COUNTER_PASSES = (
    ("core", ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE")),
    ("fetch", ("FETCH_SIZE",)),
    ("write", ("WRITE_SIZE",)),
)
CALIB_MIB = 1024
N_XCD, N_SIMD_TOTAL = 8, 1024


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_counters(workload: str):
    """The committed counter summary, if it was taken on this kernel source and workload."""
    try:
        with open(counter_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t


def _rocprofv3():
    for cand in (shutil.which("rocprofv3"), "/opt/rocm/bin/rocprofv3"):
        if cand and os.path.exists(cand):
            return cand
    return None


def _counter_rows(d: str):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _per_kernel(rows, counter: str, match: str):
    """Per-dispatch values of one counter for the kernels whose name contains `match`."""
    by = {}
    for r in rows:
        if r.get("Counter_Name") == counter and match in r.get("Kernel_Name", ""):
            by[r["Dispatch_Id"]] = (float(r["Counter_Value"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                                    r["Kernel_Name"])
    return [by[k] for k in sorted(by, key=int)]


def kernel_match(w) -> str:
    """Substring of the attention kernel's name in rocprofv3 output for a workload."""
    if w.dtype == "f32":
        return "fwd_f32_kernel"
    if w.d == 128:
        tf = lambda b: "true" if b else "false"
        return f"fwd_b128_kernel<{tf(w.causal)}, {tf(w.dtype != 'bf16')}, {tf(w.dtype == 'fp8pv')}>"
    if w.dtype == "bf16" and w.d == 32:
        return f"fwd_d32_kernel<{'true' if w.causal else 'false'}"
    return f"fwd_pp_kernel<{w.d}, {'true' if w.causal else 'false'}, {'true' if w.dtype != 'bf16' else 'false'}, 0"


def collect_counters(w, keep_dir=None, timeout_s: float = 150.0) -> dict:
    """Counter passes in child processes (rocprofv3 --pmc ... -- python3 bench.py --counter-child ...).

    Must run before this process touches the GPU.  Returns the derived figures
    for the attention kernel, or {"error": ...}."""
    rp = _rocprofv3()
    if rp is None:
        return {"error": "rocprofv3 not found"}
    base = keep_dir or tempfile.mkdtemp(prefix="fa_pmc_")
    child = [sys.executable, os.path.abspath(__file__), "--counter-child", "--workload", w.name,
             "--steps", "2", "--warmup", "1", "--calib-copy-mib", str(CALIB_MIB)]
    rows, cmds = {}, []
    try:
        for name, ctrs in COUNTER_PASSES:
            d = os.path.join(base, f"pmc_{name}")
            cmd = [rp, "--pmc", *ctrs, "--output-format", "csv", "-d", d, "-o", "p", "--", *child]
            cmds.append(" ".join(["rocprofv3", "--pmc", *ctrs, "--output-format", "csv", "-d", f"<dir>/pmc_{name}",
                                  "-o", "p", "--", "python3", "bench.py", *child[2:]]))
            print(f"[bench] counter pass {name}: {' '.join(ctrs)}", file=sys.stderr, flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout_s, cwd=ROOT)
            rows[name] = _counter_rows(d)
            if not rows[name]:
                return {"error": f"pass {name}: rocprofv3 exited {r.returncode} with no counter rows; "
                                 f"stderr tail: {r.stderr[-400:]}"}
    except subprocess.TimeoutExpired:
        return {"error": f"a counter pass exceeded {timeout_s} s"}
    finally:
        if keep_dir is None:
            shutil.rmtree(base, ignore_errors=True)
    return {**derive_counters(rows, kernel_match(w)), "commands": cmds}


def derive_counters(rows: dict, m: str) -> dict:
    """Figures for the kernels whose name contains `m` from the rows of the three passes."""
    get = lambda p, c, k=m: _per_kernel(rows[p], c, k)
    gui, mfma = get("core", "GRBM_GUI_ACTIVE"), get("core", "SQ_VALU_MFMA_BUSY_CYCLES")
    bank, lds = get("core", "SQ_LDS_BANK_CONFLICT"), get("core", "SQ_LDS_IDX_ACTIVE")
    fetch, write = get("fetch", "FETCH_SIZE"), get("write", "WRITE_SIZE")
    cf, cw = get("fetch", "FETCH_SIZE", "copyBuffer"), get("write", "WRITE_SIZE", "copyBuffer")
    if not (gui and mfma and bank and lds and fetch and write and cf and cw):
        return {"error": f"counter rows missing for '{m}' or the calibration copy"}
    mean = lambda xs: sum(x[0] for x in xs) / len(xs)
    cycles = mean(gui) / N_XCD                                 # GRBM_GUI_ACTIVE sums the eight XCDs
    dur_ns = sum(x[2] - x[1] for x in gui) / len(gui)
    calib_bytes = CALIB_MIB << 20                              # the copy reads and writes this much
    f_factor = calib_bytes / 1024.0 / cf[-1][0]
    w_factor = calib_bytes / 1024.0 / cw[-1][0]
    fetch_b = mean(fetch) * 1024.0 * f_factor
    write_b = mean(write) * 1024.0 * w_factor
    return {
        "kernel": gui[0][3], "launches": len(gui), "kernel_source_hash": kernel_source_hash(),
        "mfma_busy": round(mean(mfma) / (N_SIMD_TOTAL * cycles), 4),
        "lds_bank_conflict_share": round(mean(bank) / max(mean(lds), 1.0), 4),
        "gui_cycles_per_launch": round(cycles),
        "kernel_ms_under_profiler": round(dur_ns / 1e6, 4),
        "hbm_fetch_bytes_per_launch": round(fetch_b), "hbm_write_bytes_per_launch": round(write_b),
        "hbm_bytes_per_launch": round(fetch_b) + round(write_b),
        "calibration": {"kernel": cf[-1][3], "bytes_read_and_written": calib_bytes,
                        "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4)},
        "definitions": "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE/8); "
                       "LDS bank-conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; "
                       "HBM bytes = FETCH_SIZE, WRITE_SIZE (KiB) x the factor that maps the 1 GiB copy's reading "
                       "to 1 GiB; means over the launches of each pass",
    }


def cpu_baseline(w, q, k, v, budget_s: float):
    """Time the oracle, as it stands, on rows spread evenly over the workload until ~budget_s."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing or no BLAS info
        threads = 1
    rows_per_chunk = 256
    stride = max(1, w.N // 4096)
    t0 = time.perf_counter()
    done = 0
    heads = 0
    for h in range(w.B * w.H):
        b, hh = divmod(h, w.H)
        rows = np.arange(h % stride, w.N, stride)
        for s in range(0, len(rows), rows_per_chunk):
            oracle.attention(q[b:b + 1, hh:hh + 1], k[b:b + 1, hh:hh + 1], v[b:b + 1, hh:hh + 1],
                             w.causal, w.softmax_scale, rows=rows[s:s + rows_per_chunk])
            done += len(rows[s:s + rows_per_chunk])
            if time.perf_counter() - t0 >= budget_s:
                break
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = w.flops() * done / (w.B * w.H * w.N)      # same counting convention, pro rata per row
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "cores_note": "BLAS threads of the oracle's float64 products (the threads it used); "
                          f"the process may run on {len(os.sched_getaffinity(0))} cores",
            "kind": "oracle",
            "sample": f"{done} query rows (every {stride}th row of {heads} head(s), all {w.N} keys each, "
                      f"float64 numpy) in {dt:.1f} s; TFLOP/s counted like the GPU figure, pro rata per row",
            "seconds": round(dt, 2), "cpu_model": _cpu_model()}


def _time_calls(fn, steps: int, warmup: int = 3) -> np.ndarray:
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])


def _time_back_to_back(fn, steps: int, warmup: int = 3) -> float:
    """Mean ms per call of `steps` calls issued back to back between two events
    (for calls of tens of microseconds the per-call events of _time_calls add
    their own overhead to each call)."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def bench_splitkv(w, steps: int):
    """fa_fwd vs fa_fwd_splitkv on the per-device share at eight devices (H/8 heads)."""
    import torch
    from tiled_attention_13_amd import fwd, fwd_splitkv
    from tiled_attention_13_amd.inputs import make_inputs
    shape = (w.B, w.H // 8, w.N, w.d)
    q, k, v = (torch.from_numpy(a).to("cuda").to(torch.bfloat16) for a in make_inputs(w, shape=shape))
    flops = w.flops() / 8
    o = torch.empty_like(q)
    lse = torch.empty(shape[:3], dtype=torch.float32, device="cuda")
    base = float(_time_calls(lambda: fwd(q, k, v, causal=w.causal, out=o, lse=lse), steps).mean())
    res = {"shape": list(shape), "fa_fwd_ms": round(base, 4), "fa_fwd_tflops": round(flops / base / 1e9, 2),
           "splits": {}}
    best = None
    for n in (2, 4, 8):
        ms = float(_time_calls(lambda: fwd_splitkv(q, k, v, n, causal=w.causal, out=o, lse=lse), steps).mean())
        res["splits"][str(n)] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 2)}
        best = ms if best is None else min(best, ms)
    res["best_speedup"] = round(base / best, 3)
    return res


def blocksparse_pairs(mask: np.ndarray, N: int, causal: bool) -> int:
    """Visible (query, key) pairs of a 64x64 block table, by block arithmetic."""
    nb = mask.shape[0]
    sizes = np.minimum(64, N - 64 * np.arange(nb))
    full = np.outer(sizes, sizes)
    if causal:
        full = np.where(np.arange(nb)[:, None] > np.arange(nb)[None, :], full, 0)
        diag = sizes * (sizes + 1) // 2
        full = full + np.diag(diag)
    return int((full * (mask != 0)).sum())


def bench_blocksparse(w, tq, tk, tv, steps: int):
    import torch
    from tiled_attention_13_amd import fwd_blocksparse
    from tiled_attention_13_amd.inputs import band_global_block_mask
    nb = (w.N + 63) // 64
    mask = band_global_block_mask(nb)
    tm = torch.from_numpy(mask).to("cuda")
    o = torch.empty_like(tq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    ms = float(_time_calls(lambda: fwd_blocksparse(tq, tk, tv, tm, causal=w.causal, out=o, lse=lse), steps).mean())
    flops = 4.0 * w.d * w.B * w.H * blocksparse_pairs(mask, w.N, w.causal)
    kept = int(np.tril(mask).sum()) if w.causal else int(mask.sum())
    total = nb * (nb + 1) // 2 if w.causal else nb * nb
    return {"table": "sliding window 16 blocks + 2 global blocks (64x64)", "blocks_kept": kept,
            "blocks_total": total, "ms_per_call": round(ms, 4), "tflops_visible": round(flops / ms / 1e9, 2)}


def _stats(ms: np.ndarray) -> dict:
    return {"median": round(float(np.median(ms)), 5), "p10": round(float(np.percentile(ms, 10)), 5),
            "p90": round(float(np.percentile(ms, 90)), 5)}


def _time_cold(fn, steps: int, flush) -> np.ndarray:
    """Per-call times with the caches flushed before every call (outside the events)."""
    import torch
    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        flush(i)
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])


# VALU floor for the small-d shapes: per score one scale-and-subtract FMA, one
# v_exp_f32, one add to the running sum and half a bf16 pack (the row max is
# skipped while the reference holds), at 4 cycles per wave64 instruction on a
# 16-lane SIMD and 8 for v_exp_f32: the d = 32 kernel's counters give
# SQ_ACTIVE_INST_VALU / SQ_INSTS_VALU = 1.23 quad-cycles per instruction, one
# in four of them v_exp_f32, i.e. 1 quad-cycle per ordinary instruction and 2
# per exp (profiles/fa_fwd_c2_bf16_valu_counters.md); over 256 CUs x 4 SIMDs
# at 2.4 GHz.
VALU_CYCLES_PER_SCORE = (4 + 8 + 4 + 2) / 64.0
N_SIMD = 256 * 4
CLOCK_HZ = 2.4e9


def bench_configs(flush_mib: int = 512):
    """Every other forward workload once: warm (back to back) and, where the
    working set fits the 256 MB MALL, cold (a 512 MiB write before each call).
    HBM GB/s are compulsory bytes over the cold median."""
    import torch
    from tiled_attention_13_amd import fwd
    from tiled_attention_13_amd.inputs import WORKLOADS, make_inputs
    flush_buf = torch.empty(flush_mib << 20, dtype=torch.uint8, device="cuda")
    flush = lambda i: flush_buf.fill_(i & 0xFF)
    out = {}
    # c3 runs 100 calls after 20 warm-up calls: with fewer, the clock is still settling under load
    for name, steps, warm in (("c1_f32", 200, 5), ("c2_bf16", 200, 5), ("c2_bf16_causal", 200, 5), ("c3_bf16", 100, 20)):
        w = WORKLOADS[name]
        tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        q, k, v = (torch.from_numpy(a).to("cuda").to(tdt) for a in make_inputs(w))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
        call = lambda: fwd(q, k, v, causal=w.causal, dtype=w.dtype, out=o, lse=lse)
        warm = _time_calls(call, steps, warmup=warm)
        med = _time_back_to_back(call, steps, warmup=5)
        r = {"shape": list(w.shape), "dtype": w.dtype, "causal": w.causal,
             "warm_ms_back_to_back": round(med, 5), "warm_ms": _stats(warm),
             "tflops": round(w.flops() / med / 1e9, 3),
             "pct_mfma_peak": round(100.0 * w.flops() / med / 1e9 / PEAK_TFLOPS[w.dtype], 2),
             "compulsory_bytes": w.compulsory_bytes()}
        if w.compulsory_bytes() < (256 << 20):
            cold = _time_cold(call, min(steps, 50), flush)
            cmed = float(np.median(cold))
            r["cold_ms"] = _stats(cold)
            r["hbm_gbps_cold"] = round(w.compulsory_bytes() / cmed / 1e6, 1)
            r["pct_hbm_peak_cold"] = round(100.0 * w.compulsory_bytes() / cmed / 1e6 / PEAK_HBM_GBPS, 2)
        if w.d <= 64 and w.dtype == "bf16":
            # floors: vector ALU work, compulsory HBM bytes, matrix-core FLOPs; when the call
            # takes more than twice the largest, none of them binds (each workgroup's
            # sequential walk over its key tiles does)
            scores = w.B * w.H * float(w.N) ** 2 * (0.5 if w.causal else 1.0)
            floors = {"valu": scores * VALU_CYCLES_PER_SCORE / N_SIMD / CLOCK_HZ * 1e3,
                      "hbm": w.compulsory_bytes() / (PEAK_HBM_GBPS * 1e6),
                      "mfma": w.flops() / (PEAK_TFLOPS[w.dtype] * 1e9)}
            r["floors_ms"] = {k: round(x, 4) for k, x in floors.items()}
            r["valu_estimate_ms"] = r["floors_ms"]["valu"]
            top = max(floors, key=floors.get)
            r["bound"] = top if med <= 2.0 * floors[top] else "latency"
        elif w.dtype == "f32":
            r["bound"] = "launch latency"
        else:
            r["bound"] = "mfma"
        t = committed_counters(name)
        if t is not None:
            # the committed counter summary of this kernel source (profiles/fa_fwd_<workload>_counters.json)
            r["counters"] = {k: t[k] for k in ("mfma_busy", "lds_bank_conflict_share", "hbm_bytes_per_launch",
                                               "kernel_ms_under_profiler")}
            r["counters"]["hbm_gbps_under_profiler"] = round(t["hbm_bytes_per_launch"] /
                                                             t["kernel_ms_under_profiler"] / 1e6, 1)
        out[name] = r
        del q, k, v, o, lse
    del flush_buf
    return out


def bench_fp8(steps: int):
    """The FP8 workload (1x16x32768x128 causal) with Q/K on e4m3 (bf16 P*V) and with P*V on e4m3 too."""
    import torch
    from tiled_attention_13_amd import fwd
    from tiled_attention_13_amd.inputs import WORKLOADS, make_inputs
    w = WORKLOADS["c5_fp8"]
    q, k, v = (torch.from_numpy(a).to("cuda").to(torch.bfloat16) for a in make_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    res = {"shape": list(w.shape), "causal": w.causal}
    for dt in ("fp8", "fp8pv"):
        ms = float(_time_calls(lambda: fwd(q, k, v, causal=w.causal, dtype=dt, out=o, lse=lse), steps).mean())
        res[dt] = {"ms_per_call": round(ms, 4), "tflops": round(w.flops() / ms / 1e9, 2),
                   "pct_fp8_peak": round(100.0 * w.flops() / ms / 1e9 / PEAK_TFLOPS["fp8"], 2)}
    # the attention kernel alone on pre-quantised Q/K (the pre-pass timed on its own)
    from tiled_attention_13_amd import fwd_fp8, quant_fp8
    pre = _time_calls(lambda: (quant_fp8(q), quant_fp8(k)), steps)
    q8, qs = quant_fp8(q)
    k8, ks = quant_fp8(k)
    alone = _time_calls(lambda: fwd_fp8(q8, qs, k8, ks, v, causal=w.causal, out=o, lse=lse), steps)
    ms = float(alone.mean())
    # mixed ceiling: Q.K^T (half the FLOPs) at the fp8 peak, P.V at the bf16 peak
    mixed = 1.0 / (0.5 / PEAK_TFLOPS["fp8"] + 0.5 / PEAK_TFLOPS["bf16"])
    res["fp8"]["prepass_ms"] = round(float(pre.mean()), 4)
    from tiled_attention_13_amd import quant_v_pow2
    pre_pv = _time_calls(lambda: (quant_fp8(q), quant_fp8(k), quant_v_pow2(v)), steps)
    res["fp8pv"]["prepass_ms"] = round(float(pre_pv.mean()), 4)
    # vector-ALU estimate: the same per-score cost as the small-d floors (one FMA, one
    # exp, one add, half a bf16 pack; the FP8 softmax skips the row max while the
    # reference holds) over the causal half of the scores, at 2.4 GHz; in the
    # ping-pong each wave's softmax runs beside the other wave's MFMAs, so the call
    # is bound by the larger of the two
    scores = w.B * w.H * float(w.N) ** 2 * (0.5 if w.causal else 1.0)
    res["fp8"]["kernel_only"] = {"ms_per_call": round(ms, 4), "tflops": round(w.flops() / ms / 1e9, 2),
                                 "pct_fp8_peak": round(100.0 * w.flops() / ms / 1e9 / PEAK_TFLOPS["fp8"], 2),
                                 "pct_mixed_ceiling": round(100.0 * w.flops() / ms / 1e9 / mixed, 2),
                                 "mixed_ceiling_tflops": round(mixed, 1),
                                 "mixed_ceiling_ms": round(w.flops() / (mixed * 1e9), 4),
                                 "valu_estimate_ms": round(scores * VALU_CYCLES_PER_SCORE / N_SIMD / CLOCK_HZ * 1e3, 4)}
    t = committed_counters("c5_fp8")
    if t is not None:
        res["fp8"]["kernel_only"]["counters"] = {k: t[k] for k in ("mfma_busy", "lds_bank_conflict_share",
                                                                   "hbm_bytes_per_launch", "kernel_ms_under_profiler")}
    t = committed_counters("c5_fp8pv")
    if t is not None:
        res["fp8pv"]["counters"] = {k: t[k] for k in ("mfma_busy", "lds_bank_conflict_share",
                                                      "hbm_bytes_per_launch", "kernel_ms_under_profiler")}
    res["note"] = ("fp8: Q.K^T on e4m3, P.V on bf16; fp8pv: both on e4m3; ms_per_call includes the "
                   "quantisation pre-passes (prepass_ms: those pre-passes alone, Q and K; fp8pv also V), "
                   "kernel_only is fa_fwd_fp8 on pre-quantised Q/K")
    return res


def sample_power(call, seconds: float = 2.0, settle_s: float = 0.8):
    """Socket power and graphics clock while `call` runs back to back (untimed).

    Read from amdsmi's GPU metrics table, which the driver refreshes only every
    few hundred milliseconds: samples from the first `settle_s` seconds of load
    are dropped, the rest summarised by their median.  Returns {"error": ...}
    where the library or the metrics are not available."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception as e:                                  # noqa: BLE001 - any failure is reported
        return {"error": f"amdsmi: {e!r}"}
    try:
        hs = amdsmi.amdsmi_get_processor_handles()
        if len(hs) != 1:
            return {"error": f"{len(hs)} devices: the reading could not be tied to the timed one"}
        h = hs[0]
        limit = amdsmi.amdsmi_get_power_info(h).get("power_limit")
        clk = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
        samples, stop = [], threading.Event()

        def sampler():
            while not stop.is_set():
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                samples.append((time.perf_counter(), m.get("current_socket_power"), m.get("current_gfxclk")))
                time.sleep(0.005)

        th = threading.Thread(target=sampler, daemon=True)
        t0 = time.perf_counter()
        th.start()
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                call()
            torch.cuda.synchronize()
        stop.set()
        th.join()
        keep = [(pw, ck) for t, pw, ck in samples if t - t0 >= settle_s
                and isinstance(pw, (int, float)) and isinstance(ck, (int, float))]
        if not keep:
            return {"error": "no metrics samples after the settling time"}
        return {"socket_power_w": float(np.median([x[0] for x in keep])),
                "gfxclk_mhz": float(np.median([x[1] for x in keep])),
                "power_limit_w": round(limit / 1e6, 1) if isinstance(limit, (int, float)) else None,
                "max_gfxclk_mhz": clk.get("max_clk"),
                "samples": len(keep), "seconds_under_load": seconds,
                "source": "amdsmi_get_gpu_metrics_info (current_socket_power, current_gfxclk), "
                          "untimed calls after the timed region"}
    except Exception as e:                                  # noqa: BLE001
        return {"error": f"amdsmi: {e!r}"}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:                                   # noqa: BLE001
            pass


def bench_backward(w, tq, tk, tv, o, lse, steps: int, warmup: int):
    """Time fa_bwd on the resident forward inputs, output and lse (one call = one step)."""
    import torch
    from tiled_attention_13_amd import bwd
    from tiled_attention_13_amd.inputs import make_grad
    g = torch.from_numpy(make_grad(w)).to("cuda").to(torch.bfloat16)
    gq, gk, gv = (torch.empty_like(tq) for _ in range(3))
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        bwd(tq, tk, tv, o, g, lse, causal=w.causal, dq=gq, dk=gk, dv=gv)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        bwd(tq, tk, tv, o, g, lse, causal=w.causal, dq=gq, dk=gk, dv=gv)
        ends[i].record(stream)
    torch.cuda.synchronize()
    per_call = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    ms = float(per_call.mean())
    conv = 2.5 * w.flops()
    executed = 3.5 * w.flops()     # d = 128: S twice (dK/dV, dQ kernels), dP twice, dV, dK, dQ once
    return {"ms_per_call": round(ms, 4), "median_ms": round(float(np.median(per_call)), 4),
            "tflops": round(conv / (ms * 1e-3) / 1e12, 2),
            "flop_convention": "2.5 x forward FLOPs (dV, dP, dQ, dK plus the recomputed S)",
            "mfma_tflops_executed": round(executed / (ms * 1e-3) / 1e12, 2),
            "pct_mfma_peak": round(100.0 * executed / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 2),
            "kernels": "bwd_prep_kernel, bwd_kvf_kernel (dK and dV, S once, 64-query slots), bwd_dq_pp_kernel "
                       "(64-key slots); no transposition pre-pass at d = 128"}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 calls (~0.4 s of the headline) after 20 warm-up calls: long enough for the clock to settle
    # under load, so the figure is the steady state rather than the ramp after idle
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c4_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0)
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload object (fp32, the two small-d shapes, the B=4 N=4096 shape)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline fa_fwd (no split-KV, block-sparse or backward objects)")
    ap.add_argument("--no-counters", action="store_true", help="skip the rocprofv3 counter passes")
    ap.add_argument("--no-power", action="store_true", help="skip the power and clock reading")
    ap.add_argument("--counter-dir", default=None, help="keep the counter passes' raw output here")
    ap.add_argument("--write-profile", default=None, help="write the counter summary (JSON) to this file")
    ap.add_argument("--counter-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}); "
              "heads shard independently across GPUs, so per-GPU throughput is the single-GPU figure.",
              file=sys.stderr)
        sys.exit(2)

    from tiled_attention_13_amd.inputs import WORKLOADS, digest, make_inputs
    w = WORKLOADS[args.workload]
    if args.counter_child:           # one counter pass: the calls and the calibration copy only
        args.headline_only, args.no_cpu_baseline, args.no_counters = True, True, True
    counters = None
    if not args.no_counters:
        # child processes first: this process has not touched the GPU yet
        counters = collect_counters(w, keep_dir=args.counter_dir)
        if args.write_profile and "error" not in counters:
            with open(args.write_profile, "w") as fh:
                json.dump({"workload": w.name, **counters}, fh, indent=1)

    import torch
    from tiled_attention_13_amd import fwd, load

    load()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    t_gen = time.perf_counter()
    q, k, v = make_inputs(w)
    gen_s = time.perf_counter() - t_gen
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    dq, dk, dv = (torch.from_numpy(a).to("cuda").to(tdt) for a in (q, k, v))
    out = torch.empty_like(dq)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        fwd(dq, dk, dv, causal=w.causal, dtype=w.dtype, out=out, lse=lse)
    torch.cuda.synchronize()

    # timed region: K calls back to back; per-call events on the launch stream
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for i in range(args.steps):
        starts[i].record(stream)
        fwd(dq, dk, dv, causal=w.causal, dtype=w.dtype, out=out, lse=lse)
        ends[i].record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    total_ms = t_all0.elapsed_time(t_all1)
    per_call = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    ms_per_step = total_ms / args.steps

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.counter_child:
        return
    # power and clock under the same calls, after the timed region: the headline
    # runs at the part's power limit, well below its peak clock
    power = None if args.no_power else sample_power(
        lambda: fwd(dq, dk, dv, causal=w.causal, dtype=w.dtype, out=out, lse=lse))
    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    kern_ms = float(per_call.mean())
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    if counters is None or "error" in counters:
        committed = committed_counters(w.name)
        if committed is not None:
            committed = {**committed, "source": "committed summary taken on these kernel sources"}
        counters = committed or counters
    traffic = counters.get("hbm_bytes_per_launch") if counters and "error" not in counters else None
    if traffic is not None:
        # counter cycles over the live kernel time: the clock the timed calls ran at (if it held)
        counters = {**counters, "shader_clock_ghz_est": round(counters["gui_cycles_per_launch"] / (kern_ms * 1e6), 3),
                    "hbm_gbps": round(traffic / (kern_ms * 1e-3) / 1e9, 1)}
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "seed": w.seed, "inputs": w.note, "parallelism": "single GPU"},
        "pct_mfma_peak": round(100.0 * value / peak, 2),
        "ms_per_call": {"mean": round(kern_ms, 4), "p10": round(float(np.percentile(per_call, 10)), 4),
                        "median": round(float(np.median(per_call)), 4),
                        "p90": round(float(np.percentile(per_call, 90)), 4)},
        "hbm_gbps_compulsory": round(w.compulsory_bytes() / (kern_ms * 1e-3) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": f"{kernel_match(w)} (the only launch of a {w.dtype} fa_fwd call)"
                               if w.dtype in ("bf16", "f32") else f"{kernel_match(w)} (plus pre-passes)",
                     "kernel_ms": round(kern_ms, 4), "per_launch_flops": flops,
                     "algorithmic_bytes": w.compulsory_bytes()},
        "counters": counters,
        "power": power,
        "input_sha256": digest(q, k, v)[:16],
        "input_gen_s": round(gen_s, 2),
    }
    extras = not args.headline_only and w.dtype == "bf16"
    if extras and w.H % 8 == 0:
        result["splitkv"] = bench_splitkv(w, args.steps)
    if extras:
        result["blocksparse"] = bench_blocksparse(w, dq, dk, dv, args.steps)
    if extras:
        result["fp8"] = bench_fp8(args.steps)
    if extras and not args.no_configs:
        result["configs"] = bench_configs()
    if extras and not args.no_bwd:
        result["backward"] = bench_backward(w, dq, dk, dv, out, lse, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
