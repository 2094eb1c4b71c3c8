"""Throughput of the FA2-order attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ai2048]

One step is one fa_fwd call over one batch of the workload (inputs already in
HBM). Prints ONE JSON line with TFLOPS = 4*B*H*N^2*d / time (halved for causal),
the roofline position of the kernel, and the float64 CPU oracle timed on a
bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FA fwd TFLOPS (4·B·H·N²·d, causal halved) and % of bf16 MFMA peak, 1 GPU"
PEAK_TFLOPS = 2500.0        # MI355X dense bf16/fp16 MFMA, published
WARMUP_MIN_S = 0.3          # least back-to-back warmup before the timed steps (clock ramp)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 matrix peak, published
CSRC = os.path.join(ROOT, "io_aware_exact_fa2_amd", "csrc")
# Shapes with too few query tiles to fill the GPU, timed through fa_fwd and through
# fa_fwd_splitkv with this many key splits
SPLITKV = {"few16k": 4, "fewc16k": 3}


def kernel_hash() -> str:
    """Short hash of every HIP source file and of the build script that holds the compile
    options (identifies the kernel a profile was taken on)."""
    h = hashlib.sha256()
    paths = [os.path.join(CSRC, n) for n in sorted(os.listdir(CSRC))]
    paths.append(os.path.join(ROOT, "io_aware_exact_fa2_amd", "build.py"))
    for path in paths:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    rec = profile_record(workload)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def _launcher(w, leg="fwd"):
    """(fn, args) of one launch of the forward ("fwd") or backward ("bwd") pass on
    seeded inputs of workload w, resident on cuda:0."""
    import torch
    import io_aware_exact_fa2_amd as fa
    import workloads

    stream = torch.cuda.current_stream()
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    if leg == "fp8":
        q8, k8, v8, qs, ks, vs = workloads.make_fp8_inputs(w)
        q8, k8, v8 = (t.to("cuda:0") for t in (q8, k8, v8))
        o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device="cuda:0")
        return fa.fa_fwd_fp8, (q8, k8, v8, qs, ks, vs, o, lse, w.B, w.H, w.N, w.d, w.scale,
                               int(w.causal), stream)
    q, k, v = (t.to("cuda:0") for t in workloads.make_inputs(w))
    o = torch.empty_like(q)
    fn = fa.fa_fwd if w.dtype == "bf16" else fa.fa_fwd_fp16
    args = (q, k, v, o, lse, w.B, w.H, w.N, w.d, w.scale, int(w.causal), stream)
    if leg == "fwd":
        return fn, args
    dt = fa.FA_DTYPE_BF16 if w.dtype == "bf16" else fa.FA_DTYPE_FP16
    if leg == "fa1":
        nb = fa.fa_fwd_fa1_workspace_size(w.B, w.H, w.N, w.d)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
        return fa.fa_fwd_fa1, (q, k, v, o, lse, ws, nb, w.B, w.H, w.N, w.d, w.scale,
                               int(w.causal), dt, stream)
    if leg.startswith("splitkv"):
        ns = int(leg[len("splitkv"):] or 4)
        nb = fa.fa_fwd_splitkv_workspace_size(w.B, w.H, w.N, w.d, ns)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
        return fa.fa_fwd_splitkv, (q, k, v, o, lse, ws, nb, w.B, w.H, w.N, w.d, w.scale,
                                   int(w.causal), ns, dt, stream)
    st = fn(*args)
    if st != fa.FA_OK:
        raise fa.FAError(st)
    do = workloads.make_grad(w).to("cuda:0")
    grads = [torch.empty_like(q) for _ in range(3)]
    fn = fa.fa_bwd if w.dtype == "bf16" else fa.fa_bwd_fp16
    return fn, (q, k, v, o, lse, do, *grads, w.B, w.H, w.N, w.d, w.scale, int(w.causal),
                stream)


def time_gpu(w, steps, warmup, leg="fwd"):
    import torch
    import io_aware_exact_fa2_amd as fa

    fn, args = _launcher(w, leg)
    stream = args[-1]
    for _ in range(warmup):
        st = fn(*args)
        if st != fa.FA_OK:
            raise fa.FAError(st)
    torch.cuda.synchronize()
    # The GPU raises its clock over the first few tens of milliseconds of sustained load:
    # keep launching until WARMUP_MIN_S of back-to-back work has run, so the timed steps
    # see the steady state (the number of warmup steps actually run is reported).
    ran = warmup
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < WARMUP_MIN_S:
        for _ in range(10):
            fn(*args)
        ran += 10
        torch.cuda.synchronize()
    # events on the stream the kernel is launched on
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn(*args)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    return ms, wall, ran


def time_cold(w, steps, scrub_mib=512):
    """Median kernel time with a scrub write of scrub_mib MiB before every launch, so Q, K
    and V come from HBM rather than the L2 / MALL (events bracket the launch only)."""
    import torch
    import io_aware_exact_fa2_amd as fa
    import workloads

    q, k, v = (t.to("cuda:0") for t in workloads.make_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda:0")
    scrub = torch.empty(scrub_mib << 20, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()
    fn = fa.fa_fwd if w.dtype == "bf16" else fa.fa_fwd_fp16
    args = (q, k, v, o, lse, w.B, w.H, w.N, w.d, w.scale, int(w.causal), stream)
    times = []
    for _ in range(steps):
        scrub.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = fn(*args)
        e1.record(stream)
        if st != fa.FA_OK:
            raise fa.FAError(st)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    return times[len(times) // 2]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def calibrate_copy(mib: int):
    """A plain device copy of known size (float32 multiply by 1, out of place) whose
    FETCH_SIZE / WRITE_SIZE counters calibrate the attention kernel's traffic."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def _csv_rows(directory, suffix):
    import csv
    import glob

    rows = []
    for path in glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _counter_means(directory, counter):
    """Mean per-dispatch value of one counter, by kernel name."""
    acc = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def io_model(w, path):
    """Device-memory traffic of one launch by the HBM column of the FA1/FA2 comparison
    table (currybab.bearblog.dev, "정리": per head FA1 moves 2Nd + T_c Nd + 2 T_c Nd
    elements, FA2 Nd + 2 T_r Nd + Nd; N-sized statistics omitted), for this kernel's
    tile sizes and element sizes (16-bit tensors; the FA1 kernel keeps O_i, m_i, l_i in
    float32 and skips the read before the first key block)."""
    heads = w.B * w.H
    nd = w.N * w.d
    if path == "fa1":
        t_c = -(-w.N // 64)
        fetch = 2 * 2 * nd + 2 * t_c * nd + 4 * (t_c - 1) * nd + 8 * (t_c - 1) * w.N
        write = 4 * (t_c - 1) * nd + 2 * nd + 8 * (t_c - 1) * w.N + 4 * w.N
        elems = 2 * nd + 3 * t_c * nd
        blocks = {"T_c": t_c}
    else:
        t_r = -(-w.N // 256)
        fetch = 2 * nd + 2 * 2 * t_r * nd
        write = 2 * nd + 4 * w.N
        elems = 2 * nd + 2 * t_r * nd
        blocks = {"T_r": t_r}
    return {"table_elements_per_launch": heads * elems, **blocks,
            "model_fetch_bytes": heads * fetch, "model_write_bytes": heads * write,
            "note": "non-causal; the table assumes every re-read reaches device memory"}


def summarize_hbm(workload, fetch_dir, write_dir, copy_mib, out_path, commands, path="fwd"):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) into
    HBM bytes per launch of the attention kernel, each counter scaled by what it reads
    for the plain copy of copy_mib MiB in the same run."""
    import workloads

    w = workloads.get(workload)
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")
    if path == "fa1":
        fa_name = next(k for k in fetch if "fa_fwd_fa1" in k)
    else:  # the 16-bit forward kernel of this workload (wide, 32-query or generic)
        fa_name = next(k for k in fetch if "fa_fwd" in k and "fa1" not in k and "fp8" not in k)
    copy_name = next(k for k in fetch if "MulFunctor" in k)
    copy_kib = copy_mib * 1024.0
    f_scale = copy_kib / fetch[copy_name]
    w_scale = copy_kib / write[copy_name]
    fa_bytes = (fetch[fa_name] * f_scale + write[fa_name] * w_scale) * 1024.0
    rec = {
        "workload": w.name, "kernel": fa_name,
        "kernel_source_sha256_16": kernel_hash(),
        "fetch_kib_per_dispatch": fetch[fa_name], "write_kib_per_dispatch": write[fa_name],
        "copy_mib": copy_mib, "copy_kernel": copy_name,
        "copy_fetch_kib": fetch[copy_name], "copy_write_kib": write[copy_name],
        "fetch_scale": f_scale, "write_scale": w_scale,
        "hbm_bytes_per_launch": fa_bytes,
        "algorithmic_bytes_per_launch": w.min_bytes(),
        "traffic_over_algorithmic": fa_bytes / w.min_bytes(),
        "fetch_bytes_per_launch": fetch[fa_name] * f_scale * 1024.0,
        "write_bytes_per_launch": write[fa_name] * w_scale * 1024.0,
        "io_model": io_model(w, path),
        "commands": commands,
    }
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


SQ_PASS1 = ("GRBM_GUI_ACTIVE SQ_WAVES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA "
            "SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE")
SQ_PASS2 = ("SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU "
            "SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_SALU")
N_XCD, N_SIMD = 8, 1024      # MI355X: 8 XCDs, 256 CUs x 4 SIMDs
MFMA_FLOPS = 32768           # one v_mfma_f32_32x32x16 (16-bit inputs): 2*32*32*16


def _is_kernel(name, path):
    if path == "fa1":
        return "fa_fwd_fa1" in name
    if path == "bwd":
        return "fa_bwd" in name
    return "fa_fwd" in name and "fa1" not in name and "fp8" not in name


def _is_split(name):
    """The kernels of the split-KV pass: a forward kernel's split instantiation (its
    SPLIT template argument: the 7th of the 32-query kernel, the 6th of the wide kernel)
    and the merge."""
    if "fa_split_merge" in name:
        return True
    m = re.search(r"fa_fwd_(fast|wide)_kernel<([^>]*)>", name)
    if m is None:
        return False
    args = [a.strip() for a in m.group(2).split(",")]
    pos = 6 if m.group(1) == "fast" else 5
    return len(args) > pos and args[pos] == "true"


def _kernel_stats(directory, path):
    """(name, calls, average ns, min ns, max ns) of the kernel, from --stats output."""
    rows = _csv_rows(directory, "kernel_stats.csv")
    for r in rows:
        if _is_kernel(r["Name"], path):
            return (r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                    float(r["MaxNs"]))
    raise SystemExit(f"no {path} kernel in the kernel stats under {directory}")


def _all_counters(directory, path):
    """Mean per-dispatch value of every counter of a --pmc run, for the kernel."""
    acc = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if _is_kernel(r["Kernel_Name"], path):
            acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in sorted(acc.items())}


def summarize_profile(workload, dirs, copy_mib, path="fwd", cmd_args="", out_dir=None):
    """Write profiles/<stem>_<workload>_rocprof.md and _hbm_counters.json from five
    rocprofv3 runs of the same bench.py command: --kernel-trace --stats, two --pmc
    passes of SQ counters (SQ_PASS1, SQ_PASS2), FETCH_SIZE and WRITE_SIZE."""
    import workloads

    kt_dir, sq1_dir, sq2_dir, fetch_dir, write_dir = dirs
    w = workloads.get(workload)
    stem = "fa_fwd" if path == "fwd" else f"fa_{path}"
    name, calls, avg, mn, mx = _kernel_stats(kt_dir, path)
    c1 = _all_counters(sq1_dir, path)
    c2 = _all_counters(sq2_dir, path)
    bench_cmd = f"python -u bench.py --workload {w.name}{cmd_args}"
    cmds = {
        "kernel_trace": f"rocprofv3 --kernel-trace --stats -f csv -d <kt_dir> -o kt -- {bench_cmd}",
        "sq_pass1": f"rocprofv3 --pmc {SQ_PASS1} -f csv -d <sq1_dir> -o p -- {bench_cmd}",
        "sq_pass2": f"rocprofv3 --pmc {SQ_PASS2} -f csv -d <sq2_dir> -o p -- {bench_cmd}",
        "fetch": f"rocprofv3 --pmc FETCH_SIZE -f csv -d <fetch_dir> -o p -- {bench_cmd} "
                 f"--calibrate-copy-mib {copy_mib}",
        "write": f"rocprofv3 --pmc WRITE_SIZE -f csv -d <write_dir> -o p -- {bench_cmd} "
                 f"--calibrate-copy-mib {copy_mib}",
        "summary": f"python bench.py --workload {w.name} --path {path} --summarize-profile "
                   f"<kt_dir> <sq1_dir> <sq2_dir> <fetch_dir> <write_dir> "
                   f"--calibrate-copy-mib {copy_mib}",
    }
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    out_json = os.path.join(out_dir, f"{stem}_{w.name}_hbm_counters.json")
    hbm = summarize_hbm(w.name, fetch_dir, write_dir, copy_mib, out_json,
                        " ; ".join(cmds[k] for k in ("fetch", "write", "summary")), path)
    work = (2.5 if path == "bwd" else 1.0) * w.flops()
    secs = avg * 1e-9
    tflops = work / secs / 1e12
    clock = c1["GRBM_GUI_ACTIVE"] / N_XCD / secs
    active = c1["GRBM_GUI_ACTIVE"] / N_XCD
    mfma_per_simd = c1["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD
    sq = {
        "clock_GHz_under_load": clock / 1e9,
        "mfma_busy_pct": 100 * mfma_per_simd / active,
        "cycles_per_mfma": c1["SQ_VALU_MFMA_BUSY_CYCLES"] / c1["SQ_INSTS_MFMA"],
        "mfma_insts": c1["SQ_INSTS_MFMA"],
        "mfma_insts_expected": work / MFMA_FLOPS,
        "valu_insts_per_mfma": c1["SQ_INSTS_VALU"] / c1["SQ_INSTS_MFMA"],
        "lds_bank_conflict_cycles": c1["SQ_LDS_BANK_CONFLICT"],
        "lds_bank_conflict_pct_of_lds_active": 100 * c1["SQ_LDS_BANK_CONFLICT"]
        / max(c1["SQ_LDS_IDX_ACTIVE"], 1.0),
        "issue_pct_of_wave_cycles": 100 * c2["SQ_ACTIVE_INST_ANY"] / c2["SQ_WAVE_CYCLES"],
        "valu_issue_pct_of_wave_cycles": 100 * c2["SQ_ACTIVE_INST_VALU"] / c2["SQ_WAVE_CYCLES"],
        "waitcnt_pct_of_wave_cycles": 100 * c2["SQ_WAIT_ANY"] / c2["SQ_WAVE_CYCLES"],
        "wait_issue_pct_of_wave_cycles": 100 * c2["SQ_WAIT_INST_ANY"] / c2["SQ_WAVE_CYCLES"],
        "mfma_valu_coexec_pct_of_mfma_busy": 100 * c2["SQ_VALU_MFMA_COEXEC_CYCLES"]
        / c1["SQ_VALU_MFMA_BUSY_CYCLES"],
    }
    hbm.update({"kernel_trace": {"calls": calls, "average_ns": avg, "min_ns": mn, "max_ns": mx,
                                 "tflops_at_average": tflops},
                "sq": sq, "sq_counters": {**c1, **c2}, "commands_all": cmds})
    with open(out_json, "w") as f:
        json.dump(hbm, f, indent=1)
    peak_clk = 256 * clock * 4096 / 1e12
    hbm_gbs = hbm["hbm_bytes_per_launch"] / secs / 1e9
    mask = "causal" if w.causal else "non-causal"
    lines = [
        f"# {stem} kernel, workload {w.name} — rocprofv3 summary", "",
        f"Workload: {w.name} = B={w.B}, H={w.H}, N={w.N}, d={w.d}, {w.dtype}, {mask}, "
        f"scale = 1/sqrt(d); seeded synthetic inputs from `workloads`.",
        f"Kernel: `{name}`.",
        f"Kernel source hash (bench.py `kernel_hash`): {hbm['kernel_source_sha256_16']}. "
        "All commands run from the repository root; output directories are placeholders; "
        "every figure below is computed from the five runs by the summary command.", "",
        "## Kernel trace (`--kernel-trace --stats`)", "", "    " + cmds["kernel_trace"], "",
        f"| calls | average ns | min ns | max ns | TFLOPS at average | % of 2500 TFLOPS |",
        "|---|---|---|---|---|---|",
        f"| {calls} | {avg:.0f} | {mn:.0f} | {mx:.0f} | {tflops:.1f} | {100 * tflops / 2500:.1f} |",
        "", f"FLOPs per launch: {work:.4e} ({'2.5 x ' if path == 'bwd' else ''}4·B·H·N²·d"
        f"{', halved for the causal mask' if w.causal else ''}).", "",
        "## SQ / GRBM counters (two `--pmc` passes, mean per dispatch)", "",
        "    " + cmds["sq_pass1"], "", "    " + cmds["sq_pass2"], "",
        "| counter | mean per dispatch |", "|---|---|",
    ]
    lines += [f"| {k} | {v:.6g} |" for k, v in sorted({**c1, **c2}.items())]
    lines += [
        "", f"Derived ({N_XCD} XCDs, {N_SIMD} SIMDs, the kernel-trace average duration):",
        f"* clock under load = GRBM_GUI_ACTIVE / {N_XCD} / kernel time = "
        f"{clock / 1e9:.3f} GHz; the 16-bit MFMA peak at that clock is 256 CUs x 4096 "
        f"flop/cycle = {peak_clk:.0f} TFLOPS, of which this launch reaches "
        f"{100 * tflops / peak_clk:.1f}%",
        f"* cycles per MFMA = SQ_VALU_MFMA_BUSY_CYCLES / SQ_INSTS_MFMA = {sq['cycles_per_mfma']:.1f}",
        f"* MFMA busy per SIMD = {mfma_per_simd:.0f} cycles = {sq['mfma_busy_pct']:.1f}% "
        "of the active cycles",
        f"* MFMA instructions: FLOPs / 32768 = {sq['mfma_insts_expected']:.4g} expected, "
        f"{sq['mfma_insts']:.4g} counted",
        f"* VALU instructions per MFMA = {sq['valu_insts_per_mfma']:.2f}",
        f"* LDS bank-conflict cycles = {sq['lds_bank_conflict_cycles']:.6g} "
        f"({sq['lds_bank_conflict_pct_of_lds_active']:.3f}% of SQ_LDS_IDX_ACTIVE)",
        f"* of the wave cycles: issuing {sq['issue_pct_of_wave_cycles']:.1f}% (VALU incl. MFMA "
        f"issue {sq['valu_issue_pct_of_wave_cycles']:.1f}%), waiting on a counter (s_waitcnt) "
        f"{sq['waitcnt_pct_of_wave_cycles']:.1f}%, waiting to issue "
        f"{sq['wait_issue_pct_of_wave_cycles']:.1f}%; MFMA and VALU co-execute "
        f"{sq['mfma_valu_coexec_pct_of_mfma_busy']:.1f}% of the MFMA-busy cycles", "",
        "## HBM traffic (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`)", "",
        "    " + cmds["fetch"], "", "    " + cmds["write"], "", "    " + cmds["summary"], "",
        f"Each counter is scaled by what it reads for a plain {copy_mib} MiB device copy "
        "(torch float32 multiply, out of place) in the same run:", "",
        f"| | kernel KiB/dispatch | copy KiB/dispatch ({copy_mib} MiB true) | scale |",
        "|---|---|---|---|",
        f"| FETCH_SIZE | {hbm['fetch_kib_per_dispatch']:.1f} | {hbm['copy_fetch_kib']:.1f} | "
        f"{hbm['fetch_scale']:.3f} |",
        f"| WRITE_SIZE | {hbm['write_kib_per_dispatch']:.1f} | {hbm['copy_write_kib']:.1f} | "
        f"{hbm['write_scale']:.3f} |", "",
        f"HBM bytes per launch = {hbm['hbm_bytes_per_launch'] / 1e6:.1f} MB; algorithmic "
        f"(Q, K, V read once, O written once, 4 B of L per row) = "
        f"{hbm['algorithmic_bytes_per_launch'] / 1e6:.1f} MB; ratio "
        f"{hbm['traffic_over_algorithmic']:.3f}. At the average kernel time that is "
        f"{hbm_gbs:.0f} GB/s of the 8000 GB/s HBM peak.", "",
    ]
    out_md = os.path.join(out_dir, f"{stem}_{w.name}_rocprof.md")
    with open(out_md, "w") as f:
        f.write("\n".join(lines))
    return hbm


def _all_kernel_stats(directory, pred):
    """(name, calls, average ns, min ns, max ns) of every kernel that pred accepts."""
    out = []
    for r in _csv_rows(directory, "kernel_stats.csv"):
        if pred(r["Name"]):
            out.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                        float(r["MaxNs"])))
    return sorted(out)


def _counters_by_kernel(directory, pred):
    acc = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if pred(r["Kernel_Name"]):
            acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in acc.items()}


def _shape(w, path="fwd"):
    mask = "causal" if w.causal else "non-causal"
    dt = "E4M3 Q, K, V with per-tensor scales, bf16 O" if path == "fp8" else w.dtype
    return f"B={w.B}, H={w.H}, N={w.N}, d={w.d}, {dt}, {mask}"


def summarize_traces(path, entries, sq_dirs=None, hbm_dirs=None, copy_mib=512,
                     cmd_args=" --steps 20 --warmup 3", out_dir=None):
    """profiles/fa_<path>_rocprof.md (and a JSON of its figures) from rocprofv3 runs of
    `bench.py --path <path>` (bwd: the three backward kernels; fp8: the 8-bit forward;
    fa1: the FA1-order forward): a --kernel-trace --stats directory per workload, for the
    backward also the two SQ --pmc passes of its first workload, for fa1 also the
    FETCH_SIZE / WRITE_SIZE runs."""
    import workloads

    out_dir = out_dir or os.path.join(ROOT, "profiles")
    pred = {"bwd": lambda n: "fa_bwd" in n, "fp8": lambda n: "fa_fwd_fp8" in n,
            "fa1": lambda n: "fa_fwd_fa1" in n,
            "splitkv": lambda n: _is_split(n) or _is_kernel(n, "fwd")}[path]
    factor = 2.5 if path == "bwd" else 1.0
    title = {"bwd": "fa_bwd backward kernels", "fp8": "fa_fwd_fp8 (E4M3 forward)",
             "fa1": "fa_fwd_fa1 (the FA1 loop order)",
             "splitkv": "fa_fwd_splitkv (keys split across workgroups) against fa_fwd"}[path]
    rec = {"path": path, "kernel_source_sha256_16": kernel_hash(), "workloads": {}}
    lines = [f"# {title} — rocprofv3 summary", "",
             f"Kernel source hash (bench.py `kernel_hash`): {rec['kernel_source_sha256_16']}. "
             "Seeded synthetic inputs from `workloads`; all commands run from the repository "
             "root, output directories are placeholders; every figure below is computed from "
             "the runs by the summary command.", "", "## Kernel trace (`--kernel-trace --stats`)",
             ""]
    for wl, kt_dir in entries:
        lines.append(f"    rocprofv3 --kernel-trace --stats -f csv -d <kt_dir_{wl}> -o kt -- "
                     f"python -u bench.py --workload {wl} --path {path}{cmd_args}")
    lines.append("")
    if path == "bwd":
        lines += ["Work convention: 2.5x the forward flops (five N x N x d products), halved "
                  "for causal; one backward is the three kernels once each.", "",
                  "| workload | shape | kernel | calls | average µs | min µs | max µs |",
                  "|---|---|---|---|---|---|---|"]
    else:
        lines += ["| workload | shape | kernel | calls | average µs | min µs | max µs | TFLOPS |",
                  "|---|---|---|---|---|---|---|---|"]
    summary = []
    for wl, kt_dir in entries:
        w = workloads.get(wl)
        ks = _all_kernel_stats(kt_dir, pred)
        if path == "splitkv":
            # the split pass is its partial kernel plus the merge; fa_fwd is one kernel
            total = sum(k[2] for k in ks if _is_split(k[0]))
            plain = sum(k[2] for k in ks if not _is_split(k[0]))
        else:
            total = sum(k[2] for k in ks)
        tf = factor * w.flops() / (total * 1e-9) / 1e12 if total else 0.0
        rec["workloads"][wl] = {"kernels": {k[0]: {"calls": k[1], "average_ns": k[2],
                                                   "min_ns": k[3], "max_ns": k[4]} for k in ks},
                                "sum_of_averages_ns": total, "tflops": tf}
        if path == "splitkv":
            rec["workloads"][wl].update({
                "splits": SPLITKV.get(wl, 4), "fa_fwd_ns": plain,
                "fa_fwd_tflops": w.flops() / (plain * 1e-9) / 1e12 if plain else 0.0,
                "speedup": plain / total if total else 0.0})
        for k in ks:
            row = f"| {wl} | {_shape(w, path)} | `{k[0]}` | {k[1]} | {k[2] / 1e3:.1f} | " \
                  f"{k[3] / 1e3:.1f} | {k[4] / 1e3:.1f} |"
            if "fa_split_merge" in k[0]:
                row += " (merge) |"
            elif path != "bwd":
                row += f" {w.flops() / (k[2] * 1e-9) / 1e12:.1f} |"
            lines.append(row)
        summary.append((wl, total, tf))
    lines.append("")
    if path == "bwd":
        lines += ["| workload | backward µs (sum of the averages) | TFLOPS (2.5x convention) | "
                  "% of 2500 |", "|---|---|---|---|"]
        lines += [f"| {wl} | {t / 1e3:.1f} | {tf:.1f} | {100 * tf / 2500:.1f} |"
                  for wl, t, tf in summary]
        lines.append("")
    elif path == "splitkv":
        lines += ["Split-KV time = the partial kernel's average + the merge kernel's average "
                  "(one call runs both); fa_fwd time = its one kernel's average, same shape.", "",
                  "| workload | splits | fa_fwd µs | TFLOPS | split-KV µs | TFLOPS | speedup |",
                  "|---|---|---|---|---|---|---|"]
        for wl, t, tf in summary:
            r = rec["workloads"][wl]
            lines.append(f"| {wl} | {r['splits']} | {r['fa_fwd_ns'] / 1e3:.1f} | "
                         f"{r['fa_fwd_tflops']:.1f} | {t / 1e3:.1f} | {tf:.1f} | "
                         f"{r['speedup']:.2f} |")
        lines.append("")
    elif path == "fp8":
        lines += ["Against the 5000 TFLOPS dense FP8 peak: " + ", ".join(
            f"{wl} {100 * tf / 5000:.1f}%" for wl, _, tf in summary) + ".", ""]
    if sq_dirs:
        wl0 = entries[0][0]
        c1 = _counters_by_kernel(sq_dirs[0], pred)
        c2 = _counters_by_kernel(sq_dirs[1], pred)
        lines += [f"## SQ counters, {wl0} (two `--pmc` passes, mean per dispatch of each kernel)",
                  "", f"    rocprofv3 --pmc {SQ_PASS1} -f csv -d <sq1_dir> -o p -- python -u "
                  f"bench.py --workload {wl0} --path {path}{cmd_args}",
                  "", f"    rocprofv3 --pmc {SQ_PASS2} -f csv -d <sq2_dir> -o p -- python -u "
                  f"bench.py --workload {wl0} --path {path}{cmd_args}", "",
                  "| kernel | VALU per MFMA | MFMA busy % of active cycles | clock GHz | issuing % "
                  "of wave cycles | s_waitcnt % | waiting to issue % | LDS bank-conflict cycles |",
                  "|---|---|---|---|---|---|---|---|"]
        kt = dict((k[0], k[2]) for k in _all_kernel_stats(entries[0][1], pred))
        rec["sq"] = {}
        for name in sorted(c1):
            a, b = c1[name], c2.get(name, {})
            if not a.get("SQ_INSTS_MFMA") or name not in kt:
                continue
            act = a["GRBM_GUI_ACTIVE"] / N_XCD
            sq = {"valu_insts_per_mfma": a["SQ_INSTS_VALU"] / a["SQ_INSTS_MFMA"],
                  "mfma_busy_pct": 100 * a["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / act,
                  "clock_GHz_under_load": act / (kt[name] * 1e-9) / 1e9,
                  "lds_bank_conflict_cycles": a["SQ_LDS_BANK_CONFLICT"]}
            if b.get("SQ_WAVE_CYCLES"):
                sq["issue_pct_of_wave_cycles"] = 100 * b["SQ_ACTIVE_INST_ANY"] / b["SQ_WAVE_CYCLES"]
                sq["waitcnt_pct_of_wave_cycles"] = 100 * b["SQ_WAIT_ANY"] / b["SQ_WAVE_CYCLES"]
                sq["wait_issue_pct_of_wave_cycles"] = 100 * b["SQ_WAIT_INST_ANY"] / b["SQ_WAVE_CYCLES"]
            rec["sq"][name] = {**sq, "counters": {**a, **b}}
            lines.append(f"| `{name}` | {sq['valu_insts_per_mfma']:.2f} | {sq['mfma_busy_pct']:.1f} | "
                         f"{sq['clock_GHz_under_load']:.3f} | {sq.get('issue_pct_of_wave_cycles', 0):.1f} | "
                         f"{sq.get('waitcnt_pct_of_wave_cycles', 0):.1f} | "
                         f"{sq.get('wait_issue_pct_of_wave_cycles', 0):.1f} | "
                         f"{sq['lds_bank_conflict_cycles']:.6g} |")
        lines += ["", "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8 "
                  "XCDs); the clock is GRBM_GUI_ACTIVE / 8 / the kernel's trace average; the "
                  "issue and wait shares divide by SQ_WAVE_CYCLES.", ""]
    if hbm_dirs:
        wl0 = entries[0][0]
        hrec = summarize_hbm(wl0, hbm_dirs[0], hbm_dirs[1], copy_mib,
                             os.path.join(out_dir, f"fa_{path}_{wl0}_hbm_counters.json"),
                             "see the summary", path)
        rec["hbm"] = {k: hrec[k] for k in ("hbm_bytes_per_launch", "fetch_bytes_per_launch",
                                           "write_bytes_per_launch", "fetch_scale",
                                           "write_scale")}
        m = hrec["io_model"]
        lines += ["## HBM traffic (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`)", "",
                  f"    rocprofv3 --pmc FETCH_SIZE -f csv -d <fetch_dir> -o p -- python -u bench.py "
                  f"--workload {wl0} --path {path}{cmd_args} --calibrate-copy-mib {copy_mib}", "",
                  f"    rocprofv3 --pmc WRITE_SIZE -f csv -d <write_dir> -o p -- python -u bench.py "
                  f"--workload {wl0} --path {path}{cmd_args} --calibrate-copy-mib {copy_mib}", "",
                  f"Counters scaled by a plain {copy_mib} MiB copy in the same run (FETCH_SIZE "
                  f"scale {hrec['fetch_scale']:.3f}, WRITE_SIZE scale {hrec['write_scale']:.3f}).", "",
                  "| | model (the pages' HBM column, this kernel's element sizes) | measured |",
                  "|---|---|---|",
                  f"| FA1 order (this kernel), fetch GB | {m['model_fetch_bytes'] / 1e9:.3f} | "
                  f"{hrec['fetch_bytes_per_launch'] / 1e9:.3f} |",
                  f"| FA1 order (this kernel), write GB | {m['model_write_bytes'] / 1e9:.3f} | "
                  f"{hrec['write_bytes_per_launch'] / 1e9:.3f} |"]
        fa2 = profile_record(wl0)
        if fa2 is not None:
            m2 = fa2["io_model"]
            lines += [f"| FA2 order (fa_fwd, from `profiles/fa_fwd_{wl0}_hbm_counters.json`), "
                      f"fetch GB | {m2['model_fetch_bytes'] / 1e9:.3f} | "
                      f"{fa2['fetch_bytes_per_launch'] / 1e9:.3f} |",
                      f"| FA2 order (fa_fwd), write GB | {m2['model_write_bytes'] / 1e9:.3f} | "
                      f"{fa2['write_bytes_per_launch'] / 1e9:.3f} |"]
        lines += ["", "Model: the HBM column of the FA1/FA2 comparison table of "
                  "currybab.bearblog.dev (section \"정리\"): FA1 reads Q T_c times and reads "
                  "and writes O_i T_c times; FA2 reads K and V T_r times, Q once and writes O "
                  "once. The FA1 order meets its model to the byte (its re-read tensors do not "
                  "fit an XCD's 4 MB L2); the FA2 order's K/V re-reads are served by the L2, "
                  "since all query tiles of a head run at once on one XCD.", ""]
    lines.append("    python bench.py --path " + path + " --summarize-traces " + " ".join(
        f"{wl}=<kt_dir_{wl}>" for wl, _ in entries) +
        (" --sq-dirs <sq1_dir> <sq2_dir>" if sq_dirs else "") +
        (f" --hbm-dirs <fetch_dir> <write_dir> --calibrate-copy-mib {copy_mib}" if hbm_dirs else ""))
    lines.append("")
    with open(os.path.join(out_dir, f"fa_{path}_rocprof.md"), "w") as f:
        f.write("\n".join(lines))
    with open(os.path.join(out_dir, f"fa_{path}_counters.json"), "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def profile_record(workload: str, path: str = "fwd"):
    """The committed counter summary of a workload, if it was taken on the current
    kernel source; else None."""
    stem = "fa_fwd" if path == "fwd" else f"fa_{path}"
    fn = os.path.join(ROOT, "profiles", f"{stem}_{workload}_hbm_counters.json")
    try:
        with open(fn) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_hash():
        return None
    return rec


def profile_fields(workload: str, ms: float):
    """Per-config figures from the committed profile (HBM bytes and their rate at this
    run's time, MFMA busy, VALU busy, LDS bank conflicts, clock under load), or a null
    marker."""
    rec = profile_record(workload)
    if rec is None:
        return {"profile": None}
    out = {"hbm_bytes_per_launch": round(rec["hbm_bytes_per_launch"]),
           "hbm_GBps": round(rec["hbm_bytes_per_launch"] / (ms * 1e-3) / 1e9, 1),
           "traffic_over_algorithmic": round(rec["traffic_over_algorithmic"], 3)}
    sq = rec.get("sq")
    if sq:
        out.update({"mfma_busy_pct": round(sq["mfma_busy_pct"], 1),
                    "lds_bank_conflict_cycles": sq["lds_bank_conflict_cycles"],
                    "valu_insts_per_mfma": round(sq["valu_insts_per_mfma"], 2),
                    "clock_GHz_under_load": round(sq["clock_GHz_under_load"], 3)})
        if "valu_issue_pct_of_wave_cycles" in sq:
            out["valu_busy_pct_of_wave_cycles"] = round(sq["valu_issue_pct_of_wave_cycles"], 1)
    out["profile"] = f"profiles/fa_fwd_{workload}_rocprof.md"
    return out


def device_peak():
    """16-bit MFMA peak from the device's CU count and peak engine clock."""
    import io_aware_exact_fa2_amd as fa

    cus, khz = fa.fa_device_info(0)
    return cus, khz, cus * khz * 1e3 * 4096 / 1e12


def cpu_baseline(w, budget_s: float):
    """The float64 oracle on whole heads of the same workload until ~budget_s."""
    import numpy as np
    import oracle
    from oracle.attention import default_workers
    import workloads

    q, k, v = workloads.make_inputs(w)
    qf, kf, vf = (workloads.to_f64(t) for t in (q, k, v))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    workers = default_workers()
    done = 0
    t0 = time.perf_counter()
    step = max(1, min(len(heads), workers))
    # whole heads (all rows) until the budget is spent; passes repeat if one is shorter
    while True:
        i = done % len(heads)
        batch = heads[i:i + step]
        oracle.attention_rows(qf, kf, vf, w.scale, w.causal, batch, np.arange(w.N),
                              workers=workers)
        done += len(batch)
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = w.flops() * done / len(heads)
    return {"value": flops / dt / 1e12, "unit": "TFLOPS", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{done} whole-head passes (all {w.N} rows each) cycling over the "
                      f"{len(heads)} (b,h) heads of {w.name}, float64 numpy, {dt:.1f} s"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ai2048")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for cpu_baseline (0 disables)")
    ap.add_argument("--also", default="causal8k,long32k,stress4000",
                    help="extra workloads timed for the 'workloads' field ('' for none)")
    ap.add_argument("--path", default="fwd",
                    help="with --summarize-hbm or for profiling runs: fwd (the FA2-order "
                         "forward, the default and the headline), bwd, fp8, fa1, splitkvS "
                         "(S key splits), splitkv (fa_fwd, then the split-KV pass)")
    ap.add_argument("--backward", default="ai2048,causal8k,long32k,stress4000",
                    help="workloads whose backward pass is also timed (comma list; empty: none)")
    ap.add_argument("--fp8", default="ai2048,causal8k,long32k",
                    help="workloads whose 8-bit (E4M3) forward is also timed (empty: none)")
    ap.add_argument("--splitkv", default=",".join(f"{k}:{v}" for k, v in SPLITKV.items()),
                    help="few-tile workloads timed through fa_fwd and fa_fwd_splitkv "
                         "(name:splits comma list; empty: none)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-hbm", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize two rocprofv3 --pmc runs into profiles/ (no GPU work)")
    ap.add_argument("--commands", default="", help="commands recorded in the summary")
    ap.add_argument("--summarize-profile", nargs=5,
                    metavar=("KT_DIR", "SQ1_DIR", "SQ2_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/*_rocprof.md and *_hbm_counters.json from five "
                         "rocprofv3 runs (no GPU work)")
    ap.add_argument("--summarize-traces", nargs="+", metavar="WORKLOAD=KT_DIR",
                    help="with --path bwd|fp8|fa1: write profiles/fa_<path>_rocprof.md from "
                         "kernel-trace runs (no GPU work)")
    ap.add_argument("--sq-dirs", nargs=2, metavar=("SQ1_DIR", "SQ2_DIR"))
    ap.add_argument("--hbm-dirs", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--profile-args", default=" --cpu-budget 0 --also '' --backward '' "
                    "--fp8 '' --splitkv '' --steps 20 --warmup 3",
                    help="bench.py arguments the profiled runs used (recorded)")
    a = ap.parse_args(argv)
    if a.summarize_traces:
        entries = [tuple(e.split("=", 1)) for e in a.summarize_traces]
        rec = summarize_traces(a.path, entries, a.sq_dirs, a.hbm_dirs,
                               a.calibrate_copy_mib or 512)
        print(json.dumps({k: v["tflops"] for k, v in rec["workloads"].items()}))
        return 0
    if a.summarize_profile:
        rec = summarize_profile(a.workload, a.summarize_profile, a.calibrate_copy_mib or 512,
                                a.path, a.profile_args)
        print(json.dumps({"workload": rec["workload"], "sq": rec["sq"],
                          "traffic_over_algorithmic": rec["traffic_over_algorithmic"]}))
        return 0
    if a.summarize_hbm:
        stem = "fa_fwd" if a.path == "fwd" else f"fa_{a.path}"
        out = os.path.join(ROOT, "profiles", f"{stem}_{a.workload}_hbm_counters.json")
        rec = summarize_hbm(a.workload, a.summarize_hbm[0], a.summarize_hbm[1],
                            a.calibrate_copy_mib, out, a.commands, a.path)
        print(json.dumps(rec))
        return 0
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}): the attention forward "
              "here is built and timed on a single MI355X; see DESIGN.md for how it would "
              "shard.", file=sys.stderr)
        return 2

    import torch
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if a.calibrate_copy_mib:
        calibrate_copy(a.calibrate_copy_mib)
    w = workloads.get(a.workload)
    if a.path == "splitkv":
        # the plain forward, then the split-KV pass, on one shape (for profiling runs)
        for leg in ("fwd", f"splitkv{SPLITKV.get(w.name, 4)}"):
            msx, _, ranx = time_gpu(w, a.steps, a.warmup, leg=leg)
            print(json.dumps({"path": leg, "workload": w.name, "ms": round(msx, 5),
                              "tflops": round(w.flops() / (msx * 1e-3) / 1e12, 2),
                              "steps": a.steps, "warmup_steps_run": ranx}), flush=True)
        return 0
    if a.path != "fwd":
        # one pass other than the headline forward, for profiling runs
        msx, wallx, ranx = time_gpu(w, a.steps, a.warmup, leg=a.path)
        work = 2.5 * w.flops() if a.path == "bwd" else w.flops()
        print(json.dumps({"path": a.path, "workload": w.name, "ms": round(msx, 5),
                          "tflops": round(work / (msx * 1e-3) / 1e12, 2),
                          "steps": a.steps, "warmup_steps_run": ranx}), flush=True)
        return 0
    ms, wall, warm_ran = time_gpu(w, a.steps, a.warmup)
    tflops = w.flops() / (ms * 1e-3) / 1e12
    traffic = measured_traffic(w.name)
    roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tflops / PEAK_TFLOPS, 4), "traffic": traffic}
    cus, khz, peak_dev = device_peak()
    peaks = {"published_tflops": PEAK_TFLOPS, "frac_published": round(tflops / PEAK_TFLOPS, 4),
             "device_cus": cus, "device_clock_mhz": khz / 1e3,
             "clock_derived_tflops": round(peak_dev, 1),
             "frac_clock_derived": round(tflops / peak_dev, 4),
             "formula": "CUs x peak engine clock x 4096 flop/cycle (hipDeviceProp_t)"}
    prof = profile_fields(w.name, ms)
    if prof.get("clock_GHz_under_load"):
        ghz = prof["clock_GHz_under_load"]
        peaks["clock_under_load_GHz"] = ghz
        peaks["at_clock_under_load_tflops"] = round(cus * ghz * 1e9 * 4096 / 1e12, 1)
        peaks["frac_at_clock_under_load"] = round(tflops / peaks["at_clock_under_load_tflops"], 4)
    ms_cold = time_cold(w, 10)
    cold = {"ms": round(ms_cold, 4), "tflops": round(w.flops() / (ms_cold * 1e-3) / 1e12, 1),
            "scrub_mib": 512, "statistic": "median of 10 launches, each after the scrub"}
    extra = {}
    for name in [s for s in a.also.split(",") if s]:
        wx = workloads.get(name)
        msx, _, _ = time_gpu(wx, max(5, a.steps // 5), 3)
        tx = wx.flops() / (msx * 1e-3) / 1e12
        extra[name] = {"ms": round(msx, 4), "tflops": round(tx, 1),
                       "pct_bf16_peak": round(100 * tx / PEAK_TFLOPS, 1),
                       "pct_clock_derived_peak": round(100 * tx / peak_dev, 1), "dtype": wx.dtype,
                       "causal": wx.causal, "shape": [wx.B, wx.H, wx.N, wx.d],
                       **profile_fields(name, msx)}
    bwd = {}
    for name in [s for s in a.backward.split(",") if s]:
        wx = workloads.get(name)
        msx, _, _ = time_gpu(wx, max(5, a.steps // 5), 3, leg="bwd")
        tx = 2.5 * wx.flops() / (msx * 1e-3) / 1e12
        bwd[name] = {"ms": round(msx, 4), "tflops": round(tx, 1),
                     "pct_bf16_peak": round(100 * tx / PEAK_TFLOPS, 1), "dtype": wx.dtype,
                     "causal": wx.causal, "shape": [wx.B, wx.H, wx.N, wx.d],
                     "flops": "2.5 x forward: five N x N x d products (dV, dP, dQ, dK, S)"}
    f8 = {}
    for name in [s for s in a.fp8.split(",") if s]:
        wx = workloads.get(name)
        msx, _, _ = time_gpu(wx, max(5, a.steps // 5), 3, leg="fp8")
        tx = wx.flops() / (msx * 1e-3) / 1e12
        f8[name] = {"ms": round(msx, 4), "tflops": round(tx, 1),
                    "pct_fp8_peak": round(100 * tx / PEAK_FP8_TFLOPS, 1),
                    "causal": wx.causal, "shape": [wx.B, wx.H, wx.N, wx.d],
                    "inputs": "E4M3 codes with per-tensor scales, bf16 O"}
    skv = {}
    for item in [s for s in a.splitkv.split(",") if s]:
        name, _, ns = item.partition(":")
        wx = workloads.get(name)
        ns = int(ns or SPLITKV.get(name, 4))
        ms_f, _, _ = time_gpu(wx, max(5, a.steps // 5), 3)
        ms_s, _, _ = time_gpu(wx, max(5, a.steps // 5), 3, leg=f"splitkv{ns}")
        skv[name] = {"shape": [wx.B, wx.H, wx.N, wx.d], "causal": wx.causal, "dtype": wx.dtype,
                     "splits": ns, "fa_fwd_ms": round(ms_f, 4),
                     "fa_fwd_tflops": round(wx.flops() / (ms_f * 1e-3) / 1e12, 1),
                     "splitkv_ms": round(ms_s, 4),
                     "splitkv_tflops": round(wx.flops() / (ms_s * 1e-3) / 1e12, 1),
                     "speedup": round(ms_f / ms_s, 3)}
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "warmup_steps_run": warm_ran,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded N(0,1) Q, K, V rounded to bf16",
        "config": {"workload": f"{w.name}: non-causal attention forward" if not w.causal
                   else f"{w.name}: causal attention forward",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
                   "scale": w.scale},
        "pct_bf16_peak": round(100 * tflops / PEAK_TFLOPS, 2),
        "peak": peaks,
        "profile": prof,
        "algorithmic_GBps": round(w.min_bytes() / (ms * 1e-3) / 1e9, 1),
        "wall_s_timed": round(wall, 4),
        "kernel_source_sha256_16": kernel_hash(),
        "roofline": roof,
        "cold": cold,
        "workloads": extra,
        "backward": bwd,
        "fp8": f8,
        "splitkv": skv,
    }
    if a.cpu_budget > 0:
        line["cpu_baseline"] = cpu_baseline(w, a.cpu_budget)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
