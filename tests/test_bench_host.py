"""Host logic of bench.py: the one-GPU guard and the rocprofv3 summary arithmetic, on
synthetic profiler output written here (no GPU)."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402

FA = "void fa::fa_fwd_wide_kernel<true, 128, false, 64, 4>(fa::Params)"
COPY = "void at::native::vectorized_elementwise_kernel<4, MulFunctor<float> >(int)"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def _pmc(d, per_kernel):
    rows = []
    for kernel, counters in per_kernel.items():
        for name, vals in counters.items():
            rows += [[kernel, name, v] for v in vals]
    _write(os.path.join(d, "host", "p_counter_collection.csv"),
           ["Kernel_Name", "Counter_Name", "Counter_Value"], rows)


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_profile_summary_arithmetic(tmp_path):
    """A launch of 125 us that counts 8 x 2.2e6 x 125e-6 ... GRBM cycles runs at 2.2 GHz;
    MFMA busy, VALU per MFMA and the copy-calibrated HBM bytes follow from the counters."""
    w = workloads.get("ai2048")
    avg_ns = 125_000.0
    grbm = 8 * 2.2e9 * avg_ns * 1e-9            # 2.2 GHz on all 8 XCDs
    mfma = w.flops() / 32768
    busy = 0.5 * (grbm / 8) * 1024              # half the active cycles on every SIMD
    dirs = [str(tmp_path / n) for n in ("kt", "sq1", "sq2", "fetch", "write")]
    _write(os.path.join(dirs[0], "host", "kt_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
            "StdDev"],
           [[COPY, 3, 3000, 1000, 1, 900, 1100, 10],
            [FA, 100, 100 * avg_ns, avg_ns, 99, avg_ns - 1e3, avg_ns + 1e3, 5]])
    _pmc(dirs[1], {FA: {"GRBM_GUI_ACTIVE": [grbm, grbm], "SQ_WAVES": [2048],
                        "SQ_BUSY_CYCLES": [1.0], "SQ_VALU_MFMA_BUSY_CYCLES": [busy],
                        "SQ_INSTS_MFMA": [mfma], "SQ_INSTS_VALU": [6 * mfma],
                        "SQ_INSTS_LDS": [1.0], "SQ_LDS_BANK_CONFLICT": [0.0],
                        "SQ_LDS_IDX_ACTIVE": [1e6]}})
    _pmc(dirs[2], {FA: {"SQ_WAVE_CYCLES": [100.0], "SQ_WAIT_ANY": [20.0],
                        "SQ_WAIT_INST_ANY": [10.0], "SQ_ACTIVE_INST_ANY": [70.0],
                        "SQ_ACTIVE_INST_VALU": [50.0], "SQ_ACTIVE_INST_LDS": [5.0],
                        "SQ_VALU_MFMA_COEXEC_CYCLES": [busy / 4], "SQ_INSTS_SALU": [1.0]}})
    # the copy of 512 MiB reads half (fetch counter in 64-byte units of 32 B ...): scale 2
    _pmc(dirs[3], {FA: {"FETCH_SIZE": [50_000.0]}, COPY: {"FETCH_SIZE": [512 * 1024 / 2]}})
    _pmc(dirs[4], {FA: {"WRITE_SIZE": [30_000.0]}, COPY: {"WRITE_SIZE": [512 * 1024.0]}})
    out = tmp_path / "out"
    out.mkdir()
    rec = bench.summarize_profile("ai2048", dirs, 512, out_dir=str(out))
    sq = rec["sq"]
    assert sq["clock_GHz_under_load"] == pytest.approx(2.2)
    assert sq["mfma_busy_pct"] == pytest.approx(50.0)
    assert sq["cycles_per_mfma"] == pytest.approx(busy / mfma)
    assert sq["valu_insts_per_mfma"] == pytest.approx(6.0)
    assert sq["mfma_insts_expected"] == pytest.approx(mfma)
    assert sq["waitcnt_pct_of_wave_cycles"] == pytest.approx(20.0)
    assert sq["mfma_valu_coexec_pct_of_mfma_busy"] == pytest.approx(25.0)
    assert rec["hbm_bytes_per_launch"] == pytest.approx((2 * 50_000.0 + 30_000.0) * 1024)
    assert rec["traffic_over_algorithmic"] == pytest.approx(
        rec["hbm_bytes_per_launch"] / w.min_bytes())
    assert rec["kernel_trace"]["calls"] == 100
    assert rec["kernel_trace"]["tflops_at_average"] == pytest.approx(
        w.flops() / (avg_ns * 1e-9) / 1e12)
    md = (out / "fa_fwd_ai2048_rocprof.md").read_text()
    assert "2.200 GHz" in md and "rocprofv3 --pmc FETCH_SIZE" in md
    assert json.loads((out / "fa_fwd_ai2048_hbm_counters.json").read_text())["sq"] == sq


def test_trace_summary_backward(tmp_path):
    """The backward summary sums its three kernels' trace averages into one pass and
    prices it at 2.5x the forward flops; the SQ table is per kernel."""
    w = workloads.get("ai2048")
    names = ["void fa::fa_bwd_delta_kernel<true, 128>(fa::BwdParams)",
             "void fa::fa_bwd_dkdv_kernel<true, 128, false>(fa::BwdParams)",
             "void fa::fa_bwd_dq_kernel<true, 128, false>(fa::BwdParams)"]
    avgs = [10_000.0, 300_000.0, 200_000.0]
    kt = str(tmp_path / "kt")
    _write(os.path.join(kt, "host", "kt_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
            "StdDev"],
           [[COPY, 1, 5, 5, 0, 5, 5, 0]] + [[n, 10, 10 * a, a, 30, a, a, 0]
                                             for n, a in zip(names, avgs)])
    sq1, sq2 = str(tmp_path / "sq1"), str(tmp_path / "sq2")
    grbm = 8 * 2.0e9 * 300_000e-9
    _pmc(sq1, {names[1]: {"GRBM_GUI_ACTIVE": [grbm], "SQ_INSTS_MFMA": [100.0],
                          "SQ_INSTS_VALU": [650.0], "SQ_VALU_MFMA_BUSY_CYCLES":
                          [0.25 * 1024 * grbm / 8], "SQ_LDS_BANK_CONFLICT": [0.0]}})
    _pmc(sq2, {names[1]: {"SQ_WAVE_CYCLES": [10.0], "SQ_ACTIVE_INST_ANY": [4.0],
                          "SQ_WAIT_ANY": [3.0], "SQ_WAIT_INST_ANY": [2.0]}})
    out = tmp_path / "out"
    out.mkdir()
    rec = bench.summarize_traces("bwd", [("ai2048", kt)], (sq1, sq2), out_dir=str(out))
    total = sum(avgs)
    assert rec["workloads"]["ai2048"]["sum_of_averages_ns"] == pytest.approx(total)
    assert rec["workloads"]["ai2048"]["tflops"] == pytest.approx(
        2.5 * w.flops() / (total * 1e-9) / 1e12)
    sq = rec["sq"][names[1]]
    assert sq["valu_insts_per_mfma"] == pytest.approx(6.5)
    assert sq["mfma_busy_pct"] == pytest.approx(25.0)
    assert sq["clock_GHz_under_load"] == pytest.approx(2.0)
    assert sq["waitcnt_pct_of_wave_cycles"] == pytest.approx(30.0)
    md = (out / "fa_bwd_rocprof.md").read_text()
    assert "--summarize-traces ai2048=<kt_dir_ai2048>" in md and names[2] in md


def test_trace_summary_splitkv(tmp_path):
    """The split-KV summary adds the partial kernel and the merge into one pass and sets it
    against the plain forward's one kernel on the same shape."""
    w = workloads.get("few16k")
    fwd = "void fa::fa_fwd_wide_kernel<true, 128, false, 64, 4>(fa::Params)"
    part = "void fa::fa_fwd_wide_kernel<true, 128, false, 64, 4, true>(fa::Params)"
    merge = "void fa::fa_split_merge_kernel<true, 128>(float const*, float const*, " \
            "unsigned short*, float*, long long, int)"
    kt = str(tmp_path / "kt")
    _write(os.path.join(kt, "host", "kt_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
            "StdDev"],
           [[COPY, 1, 5, 5, 0, 5, 5, 0], [fwd, 10, 4e6, 400_000.0, 60, 4e5, 4e5, 0],
            [part, 10, 15e5, 150_000.0, 30, 1.5e5, 1.5e5, 0],
            [merge, 10, 1e5, 10_000.0, 10, 1e4, 1e4, 0]])
    out = tmp_path / "out"
    out.mkdir()
    rec = bench.summarize_traces("splitkv", [("few16k", kt)], out_dir=str(out))
    r = rec["workloads"]["few16k"]
    assert r["sum_of_averages_ns"] == pytest.approx(160_000.0)
    assert r["fa_fwd_ns"] == pytest.approx(400_000.0)
    assert r["speedup"] == pytest.approx(2.5)
    assert r["tflops"] == pytest.approx(w.flops() / 160e-6 / 1e12)
    assert r["fa_fwd_tflops"] == pytest.approx(w.flops() / 400e-6 / 1e12)
    assert r["splits"] == bench.SPLITKV["few16k"]
    md = (out / "fa_splitkv_rocprof.md").read_text()
    assert "| few16k | 4 | 400.0 |" in md and "(merge)" in md


def test_split_kernel_names():
    """The split-KV pass's kernels (either forward kernel's split instantiation, and the
    merge) are told apart from the plain forward by name."""
    assert bench._is_split("void fa::fa_fwd_wide_kernel<true, 128, true, 64, 4, true>(fa::Params)")
    assert bench._is_split("void fa::fa_fwd_fast_kernel<false, 64, false, 4, 64, 2, true, 1>"
                           "(fa::Params)")
    assert not bench._is_split("void fa::fa_fwd_fast_kernel<false, 64, true, 4, 64, 2, false, 1>"
                               "(fa::Params)")
    assert bench._is_split("void fa::fa_split_merge_kernel<true, 128>(float const*)")
    assert not bench._is_split("void fa::fa_fwd_wide_kernel<true, 128, false, 64, 4, false>"
                               "(fa::Params)")
