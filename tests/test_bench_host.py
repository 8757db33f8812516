"""Host tests of bench.py's measurement helpers (no GPU): kernel classification,
the HBM-traffic record built from rocprofv3 counter CSVs (calibrated on the
largest copy dispatch, stamped with the kernel sources' hash) and dW's
algorithmic bytes per launch."""
import csv
import json
import os

import pytest

import bench
from workloads import gen

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]

COPY = "__amd_rocclr_copyBuffer"
DW = "void sbp::gemm_bf16_pp_kernel<sbp::EpiAccum<1>, 0, 2>(sbp::OperandView, sbp::OperandView, int)"
LOGITS = "void sbp::gemm_bf16_pp_kernel<sbp::EpiLogits, 1, 0>(sbp::OperandView, sbp::OperandView, int)"


def _write_counters(d, counter, rows):
    """rows: (dispatch id, kernel name, value per instance, instances)."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for disp, name, val, inst in rows:
            for _ in range(inst):  # one row per counter instance (summed per dispatch)
                w.writerow({**{f: 0 for f in FIELDS}, "Dispatch_Id": disp, "Kernel_Name": name,
                            "Counter_Name": counter, "Counter_Value": val})


def test_kernel_kind():
    assert bench.kernel_kind(COPY) == "copy"
    assert bench.kernel_kind(DW) == "dw_gemm"
    assert bench.kernel_kind(LOGITS) == "logits_lse"
    assert bench.kernel_kind("void sbp::gemm_bf16_pp_kernel<sbp::EpiStore, 1, 2>(...)") == "dh_gemm"
    assert bench.kernel_kind("void sbp::(anonymous namespace)::rows_kernel<true, true, false>(...)") == "rows_lse_dlogits"
    assert bench.kernel_kind("at::native::FillFunctor<int>") is None
    # the split-K reduce is not torch's read-only reduction of the calibration
    assert bench.kernel_kind("sbp::(anonymous namespace)::splitk_reduce_kernel(float const*, int)") == "dh_splitk_reduce"
    assert bench.kernel_kind("void at::native::reduce_kernel<512, 1, at::native::ReduceOp<float>>") == "read_only"


def test_trace_roofline(tmp_path):
    """Per-kind fractions from a kernel trace's stats: mean launch time over
    the kinds' kernels (the two dW variants pooled, weighted by calls) and the
    workload's algorithmic flops and bytes per launch at T / chunks rows."""
    d = tmp_path / "t"
    d.mkdir()
    with open(d / "t_kernel_stats.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                                           "MaxNs", "StdDev"])
        w.writeheader()
        for name, calls, avg in ((LOGITS, 10, 800e3), (DW, 8, 1000e3),
                                 ("void sbp::gemm_bf16_pp_persistent_kernel<sbp::EpiAccum<0, true>, 0, 2, true>()", 2,
                                  500e3), (COPY, 1, 5e3)):
            w.writerow({"Name": name, "Calls": calls, "TotalDurationNs": calls * avg, "AverageNs": avg,
                        "Percentage": 0, "MinNs": avg, "MaxNs": avg, "StdDev": 0})
    wl = gen.SFT_9K.with_(T=2000, C=1024)       # 2 chunks of 1000 rows on average
    rl = bench.trace_roofline(str(d), wl)
    assert set(rl) == {"logits_lse", "dw_gemm"}  # the copy is left out
    f = 2.0 * 1000 * wl.V * wl.D
    assert rl["logits_lse"]["launches"] == 10 and rl["logits_lse"]["avg_us"] == pytest.approx(800.0)
    assert rl["logits_lse"]["tflops"] == pytest.approx(f / 800e-6 / 1e12)
    assert rl["logits_lse"]["frac_mfma"] == pytest.approx(f / 800e-6 / 1e12 / bench.PEAK_BF16_TFLOPS)
    assert "frac_hbm" not in rl["logits_lse"]
    assert rl["dw_gemm"]["avg_us"] == pytest.approx(900.0)   # (8 x 1000 + 2 x 500) / 10
    b = bench.dw_bytes_per_launch(1000, 2, wl)
    assert rl["dw_gemm"]["frac_hbm"] == pytest.approx(b / 900e-6 / 1e9 / bench.PEAK_HBM_GBS)
    assert "| dw_gemm | 10 | 900.0 |" in bench.roofline_markdown(rl)


def test_traffic_record_calibration_and_staleness(tmp_path, monkeypatch):
    root = tmp_path / "root"
    (root / "loss_head_amd" / "csrc").mkdir(parents=True)
    (root / "profiles").mkdir()
    src = root / "loss_head_amd" / "csrc" / "k.hip"
    src.write_text("// kernel source v1\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    mib = 1024
    # FETCH_SIZE reads twice the copy's size in KiB (so the scale is 0.5), WRITE_SIZE
    # exactly; a small copy of the workload must not be taken for the calibration
    kib = (mib << 20) / 1024
    fdir, wdir = str(tmp_path / "f"), str(tmp_path / "w")
    _write_counters(fdir, "FETCH_SIZE", [(1, COPY, kib, 2), (2, COPY, 3.0, 1), (3, DW, 1000.0, 2), (4, DW, 3000.0, 2),
                                         (5, LOGITS, 500.0, 4)])
    _write_counters(wdir, "WRITE_SIZE", [(1, COPY, kib, 1), (2, COPY, 1.0, 1), (3, DW, 700.0, 1), (4, DW, 900.0, 1),
                                         (5, LOGITS, 250.0, 1)])
    bench.write_traffic("wl", fdir, wdir, mib)
    rec = json.load(open(root / "profiles" / "wl_traffic.json"))
    assert rec["source_sha256"] == bench.kernel_source_sha256()
    assert rec["calibration"]["fetch_scale"] == pytest.approx(0.5)
    assert rec["calibration"]["write_scale"] == pytest.approx(1.0)
    dw = rec["per_launch"]["dw_gemm"]
    # per dispatch: instances summed (2000, 6000 KiB), then averaged, then scaled
    assert dw["dispatches"] == 2
    assert dw["fetch_bytes"] == pytest.approx(4000 * 1024 * 0.5)
    assert dw["write_bytes"] == pytest.approx(800 * 1024)
    assert rec["per_launch"]["logits_lse"]["fetch_bytes"] == pytest.approx(2000 * 1024 * 0.5)
    assert "copy" not in rec["per_launch"]
    assert bench.recorded_traffic("wl", "dw_gemm") == pytest.approx(4000 * 1024 * 0.5 + 800 * 1024)
    assert bench.recorded_traffic("wl", "dh_gemm") is None
    # any change to the kernel sources makes the record stale
    src.write_text("// kernel source v2\n")
    assert bench.recorded_traffic("wl", "dw_gemm") is None


def test_dw_algorithmic_bytes():
    wl = gen.SFT_9K
    # 9 chunks averaging 1000 rows: G and H_c read, dW written, and the old dW
    # read on 8 of the 9 launches
    got = bench.dw_bytes_per_launch(1000, 9, wl)
    vd4 = 4 * wl.V * wl.D
    assert got == pytest.approx(1000 * wl.V * 2 + 1000 * wl.D * 2 + vd4 + vd4 * 8 / 9)
    assert got == pytest.approx(3247771876, abs=1)
    assert bench.dw_bytes_per_launch(1000, 1, wl) == pytest.approx(1000 * wl.V * 2 + 1000 * wl.D * 2 + vd4)


def test_row_pass_bytes_are_dominated_by_the_logits_buffer():
    # the backward row pass reads the chunk logits and writes the gradient in
    # place (2 bytes each at bf16); everything else it touches is a few percent
    wl = gen.SFT_9K
    b = bench.rows_bytes_per_launch(1024, wl)
    zg = 2 * 1024 * wl.V * 2
    assert zg < b < 1.05 * zg
    assert bench.rows_bytes_per_launch(0, wl) == 0
