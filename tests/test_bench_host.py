"""Host logic of bench.py (no GPU): the kernel-class map, the traffic summary
from rocprofv3 counter files, and the per-kernel window of a kernel trace,
on small synthetic CSV fixtures."""

import csv
import json
import os

import pytest

import bench


def test_kernel_classes_of_the_product_kernels():
    cases = {
        "void poetx::gemm_wide_kernel<false>(poetx::GemmArgs, int, int, int)": ("gemm_nt", 1),
        "void poetx::gemm_wide_kernel<true>(poetx::GemmArgs, int, int, int)": ("gemm_nn", 1),
        "void poetx::gemm_bf16_kernel<false, false, false>(poetx::GemmArgs, int, int, int)": ("gemm_nt", 1),
        "void poetx::gemm_bf16_kernel<true, false, true>(poetx::GemmArgs, int, int, int)": ("gemm_nn", 1),
        "void poetx::gemm_bf16_kernel<false, true, false>(poetx::GemmArgs, int, int, int)": ("xform_blockmul", 1),
        "void poetx::blockdiag_kernel<256>(unsigned short const*, ...)": ("xform_blockmul", 1),
        "void poetx::permute_gather_kernel<true>(poetx::PermArgs)": ("xform_permute", 1),
        "void poetx::permute_stream_kernel<false, false>(poetx::PermArgs)": ("xform_permute", 1),
        "poetx::gram_stream_kernel(unsigned short const*, ...)": ("gram", 2),
        "poetx::gram_reduce_kernel(float const*, int, long, float*)": ("gram", 2),
        "void poetx::chain_product_kernel<128, false, true>(poetx::ChainSegs, ...)": ("chain_rule", 3),
        "poetx::skew_project_kernel(float const*, ...)": ("chain_rule", 3),
        "void poetx::gj_kernel<256, 6>(poetx::GJArgs)": ("cayley_build", 1),
        "poetx::dequant_rows_kernel(signed char const*, ...)": ("dequant", 1),
        "void at::native::vectorized_elementwise_kernel<...>": (None, 1),
    }
    for name, want in cases.items():
        assert bench.kernel_class(name) == want, name


def _write_pmc(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for did, name, counter, val in rows:
            w.writerow(dict(Dispatch_Id=did, Kernel_Name=name, Counter_Name=counter, Counter_Value=val))


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda files: "feedbeef")
    nt = "void poetx::gemm_wide_kernel<false>(poetx::GemmArgs, int, int, int)"
    red = "poetx::gram_reduce_kernel(float const*, int, long, float*)"
    gram = "poetx::gram_stream_kernel(unsigned short const*, ...)"
    neg = "void at::native::neg_kernel_cuda(...)"
    mib = bench.CALIBRATION_BYTES / 1024.0
    # FETCH_SIZE reads half the copy's bytes (scale 2), WRITE_SIZE all of them;
    # counters arrive per XCD and are summed per dispatch
    _write_pmc(str(tmp_path / "f"), [(1, nt, "FETCH_SIZE", 600.0), (1, nt, "FETCH_SIZE", 400.0),
                                     (2, nt, "FETCH_SIZE", 3000.0),
                                     (3, gram, "FETCH_SIZE", 100.0), (4, red, "FETCH_SIZE", 20.0),
                                     (9, neg, "FETCH_SIZE", mib / 2)])
    _write_pmc(str(tmp_path / "w"), [(1, nt, "WRITE_SIZE", 50.0), (2, nt, "WRITE_SIZE", 150.0),
                                     (3, gram, "WRITE_SIZE", 8.0), (4, red, "WRITE_SIZE", 2.0),
                                     (9, neg, "WRITE_SIZE", mib)])
    bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"))
    rec = json.load(open(tmp_path / "profiles" / "traffic_gemm_nt.json"))
    assert rec["source_hash"] == "feedbeef" and rec["launches"] == 2
    assert rec["fetch_bytes_per_launch"] == round((1000.0 + 3000.0) * 1024 * 2 / 2)
    assert rec["write_bytes_per_launch"] == round((50.0 + 150.0) * 1024 / 2)
    assert rec["calibration"]["fetch_scale"] == 2.0 and rec["calibration"]["write_scale"] == 1.0
    # a Gram launch is the streaming kernel plus its reduction (two dispatches)
    g = json.load(open(tmp_path / "profiles" / "traffic_gram.json"))
    assert g["launches"] == 1 and g["hbm_bytes_per_launch"] == round(120.0 * 1024 * 2 + 10.0 * 1024)


def test_traffic_summary_needs_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    nt = "void poetx::gemm_wide_kernel<false>(poetx::GemmArgs, int, int, int)"
    _write_pmc(str(tmp_path / "f"), [(1, nt, "FETCH_SIZE", 10.0)])
    _write_pmc(str(tmp_path / "w"), [(1, nt, "WRITE_SIZE", 10.0)])
    with pytest.raises(SystemExit):
        bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"))


def test_trace_window_keeps_the_marked_pass(tmp_path):
    path = str(tmp_path / "bench_kernel_trace.csv")
    rows = [("sigmoid_kernel", 0, 10),            # earlier markers are ignored
            ("poetx::gram_stream_kernel", 20, 30),
            ("sigmoid_kernel", 100, 110),         # opens the window
            ("void poetx::gemm_wide_kernel<false>", 120, 220),
            ("void poetx::gemm_wide_kernel<false>", 230, 330),
            ("poetx::gram_reduce_kernel", 340, 350),
            ("sigmoid_kernel", 400, 410),         # closes it
            ("void poetx::gemm_wide_kernel<false>", 500, 900)]
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, t0, t1 in rows:
            w.writerow(dict(Kernel_Name=name, Start_Timestamp=t0, End_Timestamp=t1))
    got = {r["Name"]: (int(r["Calls"]), float(r["TotalDurationNs"])) for r in bench._trace_window(path, None)}
    assert got == {"void poetx::gemm_wide_kernel<false>": (2, 200.0), "poetx::gram_reduce_kernel": (1, 10.0)}
