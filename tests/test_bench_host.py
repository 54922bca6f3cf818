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
        "void poetx::gemm_wide_kernel<false, false>(poetx::GemmArgs, int, int, int)": ("gemm_nt", 1),
        "void poetx::gemm_wide_kernel<false, true>(poetx::GemmArgs, int, int, int)": ("gemm_nt_rside", 1),
        "void poetx::gemm_wide_kernel<true, false>(poetx::GemmArgs, int, int, int)": ("gemm_nn", 1),
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
    nt = "void poetx::gemm_wide_kernel<false, false>(poetx::GemmArgs, int, int, int)"
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
    # the records name the run they were taken on and serve that run only
    tag = bench.profiled_run_tag()
    assert rec["workload"] == tag
    assert bench.counter_record("traffic", "gemm_nt", tag)["hbm_bytes_per_launch"] == rec["hbm_bytes_per_launch"]
    assert bench.counter_record("traffic", "gemm_nt", bench.run_tag("llama7b_mlp_11008x4096_bf16_b256", 8192)) is None
    assert bench.counter_record("traffic", "gemm_nt", bench.run_tag("llama1b_layerset_bf16_b256", 4096)) is None
    assert bench.counter_record("traffic", "gemm_nt", bench.run_tag("llama1b_layerset_bf16_b256", 8192,
                                                                      w0_int8=True)) is None
    assert bench.counter_record("traffic", "gemm_nt", bench.run_tag("llama1b_layerset_bf16_b256", 8192)) is None


def test_traffic_summary_needs_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    nt = "void poetx::gemm_wide_kernel<false, false>(poetx::GemmArgs, int, int, int)"
    _write_pmc(str(tmp_path / "f"), [(1, nt, "FETCH_SIZE", 10.0)])
    _write_pmc(str(tmp_path / "w"), [(1, nt, "WRITE_SIZE", 10.0)])
    with pytest.raises(SystemExit):
        bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"))


def test_trace_window_keeps_the_marked_pass(tmp_path):
    path = str(tmp_path / "bench_kernel_trace.csv")
    rows = [("sigmoid_kernel", 0, 10),            # earlier markers are ignored
            ("poetx::gram_stream_kernel", 20, 30),
            ("sigmoid_kernel", 100, 110),         # opens the window
            ("void poetx::gemm_wide_kernel<false, false>", 120, 220),
            ("void poetx::gemm_wide_kernel<false, false>", 230, 330),
            ("poetx::gram_reduce_kernel", 340, 350),
            ("sigmoid_kernel", 400, 410),         # closes it
            ("void poetx::gemm_wide_kernel<false, false>", 500, 900)]
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name, t0, t1 in rows:
            w.writerow(dict(Kernel_Name=name, Start_Timestamp=t0, End_Timestamp=t1))
    got = {r["Name"]: (int(r["Calls"]), float(r["TotalDurationNs"])) for r in bench._trace_window(path, None)}
    assert got == {"void poetx::gemm_wide_kernel<false, false>": (2, 200.0), "poetx::gram_reduce_kernel": (1, 10.0)}


def test_mfma_summary_from_counters(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda files: "feedbeef")
    os.makedirs(tmp_path / "profiles")
    nt = "void poetx::gemm_wide_kernel<false, false>(poetx::GemmArgs, int, int, int)"
    rows = []
    # two launches; MOPS and busy cycles arrive per SE and are summed, GUI_ACTIVE per XCD (max)
    for did, mops, busy in ((1, 1000.0, 2.0e5), (2, 3000.0, 6.0e5)):
        rows += [(did, nt, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops / 2), (did, nt, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops / 2),
                 (did, nt, "SQ_VALU_MFMA_BUSY_CYCLES", busy), (did, nt, "GRBM_GUI_ACTIVE", 1.0e6),
                 (did, nt, "SQ_BUSY_CU_CYCLES", 256 * 1000.0)]
    _write_pmc(str(tmp_path / "m"), rows)
    bench.mfma_from(str(tmp_path / "m"))
    rec = json.load(open(tmp_path / "profiles" / "mfma_gemm_nt.json"))
    assert rec["launches"] == 2 and rec["source_hash"] == "feedbeef"
    assert rec["mfma_flops_per_launch"] == (1000 + 3000) * 512 / 2
    # busy cycles per SIMD over busy cycles per compute unit
    assert rec["mfma_busy_frac"] == round(((2.0e5 + 6.0e5) / bench.SIMD_COUNT) / (2 * 1000.0), 4)
    assert rec["cu_busy_cycles_per_launch"] == 1000


def test_counter_summaries_keep_the_marked_pass(tmp_path, monkeypatch):
    # dispatches before the marker pair (warmup, timed steps) and after it
    # (the merge's small products) stay out of the per-launch figures
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda files: "feedbeef")
    os.makedirs(tmp_path / "profiles")
    nn = "void poetx::gemm_wide_kernel<true, false>(poetx::GemmArgs, int, int, int)"
    mark = "void at::native::vectorized_elementwise_kernel<4, at::native::sigmoid_kernel_cuda...>"
    rows = []
    for did, name, mops in ((1, nn, 10.0), (2, mark, 0.0), (3, nn, 4000.0), (4, nn, 4000.0), (5, mark, 0.0),
                            (6, nn, 10.0)):
        rows += [(did, name, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops), (did, name, "SQ_VALU_MFMA_BUSY_CYCLES", 1.0),
                 (did, name, "GRBM_GUI_ACTIVE", 1.0), (did, name, "SQ_BUSY_CU_CYCLES", 256.0)]
    _write_pmc(str(tmp_path / "m"), rows)
    bench.mfma_from(str(tmp_path / "m"))
    rec = json.load(open(tmp_path / "profiles" / "mfma_gemm_nn.json"))
    assert rec["launches"] == 2 and rec["mfma_flops_per_launch"] == 4000 * 512
    assert bench._marked({1: nn, 2: mark, 3: nn, 5: mark, 6: nn}) == {3}
    assert bench._marked({1: nn, 3: nn}) == {1, 3}


def test_balance_streams_places_every_matrix_once():
    # the layer set: q, k, v, o, gate, up, down at 8192 tokens over 3 streams
    shapes = [(2048, 2048)] * 4 + [(5632, 2048), (5632, 2048), (2048, 5632)]
    where = bench.balance_streams(shapes, 8192, 3)
    assert len(where) == len(shapes) and set(where) <= {0, 1, 2}
    # the three MLP matrices (largest) each go to a stream of their own
    assert len({where[4], where[5], where[6]}) == 3
    assert bench.balance_streams(shapes, 8192, 1) == [0] * len(shapes)
    # the 24-layer stack: the same shapes 24 times; loads within one matrix of each other
    stack = shapes * 24
    w24 = bench.balance_streams(stack, 8192, 3)
    cost = [6.0 * 8192 * m * n / 1.1e15 + (28.0 * n + 20.0 * m) * 8192 / 3.5e12 for m, n in stack]
    load = [sum(c for c, w in zip(cost, w24) if w == s) for s in range(3)]
    assert max(load) - min(load) <= max(cost)


def test_concurrency_summary_counts_overlapping_gemms(tmp_path, capsys):
    # two steps (each opening with its two builds), then the marker: step 2
    # spans t = 100..200 with GEMMs over 110..150 and 130..170 (two at once
    # over 130..150) and a transform to 200; the marker is not counted
    rows = [("gj_kernel<256, 6>", 0, 10), ("gj_kernel<256, 6>", 0, 10), ("void poetx::gemm_wide_kernel<true, true>", 20, 60),
            ("gj_kernel<256, 6>", 100, 105), ("gj_kernel<256, 6>", 101, 108),
            ("void poetx::gemm_wide_kernel<true, false>", 110, 150), ("void poetx::gemm_wide_kernel<true, true>", 130, 170),
            ("poetx::blockdiag_pp_kernel", 170, 200), ("void at::sigmoid_kernel", 300, 301)]
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for r in rows:
            w.writerow(r)
    bench.concurrency_from(str(path), 1)
    out = capsys.readouterr().out
    assert "1 timed steps, 0.1 us per step, 5 launches" in out
    # 100 ns in all: none running over 100..110 and 170..200, one over
    # 110..130 and 150..170, two over 130..150
    assert "running: 0   40.0 %" in out and "running: 1   40.0 %" in out and "running: 2   20.0 %" in out
