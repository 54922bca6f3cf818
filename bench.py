"""Benchmark: POET-X layer fwd+bwd tokens/s on one MI355X.

Workload (default): the LLaMA-1B-shaped layer set -- q, k, v, o 2048x2048,
gate, up 5632x2048, down 2048x5632 -- bf16 W0, block size 256, 8192 tokens,
generators ~N(0, 1e-3).  --workload square: one 2048x2048 layer, b = 256,
4096 tokens; --workload mlp7b --b B: the 11008x4096 MLP projection at block
size B, 8192 tokens; --workload stack24: the 24-layer stack's training step.  One step is the hot path over one batch: forward of
all seven matrices, then backward of all seven (reverse order) with the
blocks and activations recomputed, generator gradients for every block and
the input gradient.  Inputs are seeded synthetic tensors already resident in
HBM before the timed region.

Prints one JSON line.  Besides the throughput it reports, for the kernel class
with the largest share of the step ("dominant"), the achieved rate from HIP
events recorded on the launch stream inside the library against the MI355X
peak (bf16 MFMA 2.5 PFLOP/s dense, HBM 8 TB/s), the HBM traffic measured by
rocprofv3 counters when a matching record exists under profiles/, and the
float64 oracle timed on the host cores on a bounded token sample.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
# MFMA-bound classes and the dense peak of the arithmetic they carry (flops
# counted as the algorithm's own, fp32 for the emulated classes): the weight
# products run on bf16 MFMA at 2.5 PFLOP/s; the chain rule forms each
# fp32-accurate product from three bf16 products of split operands (hi hi +
# hi lo + lo hi), so its fp32 flops peak at 2500/3; the Cayley builder's
# trailing updates take six (three-way splits), so 2500/6
MFMA_CLASSES = {"gemm_nt": 2500.0, "gemm_nt_rside": 2500.0, "gemm_nn": 2500.0, "gemm_nn_rside": 2500.0,
                "cayley_build": 2500.0 / 6, "chain_rule": 2500.0 / 3}
# the weight products (gemm_nt_rside / gemm_nn_rside: the forward's, with the
# R-side block product in its epilogue; their flops include that product's;
# the NN form reads the transposed weight copy)
GEMM_CLASSES = ("gemm_nt", "gemm_nt_rside", "gemm_nn", "gemm_nn_rside")
CU_COUNT = 256
SIMD_COUNT = 1024   # 256 compute units x 4 SIMDs
MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_BUSY_CU_CYCLES")
# HBM-bound classes of the block transforms (permutations, block products,
# Gram products)
HBM_CLASSES = ("xform_permute", "xform_blockmul", "xform_gather", "gram")

# kernel name (demangled, as rocprofv3 prints it) -> timing class of the library,
# and the dispatches one timed launch of the class makes
KERNEL_CLASSES = [
    ("permute_gather_kernel", "xform_permute", 1),
    ("permute_scatter_kernel", "xform_permute", 1),
    ("permute_stream_kernel", "xform_permute", 1),
    ("gather_blockdiag_kernel", "xform_gather", 1),    # before its substring below
    ("blockdiag_kernel", "xform_blockmul", 1),
    ("blockdiag_pp_kernel", "xform_blockmul", 1),
    ("gemm_bf16_kernel<false, true,", "xform_blockmul", 1),
    ("gemm_bf16_kernel<false, false,", "gemm_nt", 1),
    ("gemm_wide_kernel<false, false>", "gemm_nt", 1),
    ("gemm_wide_kernel<false, true>", "gemm_nt_rside", 1),
    ("gemm_wide_kernel<true, false>", "gemm_nn", 1),
    ("gemm_wide_kernel<true, true>", "gemm_nn_rside", 1),
    ("gemm_bf16_kernel<true, false,", "gemm_nn", 1),
    ("chain_product_kernel", "chain_rule", 3),
    ("skew_project_kernel", "chain_rule", 3),
    ("gj_kernel", "cayley_build", 1),
    ("gram_bf16_kernel", "gram", 2),
    ("gram_stream_kernel", "gram", 2),
    ("gram_reduce_kernel", "gram", 2),
    ("dequant_rows_kernel", "dequant", 1),
    ("quantize_rows_kernel", "quantize", 1),
]
CALIBRATION_BYTES = 256 << 20   # the copy kernel reads and writes this many bytes each
# sources whose hash keys the committed counter records
SOURCE_FILES = ["api.hip", "build.hip", "chain.hip", "transform.hip", "blockdiag.hip", "gemm.hip", "gram.hip",
                "merge.hip", "quant.hip", "cnp.hip", "common.h", "kernels.h"]


def balance_streams(shapes, N, nstreams, kind="step"):
    """Stream index per matrix: longest first onto the least loaded stream,
    by an estimate of each matrix's fwd+bwd time (three GEMMs at 1.1 PF/s;
    28n + 20m bytes of block transforms per token at 3.5 TB/s), or for
    kind "merge" of its merge (a chain of about ten short launches, 100 us,
    and 8mn bytes of products and relayout at 3 TB/s)."""
    if kind == "merge":
        cost = [1e-4 + 8.0 * m * n / 3e12 for m, n in shapes]
    else:
        cost = [6.0 * N * m * n / 1.1e15 + (28.0 * n + 20.0 * m) * N / 3.5e12 for m, n in shapes]
    load, where = [0.0] * nstreams, [0] * len(shapes)
    for i in sorted(range(len(shapes)), key=lambda i: -cost[i]):
        w = min(range(nstreams), key=lambda w: load[w])
        where[i] = w
        load[w] += cost[i]
    return where


def dominant_roofline(per_step, tag):
    """roofline of the class with the most time in a serialized pass: achieved
    algorithmic flops (MFMA classes) or bytes over its event-timed duration,
    against the MI355X peak, with the HBM bytes per launch from the committed
    counter record (null if none for the current sources)."""
    dom = max(per_step, key=lambda k: per_step[k]["ms"])
    d = per_step[dom]
    if dom in MFMA_CLASSES:
        achieved = d["flops"] / (d["ms"] * 1e-3) / 1e12
        peak = MFMA_CLASSES[dom]
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=peak, unit="TFLOP/s",
                    frac=round(achieved / peak, 4))
    else:
        achieved = d["bytes"] / (d["ms"] * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4))
    roof["kernel"] = dom
    roof["avg_launch_ms"] = round(d["ms"] / max(d["launches"], 1), 4)
    rec = counter_record("traffic", dom, tag)
    roof["traffic"] = None if rec is None else rec["hbm_bytes_per_launch"]
    return roof


def kernel_class(name):
    for key, cls, per in KERNEL_CLASSES:
        if key in name:
            return cls, per
    return None, 1


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--tokens", type=int, default=None, help="override the token count (default 8192)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="token sample of the oracle baseline (default: 3072 for the layer set, all 4096 for the "
                         "square layer, 2048 for the MLP projection)")
    ap.add_argument("--profile-steps", type=int, default=3)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with one plain copy kernel of %d MiB (read and write) for counter calibration"
                         % (CALIBRATION_BYTES >> 20))
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of "
                         "'bench.py --calibrate-copy' into profiles/traffic_<class>.json")
    ap.add_argument("--mfma-from", metavar="PMC_DIR",
                    help="no GPU: turn a rocprofv3 --pmc run of %s into profiles/mfma_<class>.json"
                         % " ".join(MFMA_COUNTERS))
    ap.add_argument("--kernel-stats", metavar="CSV",
                    help="no GPU: summarize by kernel class a rocprofv3 kernel_stats.csv (whole run) or a "
                         "kernel_trace.csv (only the marked, serialized per-kernel timing pass)")
    ap.add_argument("--concurrency-from", metavar="CSV",
                    help="no GPU: from a rocprofv3 kernel_trace.csv of a run with --steps K, the last K timed "
                         "steps before the marked pass: how much of the step has 0, 1, 2, ... weight GEMMs running")
    ap.add_argument("--workload", choices=("layerset", "square", "mlp7b", "stack24"), default="layerset",
                    help="layerset: fwd+bwd of the LLaMA-1B layer set (default); square: the 2048x2048 layer, b=256, "
                         "4096 tokens; mlp7b: the LLaMA-7B MLP projection 11008x4096, 8192 tokens, block size --b; "
                         "stack24: one training step of the 24-layer stack with Adam and the global merge")
    ap.add_argument("--b", type=int, default=None,
                    help="block size of --workload mlp7b (64, 128, 256 or 512; default 512)")
    ap.add_argument("--streams", type=int, default=3,
                    help="HIP streams the seven independent matrices are spread over (batched mode)")
    ap.add_argument("--merge", choices=["sets", "layers"], default="sets",
                    help="stack24: each merge stream's matrices in one batched merge call, or one call per matrix")
    ap.add_argument("--chain", choices=["batched", "per-matrix"], default="batched",
                    help="layer set: one chain-rule call for all matrices after the backward pass, or one per "
                         "matrix on its stream")
    ap.add_argument("--w0-int8", action="store_true",
                    help="layer set: base weights stored as per-row INT8 codes and scales (POET-XQ), turned "
                         "into bf16 inside the GEMMs")
    ap.add_argument("--plain-w0", action="store_true",
                    help="bf16 base weights as W0p alone; by default W0p also holds its transpose "
                         "(POETX_W0_TRANSPOSED, 2 more bytes per weight), which the forward products and their "
                         "recompute read as NN GEMMs (bit-identical results)")
    ap.add_argument("--x-permuted", action="store_true",
                    help="layer set: each matrix's input gathered into the working layout once per step "
                         "(poetx_permute_input, on a stream of its own while the forward blocks are built) and "
                         "kept for the backward pass instead of X (POETX_X_PERMUTED; bit-identical results; "
                         "one N*n*2-byte buffer per matrix)")
    ap.add_argument("--bwd-build", choices=["after-fwd", "beside-fwd"], default="beside-fwd",
                    help="when the backward pass's Cayley build starts on its own stream: once the forward "
                         "build is done (after-fwd), or at once, enqueued after the forward build so that it "
                         "takes the CUs the forward build leaves idle (beside-fwd)")
    ap.add_argument("--stack-fwd-builds", choices=["per-layer", "whole"], default="per-layer",
                    help="stack24: the forward blocks built one decoder layer at a time on a side stream, "
                         "each layer's matrices waiting for their own build (per-layer), or all 168 matrices' "
                         "in one build before the forward pass (whole)")
    ap.add_argument("--keep-z2", action="store_true",
                    help="layer set: the variant without activation recompute (the forward keeps z2' for the "
                         "backward, N*m*2 bytes per matrix); the default recomputes it (POET-Xmem)")
    ap.add_argument("--per-layer-builds", action="store_true",
                    help="let every forward / backward call build its own blocks (one builder launch per call) "
                         "instead of one batched build per pass")
    args = ap.parse_args()
    args.w0_transposed = not (args.plain_w0 or args.w0_int8)
    return args


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "orthogonal_reparameterized_poetx_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _find_csv(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise SystemExit("no *%s under %s" % (suffix, d))


def _pmc_per_dispatch(d, counter):
    """{dispatch id: (kernel name, counter value)} from a rocprofv3 counter_collection.csv."""
    import csv
    out = {}
    with open(_find_csv(d, "counter_collection.csv")) as fh:
        for row in csv.DictReader(fh):
            if row.get("Counter_Name") != counter:
                continue
            did = int(row["Dispatch_Id"])
            name, val = out.get(did, (row["Kernel_Name"], 0.0))
            out[did] = (name, val + float(row["Counter_Value"]))
    return out


def _marked(names):
    """Dispatch ids strictly between the last two marker kernels (sigmoid)
    that bracket the serialized per-kernel pass, from {dispatch id: name};
    every id when the run has no markers."""
    marks = sorted(d for d, n in names.items() if "sigmoid" in n)
    if len(marks) < 2:
        return set(names)
    lo, hi = marks[-2], marks[-1]
    return {d for d in names if lo < d < hi}


def traffic_from(fetch_dir, write_dir):
    """HBM bytes per launch of every kernel class, from FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch) scaled by what they read for the calibration copy."""
    fetch = _pmc_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_dir, "WRITE_SIZE")

    def calib(tab):
        cand = [v for n, v in tab.values() if "neg" in n.lower()]
        if not cand:
            raise SystemExit("calibration copy kernel not found")
        return CALIBRATION_BYTES / (cand[-1] * 1024.0)
    kf, kw = calib(fetch), calib(write)
    agg = {}
    for tab, k, key in ((fetch, kf, "fetch"), (write, kw, "write")):
        keep = _marked({d: nv[0] for d, nv in tab.items()})
        for did, (name, v) in tab.items():
            if did not in keep:
                continue
            cls, per = kernel_class(name)
            if cls is None:
                continue
            a = agg.setdefault(cls, dict(fetch=0.0, write=0.0, dispatches_fetch=0, dispatches_write=0, per=per,
                                         kernels=set()))
            a[key] += v * 1024.0 * k
            a["dispatches_" + key] += 1
            a["kernels"].add(name.split("(")[0])
    src_files = SOURCE_FILES
    h = kernel_source_hash(src_files)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for cls, a in agg.items():
        launches_f = a["dispatches_fetch"] / a["per"]
        launches_w = a["dispatches_write"] / a["per"]
        rec = dict(kernel_class=cls, workload=profiled_run_tag(), source_hash=h, source_files=src_files,
                   hbm_bytes_per_launch=round(a["fetch"] / launches_f + a["write"] / launches_w),
                   fetch_bytes_per_launch=round(a["fetch"] / launches_f),
                   write_bytes_per_launch=round(a["write"] / launches_w),
                   launches=launches_f, calibration=dict(fetch_scale=round(kf, 4), write_scale=round(kw, 4),
                                                         copy_bytes=CALIBRATION_BYTES),
                   kernels=sorted(a["kernels"]))
        with open(os.path.join(ROOT, "profiles", "traffic_%s.json" % cls), "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        print("%-18s %12.0f B/launch (fetch %.0f, write %.0f) over %d launches"
              % (cls, rec["hbm_bytes_per_launch"], rec["fetch_bytes_per_launch"], rec["write_bytes_per_launch"],
                 launches_f))


def mfma_from(d):
    """Per-class MFMA counters from one rocprofv3 --pmc run of MFMA_COUNTERS:
    bf16 MFMA flops per launch (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts units of
    512 flops) and the MFMA pipes' busy fraction over the cycles the compute
    units ran the kernel: (SQ_VALU_MFMA_BUSY_CYCLES / SIMD_COUNT) /
    (SQ_BUSY_CU_CYCLES / CU_COUNT).  GRBM_GUI_ACTIVE is recorded but not used:
    under counter collection it also counts the collection's own time around
    each dispatch.  Writes profiles/mfma_<class>.json."""
    import csv
    per = {}
    with open(_find_csv(d, "counter_collection.csv")) as fh:
        for row in csv.DictReader(fh):
            c = row.get("Counter_Name")
            if c not in MFMA_COUNTERS:
                continue
            did = int(row["Dispatch_Id"])
            e = per.setdefault(did, dict(name=row["Kernel_Name"]))
            v = float(row["Counter_Value"])
            e[c] = max(e.get(c, 0.0), v) if c == "GRBM_GUI_ACTIVE" else e.get(c, 0.0) + v
    agg = {}
    keep = _marked({d: e["name"] for d, e in per.items()})
    for did, e in per.items():
        if did not in keep:
            continue
        cls, k = kernel_class(e["name"])
        if cls is None:
            continue
        a = agg.setdefault(cls, dict(mops=0.0, busy=0.0, cu=0.0, dispatches=0, per=k, kernels=set()))
        a["mops"] += e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        a["busy"] += e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        a["cu"] += e.get("SQ_BUSY_CU_CYCLES", 0.0)
        a["dispatches"] += 1
        a["kernels"].add(e["name"].split("(")[0])
    h = kernel_source_hash(SOURCE_FILES)
    for cls, a in agg.items():
        launches = a["dispatches"] / a["per"]
        rec = dict(kernel_class=cls, workload=profiled_run_tag(), source_hash=h, source_files=SOURCE_FILES,
                   launches=launches,
                   mfma_flops_per_launch=round(a["mops"] * 512 / launches),
                   mfma_busy_frac=round((a["busy"] / SIMD_COUNT) / (a["cu"] / CU_COUNT), 4) if a["cu"] > 0 else None,
                   cu_busy_cycles_per_launch=round(a["cu"] / CU_COUNT / launches),
                   counters=list(MFMA_COUNTERS), kernels=sorted(a["kernels"]))
        with open(os.path.join(ROOT, "profiles", "mfma_%s.json" % cls), "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        print("%-18s %14.4g bf16 MFMA flops/launch, MFMA busy %s over %d launches"
              % (cls, rec["mfma_flops_per_launch"], rec["mfma_busy_frac"], launches))


def run_tag(workload, tokens, w0_int8=False, keep_z2=False, w0_transposed=False, x_permuted=False):
    """Names the run a counter record was taken on: workload, tokens and variant."""
    w = "INT8" if w0_int8 else "bf16 + transposed" if w0_transposed else "bf16"
    return "%s, %d tokens (%s weights, activations %s%s)" % (workload, tokens, w, "kept" if keep_z2 else "recomputed",
                                                            ", inputs gathered once" if x_permuted else "")


def profiled_run_tag():
    """The run the committed counter records come from: bench.py's default
    (the layer set, bf16 weights with the transposed copy, recompute)."""
    import workloads as WL
    return run_tag(WL.CONFIGS[3]["name"], WL.CONFIGS[3]["N"], w0_transposed=True)


def counter_record(kind, cls, tag):
    """A committed counter record (traffic or mfma) of class cls taken on the
    run named tag, whose kernel-source hash still matches the sources."""
    path = os.path.join(ROOT, "profiles", "%s_%s.json" % (kind, cls))
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != kernel_source_hash(rec.get("source_files", [])):
        return None
    if rec.get("workload") != tag:
        return None
    return rec


def _trace_window(path, steps):
    """kernel_stats-like rows from a rocprofv3 kernel_trace.csv, restricted to
    the launches between the two marker kernels (sigmoid) that bracket the
    serialized per-kernel timing pass; durations divided into per-step
    figures by ``steps``."""
    import csv
    rows = list(csv.DictReader(open(path)))
    marks = [r for r in rows if "sigmoid" in r["Kernel_Name"]]
    if len(marks) < 2:
        raise SystemExit("marker kernels not found in %s" % path)
    t0, t1 = int(marks[-2]["End_Timestamp"]), int(marks[-1]["Start_Timestamp"])
    agg = {}
    for r in rows:
        if int(r["Start_Timestamp"]) >= t0 and int(r["End_Timestamp"]) <= t1:
            a = agg.setdefault(r["Kernel_Name"], [0, 0.0])
            a[0] += 1
            a[1] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return [dict(Name=k, Calls=str(v[0]), TotalDurationNs=str(v[1]), AverageNs=str(v[1] / v[0]))
            for k, v in agg.items()]


def kernel_stats(path, steps=None):
    """Per-class totals of a rocprofv3 kernel_stats.csv, or of the marked
    per-kernel timing window of a kernel_trace.csv (durations in ns)."""
    import csv
    agg = {}
    rows = _trace_window(path, steps) if path.endswith("kernel_trace.csv") else list(csv.DictReader(open(path)))
    for row in rows:
        cls, per = kernel_class(row["Name"])
        cls = cls or "other"
        a = agg.setdefault(cls, [0, 0.0, per])
        a[0] += int(row["Calls"])
        a[1] += float(row["TotalDurationNs"])
    print("%-18s %8s %14s %14s" % ("class", "launches", "total_ms", "avg_ms/launch"))
    for cls, (calls, tot, per) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        n = calls / per
        print("%-18s %8.0f %14.3f %14.4f" % (cls, n, tot * 1e-6, tot * 1e-6 / max(n, 1)))
    print()
    print("%-60s %7s %12s %12s" % ("kernel", "calls", "total_ms", "avg_ms"))
    for row in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        print("%-60s %7s %12.3f %12.4f" % (row["Name"].split("(")[0][:60], row["Calls"],
                                           float(row["TotalDurationNs"]) * 1e-6, float(row["AverageNs"]) * 1e-6))


# ---------------------------------------------------------------------------
# 24-layer stack of layer-set shapes: one training step over 168 matrices
# ---------------------------------------------------------------------------
class Stack:
    """The 24-layer stack resident in HBM: bf16 (or INT8, w0_int8) W0p per matrix in its working
    layout, all generators (and their gradients and Adam moments) in single
    fp32 buffers so the optimizer step is one launch, and per-matrix inputs,
    upstream gradients and outputs.

    Matrices listed in ``exact`` (and every matrix sharing their input) take
    their values from the shared numpy recipe of ``workloads`` so the oracle
    can check them; the rest draw the same distributions on the device from a
    torch generator seeded by (config, matrix, stream)."""

    def __init__(self, P, WL, torch, dev, N, nlayers=24, exact=(), streams=3, w0_int8=False, merge="sets",
                 w0_transposed=False, fwd_builds="per-layer"):
        import math
        import numpy as np
        self.P, self.torch, self.N = P, torch, N
        cfg = WL.CONFIGS[5]
        b = cfg["b"]
        nt = b * (b - 1) // 2
        mats = [(l, idx, m, n) for l in range(nlayers) for idx, (_, m, n) in enumerate(cfg["mats"])]
        total = sum(m // b + n // b for _, _, m, n in mats) * nt
        f32 = torch.float32
        self.theta = torch.zeros(total, dtype=f32, device=dev)
        self.grad = torch.zeros_like(self.theta)
        self.m1 = torch.zeros_like(self.theta)
        self.v1 = torch.zeros_like(self.theta)
        gen = torch.Generator(device=dev)

        def drawn(c, j, s, shape, var, dt):
            gen.manual_seed((c << 40) | (j << 8) | s)
            return (torch.randn(shape, generator=gen, device=dev, dtype=f32) * math.sqrt(var)).to(dt)

        def up(pair, dt):
            a = np.ascontiguousarray(pair[0])
            if dt == torch.bfloat16:
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(a.astype(np.float32)).to(dev)

        exact_owners = {WL.input_owner(cfg, j) for j in exact}
        # matrices run on `streams` streams (matrix i on stream where[i]);
        # each stream has its own workspace pool, shared by the matrices that
        # run on it one after another (never by two streams)
        self.nstreams = max(int(streams), 1)
        self.where = balance_streams([(m, n) for _, _, m, n in mats], N, self.nstreams)
        pools = [{} for _ in range(self.nstreams)]
        self.layers, self.X, self.gY, self.out = [], {}, [], []
        mats_done = []
        off = 0
        bf = torch.bfloat16
        for l, idx, m, n in mats:
            j = 7 * l + idx
            lay = P.PoetxLayer(m, n, b, "bf16", dev, perm_seed=WL.perm_seed(5, j),
                               ws_pool=pools[self.where[len(mats_done)]], w0_int8=w0_int8,
                               w0_transposed=w0_transposed)
            mats_done.append(j)
            kR, kP = m // b, n // b
            lay.thR = self.theta[off:off + kR * nt].view(kR, nt)
            lay.dR = self.grad[off:off + kR * nt].view(kR, nt)
            off += kR * nt
            lay.thP = self.theta[off:off + kP * nt].view(kP, nt)
            lay.dP = self.grad[off:off + kP * nt].view(kP, nt)
            off += kP * nt
            owner = WL.input_owner(cfg, j)
            if j in exact:
                inp = WL.matrix_inputs(5, j, N=N)
                lay.pack(up(inp["W0"], bf))
                lay.thR.copy_(up(inp["thR"], f32))
                lay.thP.copy_(up(inp["thP"], f32))
                gy = up(inp["gY"], bf)
            else:
                lay.pack(drawn(5, j, 1, (m, n), cfg["w_var"], bf))
                lay.thR.copy_(drawn(5, j, 2, (kR, nt), cfg["theta_var"], f32))
                lay.thP.copy_(drawn(5, j, 3, (kP, nt), cfg["theta_var"], f32))
                gy = drawn(5, j, 5, (N, m), 1.0, bf)
            if owner not in self.X:
                if owner in exact_owners:
                    self.X[owner] = up(WL.stored(WL.gaussian(5, owner, 4, (N, n), 1.0), "bf16"), bf)
                else:
                    self.X[owner] = drawn(5, owner, 4, (N, n), 1.0, bf)
            lay.x_key = owner
            lay.j = j
            self.layers.append(lay)
            self.gY.append(gy)
            self.out.append(dict(Y=torch.empty(N, m, dtype=bf, device=dev), dX=torch.empty(N, n, dtype=bf, device=dev)))
        for lay in self.layers:
            for kind in ("forward", "backward", "merge"):
                lay.block_buffers(kind)
            lay.workspace(P.OP_FORWARD_BLOCKS, N)
            lay.workspace(P.OP_BACKWARD_DQ, N)
            lay.dq_buffers()
        # the merges run on the worker streams and the side stream (idle
        # while they run; the merge is a chain of short launches per matrix,
        # so a fourth queue adds overlap), balanced by m n, each stream with
        # its own merge workspace
        self.nmerge = self.nstreams + 1
        self.mwhere = balance_streams([(m, n) for _, _, m, n in mats], N, self.nmerge, "merge")
        need = [1] * self.nmerge
        for i, lay in enumerate(self.layers):
            need[self.mwhere[i]] = max(need[self.mwhere[i]], lay.workspace_need(P.OP_MERGE_BLOCKS))
        # merge="sets": each stream merges its matrices with one batched call
        # (poetx_merge_blocks_sets: the launches after the block products are
        # shared); "layers": one poetx_merge_blocks call per matrix
        self.merge_mode = merge
        self.mgroups = [[lay for i, lay in enumerate(self.layers) if self.mwhere[i] == k] for k in range(self.nmerge)]
        if merge == "sets":
            need = [max(P.merge_sets_workspace_need(g), 1) for g in self.mgroups]
        self.merge_ws = [P.make_workspace(x, dev) for x in need]
        self.adam_steps = 0
        self.fwd_builds = fwd_builds

    def _fan_out(self, main, idx_items, fn):
        for w in self.workers[1:]:
            w.wait_stream(main)
        for i, item in idx_items:
            with self.torch.cuda.stream(self.workers[self.where[i]]):
                fn(*item)
        for w in self.workers[1:]:
            main.wait_stream(w)

    def _streams(self, main):
        if not hasattr(self, "side"):
            self.side = self.torch.cuda.Stream()      # all streams at the default priority
            self.bwd_ready = self.torch.cuda.Event()
            self.workers = [main] + [self.torch.cuda.Stream() for _ in range(self.nstreams - 1)]

    def forward_backward(self):
        P, torch = self.P, self.torch
        main = torch.cuda.current_stream()
        self._streams(main)
        n = len(self.layers)
        if self.fwd_builds == "per-layer":
            # the forward blocks of the first decoder layer now, those of each
            # later one (seven matrices, 154 blocks) on the side stream while
            # the layers before it run their forward pass: a matrix waits
            # only for its own layer's build
            groups = {}
            for lay in self.layers:
                groups.setdefault(lay.j // 7, []).append(lay)
            order = sorted(groups)
            if not hasattr(self, "fwd_ready"):
                self.fwd_ready = {l: torch.cuda.Event() for l in order}
            P.build_layer_blocks(groups[order[0]], "forward")
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                for l in order[1:]:
                    P.build_layer_blocks(groups[l], "forward")
                    self.fwd_ready[l].record(self.side)
        else:
            P.build_layer_blocks(self.layers, "forward")
            self.side.wait_stream(main)
        # the backward blocks depend only on the generators: build them on the
        # side stream while the forward pass runs
        with torch.cuda.stream(self.side):
            P.build_layer_blocks(self.layers, "backward")
            self.bwd_ready.record(self.side)

        def fwd(lay, o):
            if self.fwd_builds == "per-layer" and lay.j // 7 != order[0]:
                torch.cuda.current_stream().wait_event(self.fwd_ready[lay.j // 7])
            lay.forward_blocks(self.X[lay.x_key], Y=o["Y"])
        self._fan_out(main, [(i, (self.layers[i], self.out[i])) for i in range(n)], fwd)
        main.wait_event(self.bwd_ready)
        self._fan_out(main, [(i, (self.layers[i], self.gY[i], self.out[i])) for i in reversed(range(n))],
                      lambda lay, g, o: lay.backward_blocks_dq(self.X[lay.x_key], g, dX=o["dX"]))
        P.chain_rule_layers(self.layers, [(lay.dR, lay.dP) for lay in self.layers])

    def adam(self):
        self.adam_steps += 1
        self.P.poetx_adam_step(self.theta, self.grad, self.m1, self.v1, self.theta.numel(), self.adam_steps)

    def merge(self):
        self.P.build_layer_blocks(self.layers, "merge")
        main = self.torch.cuda.current_stream()
        self._streams(main)
        ms = self.workers + [self.side]
        for w in ms[1:]:
            w.wait_stream(main)
        if self.merge_mode == "sets":
            for k, g in enumerate(self.mgroups):
                if g:
                    with self.torch.cuda.stream(ms[k]):
                        self.P.merge_layers_sets(g, ws=self.merge_ws[k])
        else:
            for i, lay in enumerate(self.layers):
                k = self.mwhere[i]
                with self.torch.cuda.stream(ms[k]):
                    lay.merge_blocks(ws=self.merge_ws[k])
        for w in ms[1:]:
            main.wait_stream(w)

    def step(self):
        self.forward_backward()
        self.adam()
        self.merge()


def bench_stack(args):
    import torch

    import workloads as WL
    import orthogonal_reparameterized_poetx_amd as P
    dev = "cuda:0"
    torch.cuda.set_device(0)
    N = args.tokens or WL.CONFIGS[5]["N"]
    st = Stack(P, WL, torch, dev, N, streams=args.streams, w0_int8=args.w0_int8, merge=args.merge,
               w0_transposed=args.w0_transposed, fwd_builds=args.stack_fwd_builds)
    torch.cuda.synchronize()
    resident = torch.cuda.memory_allocated()
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        st.step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    fb = mg = ad = 0.0
    for _ in range(args.steps):
        ev[0].record(stream)
        st.forward_backward()
        ev[1].record(stream)
        st.adam()
        ev[2].record(stream)
        st.merge()
        ev[3].record(stream)
        torch.cuda.synchronize()
        fb += ev[0].elapsed_time(ev[1])
        ad += ev[1].elapsed_time(ev[2])
        mg += ev[2].elapsed_time(ev[3])
    k = args.steps
    ms = (fb + ad + mg) / k
    # per-kernel pass: one step with every matrix on the main stream, HIP
    # events around each launch
    saved = (st.workers, st.side)
    st.workers, st.side = [stream] * st.nstreams, stream
    P.timing_enable(True)
    st.step()
    torch.cuda.synchronize()
    kern = P.timing_summary()
    P.timing_enable(False)
    st.workers, st.side = saved
    per_step = {c: dict(v) for c, v in kern.items()}
    roof = dominant_roofline(per_step, run_tag(WL.CONFIGS[5]["name"], N, args.w0_int8,
                                               w0_transposed=args.w0_transposed))
    cpu = None
    if not args.no_cpu:
        # one layer's seven matrices on the oracle; a stack step runs 24 layers
        cpu = cpu_baseline(5, list(range(7)), None, args.cpu_tokens or 1024)
        cpu["value"] = round(cpu["value"] / 24, 3)
        cpu["sample"] += "; the rate is that sample's tokens/s over 24 layers (Adam and merge not included)"
    print(json.dumps({
        "metric": "POET-X 24-layer stack training step (fwd+bwd, Adam, global merge), 1 GPU",
        "value": round(N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": k, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded Gaussian inputs with the stack's shapes)",
        "config": {"workload": WL.CONFIGS[5]["name"], "tokens": N, "matrices": len(st.layers), "b": WL.CONFIGS[5]["b"],
                   "base_weights": "INT8 codes with per-row fp32 scales (POET-XQ)" if args.w0_int8 else
                   "bf16 with a transposed copy (POETX_W0_TRANSPOSED)" if args.w0_transposed else "bf16",
                   "merge": "one batched call per stream" if args.merge == "sets" else "one call per matrix",
                   "forward_builds": "one per decoder layer, beside the forward pass of the layers before it"
                   if args.stack_fwd_builds == "per-layer" else "one for all matrices before the forward pass"},
        "phases_ms": {"fwd_bwd": round(fb / k, 3), "adam": round(ad / k, 3), "merge": round(mg / k, 3)},
        "generators": st.theta.numel(),
        "resident_gb": round(resident / 1e9, 3),
        "peak_hbm_gb": round(torch.cuda.max_memory_allocated() / 1e9, 3),
        "roofline": roof,
        "kernels_per_step": {c: dict(ms=round(v["ms"], 4), launches=v["launches"])
                             for c, v in sorted(per_step.items(), key=lambda kv: -kv[1]["ms"])},
        "cpu_baseline": cpu,
    }), flush=True)


def concurrency_from(csv_path, steps):
    """Weight-GEMM concurrency over the timed steps of a kernel trace: the
    launches from the start of the steps-th last step (each step opens with
    its two Cayley builds) up to the first marker kernel."""
    import csv
    rows = sorted(csv.DictReader(open(csv_path)), key=lambda r: int(r["Start_Timestamp"]))
    names = [r["Kernel_Name"] for r in rows]
    marks = [i for i, nm in enumerate(names) if "sigmoid" in nm.lower()]
    if not marks:
        raise SystemExit("no marker kernels in %s" % csv_path)
    builds = [i for i in range(marks[0]) if "gj_kernel" in names[i]]
    if len(builds) < 2 * steps:
        raise SystemExit("fewer than %d steps before the marked pass" % steps)
    timed = rows[builds[-2 * steps]:marks[0]]
    t0 = int(timed[0]["Start_Timestamp"])
    t1 = max(int(r["End_Timestamp"]) for r in timed)
    ev = []
    for r in timed:
        if "gemm_wide_kernel" in r["Kernel_Name"] or "gemm_bf16_kernel<true, false" in r["Kernel_Name"]:
            ev += [(int(r["Start_Timestamp"]), 1), (int(r["End_Timestamp"]), -1)]
    ev.sort()
    hist, cur, last = {}, 0, t0
    for t, d in ev:
        hist[cur] = hist.get(cur, 0) + t - last
        cur, last = cur + d, t
    hist[cur] = hist.get(cur, 0) + t1 - last
    span = t1 - t0
    print("%d timed steps, %.1f us per step, %d launches" % (steps, span / 1e3 / steps, len(timed)))
    for k in sorted(hist):
        print("weight GEMMs running: %d  %5.1f %% of the time" % (k, 100.0 * hist[k] / span))


def main():
    args = parse()
    if args.workload == "stack24":
        if args.x_permuted:
            print("--x-permuted applies to the single-step workloads (layerset, square, mlp7b)", file=sys.stderr)
            sys.exit(2)
        if args.gpus != 1:
            print("bench.py measures one GPU. Run with --gpus 1.", file=sys.stderr)
            sys.exit(2)
        bench_stack(args)
        return
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.kernel_stats:
        kernel_stats(args.kernel_stats)
        return
    if args.concurrency_from:
        concurrency_from(args.concurrency_from, args.steps)
        return
    if args.mfma_from:
        mfma_from(args.mfma_from)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (every box has one GPU). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import workloads as WL
    import orthogonal_reparameterized_poetx_amd as P

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    if (args.keep_z2 or args.x_permuted) and args.per_layer_builds:
        print("--keep-z2 and --x-permuted use the prebuilt-block calls; drop --per-layer-builds", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    # (config number, matrix indices, block size) of the workload
    if args.workload == "square":
        c, mats, b_over = 2, [0], None
    elif args.workload == "mlp7b":
        c, mats, b_over = 4, [0], args.b or WL.CONFIGS[4]["b"]
        if b_over not in WL.C4_BLOCK_SIZES:
            print("--b must be one of %s" % (WL.C4_BLOCK_SIZES,), file=sys.stderr)
            sys.exit(2)
    else:
        c, mats, b_over = 3, list(range(len(WL.CONFIGS[3]["mats"]))), None
    cfg = WL.CONFIGS[c]
    N = args.tokens or cfg["N"]

    def up(pair, dt):
        a = np.ascontiguousarray(pair[0])
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a.astype(np.float32)).to(dev)

    # ---- resident inputs: seven packed layers, their inputs and upstream grads
    layers, Xs, gYs, outs = [], {}, [], []
    for j in mats:
        inp = WL.matrix_inputs(c, j, N=N, b=b_over)
        lay = P.PoetxLayer(inp["m"], inp["n"], inp["b"], "bf16", dev, perm_seed=inp["perm_seed"],
                           w0_int8=args.w0_int8, w0_transposed=args.w0_transposed,
                           x_permuted=args.x_permuted)
        lay.pack(up(inp["W0"], "bf16"))
        lay.thR.copy_(up(inp["thR"], "f32"))
        lay.thP.copy_(up(inp["thP"], "f32"))
        owner = WL.input_owner(cfg, j)
        if owner not in Xs:
            Xs[owner] = up(inp["X"], "bf16")
        lay.x_key = owner
        # the matrix's input in its working layout (--x-permuted)
        lay.xp = torch.empty(N, inp["n"], dtype=torch.bfloat16, device=dev) if args.x_permuted else None
        gYs.append(up(inp["gY"], "bf16"))
        outs.append(dict(Y=torch.empty(N, inp["m"], dtype=torch.bfloat16, device=dev),
                         dX=torch.empty(N, inp["n"], dtype=torch.bfloat16, device=dev),
                         dR=torch.empty_like(lay.thR), dP=torch.empty_like(lay.thP),
                         Z2=torch.empty(N, inp["m"], dtype=torch.bfloat16, device=dev) if args.keep_z2 else None))
        layers.append(lay)
        # allocate workspaces and block buffers up front (nothing is allocated in the timed region)
        if args.per_layer_builds:
            lay.workspace(P.OP_FORWARD, N)
            lay.workspace(P.OP_BACKWARD, N)
        else:
            lay.workspace(P.OP_FORWARD_BLOCKS, N)
            lay.workspace(P.OP_BACKWARD_DQ, N)
            lay.block_buffers("forward")
            lay.block_buffers("backward")
            lay.dq_buffers()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step_per_layer():
        for lay, o in zip(layers, outs):
            lay.forward(Xs[lay.x_key], Y=o["Y"])
        for lay, g, o in zip(reversed(layers), reversed(gYs), reversed(outs)):
            lay.backward(Xs[lay.x_key], g, dX=o["dX"], dthR=o["dR"], dthP=o["dP"])

    side = torch.cuda.Stream()          # default priority
    bwd_blocks_ready = torch.cuda.Event()
    # the seven matrices are independent given their inputs: spread them over
    # streams (all at the default priority), balanced by estimated cost, so one
    # matrix's kernel tails and small launches overlap another's work
    workers = [stream] + [torch.cuda.Stream() for _ in range(max(args.streams, 1) - 1)]

    gather = torch.cuda.Stream()        # default priority
    inputs_ready, step_start = torch.cuda.Event(), torch.cuda.Event()
    active = {"workers": workers, "side": side, "gather": gather}

    where = {len(workers): balance_streams([(lay.m, lay.n) for lay in layers], N, len(workers)), 1: [0] * len(layers)}

    def fan_out(items, fn):
        ws = active["workers"]
        for w in ws[1:]:
            w.wait_stream(stream)
        for item in items:
            with torch.cuda.stream(ws[where[len(ws)][layers.index(item[0])]]):
                fn(*item)
        for w in ws[1:]:
            stream.wait_stream(w)

    def step_batched():
        # blocks of all seven matrices in one build per pass; the backward pass
        # rebuilds them from the generators instead of keeping the forward's
        # (on a second stream, concurrently with the forward pass: the build
        # needs only the generators); the chain rule runs once for all seven
        # after their dL/dQ (--chain batched) or per matrix on its stream
        # right after its dL/dQ (--chain per-matrix)
        bs = active["side"]
        gs = active["gather"]
        if (args.x_permuted and gs is not stream) or (args.bwd_build == "beside-fwd" and bs is not stream):
            step_start.record(stream)
        # the backward build starts at once (--bwd-build beside-fwd),
        # enqueued after the forward build so that the forward build's
        # workgroups take their CUs first and the backward build's fill the
        # CUs it leaves idle (it has one workgroup per block, 154 for the
        # layer set), its last ones running beside the forward pass's first
        # kernels; or once the forward build is done (after-fwd)
        P.build_layer_blocks(layers, "forward")
        if args.x_permuted:
            # the inputs' gathers need no blocks: they run beside the forward
            # build, on the CUs it leaves idle (enqueued after it, so that the
            # build's workgroups take their CUs first)
            if gs is not stream:
                gs.wait_event(step_start)
            with torch.cuda.stream(gs):
                for lay in layers:
                    lay.permute_input(Xs[lay.x_key], Xp=lay.xp)
                inputs_ready.record(gs)
        if args.bwd_build == "beside-fwd" and bs is not stream:
            bs.wait_event(step_start)
        else:
            bs.wait_stream(stream)
        with torch.cuda.stream(bs):
            P.build_layer_blocks(layers, "backward")
            bwd_blocks_ready.record(bs)
        if args.x_permuted:
            stream.wait_event(inputs_ready)
        xin = (lambda lay: lay.xp) if args.x_permuted else (lambda lay: Xs[lay.x_key])
        if args.keep_z2:
            fan_out(list(zip(layers, outs)),
                    lambda lay, o: lay.forward_blocks_z2(xin(lay), Y=o["Y"], Z2=o["Z2"]))
        else:
            fan_out(list(zip(layers, outs)), lambda lay, o: lay.forward_blocks(xin(lay), Y=o["Y"]))
        stream.wait_event(bwd_blocks_ready)
        def bwd(lay, g, o):
            if args.keep_z2:
                lay.backward_blocks_dq_z2(xin(lay), g, o["Z2"], dX=o["dX"])
            else:
                lay.backward_blocks_dq(xin(lay), g, dX=o["dX"])
            if args.chain == "per-matrix":
                P.chain_rule_layers([lay], [(o["dR"], o["dP"])])
        fan_out(list(zip(reversed(layers), reversed(gYs), reversed(outs))), bwd)
        if args.chain == "batched":
            P.chain_rule_layers(layers, [(o["dR"], o["dP"]) for o in outs])

    step = step_per_layer if args.per_layer_builds else step_batched

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps

    # ---- per-kernel breakdown: a separate pass with events around every
    # launch, with the matrices serialized on one stream so that every launch
    # has the GPU to itself (its duration then measures the kernel, not its
    # neighbours).  Two marker kernels (sigmoid on a 1-element tensor)
    # bracket the pass so that a profiler trace can pick out its launches.
    marker = torch.zeros(1, device=dev)
    torch.cuda.synchronize()
    torch.sigmoid_(marker)
    torch.cuda.synchronize()
    active["workers"], active["side"], active["gather"] = [stream], stream, stream
    P.timing_enable(True)
    for _ in range(args.profile_steps):
        step()
    torch.cuda.synchronize()
    kern = P.timing_summary()
    P.timing_enable(False)
    active["workers"], active["side"], active["gather"] = workers, side, gather
    torch.sigmoid_(marker)
    torch.cuda.synchronize()
    per_step = {k: dict(v, ms=v["ms"] / args.profile_steps, launches=v["launches"] / args.profile_steps,
                        flops=v["flops"] / args.profile_steps, bytes=v["bytes"] / args.profile_steps)
                for k, v in kern.items()}
    tag = run_tag(cfg["name"] if b_over is None else "%s_b%d" % (cfg["name"], b_over), N, args.w0_int8,
                  args.keep_z2, args.w0_transposed, args.x_permuted)
    roof = dominant_roofline(per_step, tag)
    # every class against its own roofline (kernel level: the bytes or flops
    # each launch must move or compute, over its event-timed duration)
    classes = {}
    for k, v in per_step.items():
        if v["ms"] <= 0:
            continue
        if k in MFMA_CLASSES and v["flops"] > 0:
            a = v["flops"] / (v["ms"] * 1e-3) / 1e12
            classes[k] = dict(bound="mfma", achieved=round(a, 1), peak=MFMA_CLASSES[k], unit="TFLOP/s",
                              frac=round(a / MFMA_CLASSES[k], 4))
        elif k in HBM_CLASSES and v["bytes"] > 0:
            a = v["bytes"] / (v["ms"] * 1e-3) / 1e9
            classes[k] = dict(bound="hbm", achieved=round(a, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(a / PEAK_HBM_GBS, 4))
    # method level: the block transforms' algorithmic bytes per step (per token
    # and matrix: forward 4(n+m), backward 6(m+n), recompute 4n, bf16) over the
    # time of every transform kernel (permutations, block products, Gram
    # products) in the serialized pass
    shapes = [(cfg["mats"][j % len(cfg["mats"])][1], cfg["mats"][j % len(cfg["mats"])][2]) for j in mats]
    algo = N * sum(10 * (m + n) + 4 * n for m, n in shapes)
    xms = sum(per_step[k]["ms"] for k in HBM_CLASSES if k in per_step)
    transforms = dict(algorithmic_bytes=algo, ms=round(xms, 4),
                      achieved=round(algo / (xms * 1e-3) / 1e9, 1) if xms > 0 else None, peak=PEAK_HBM_GBS,
                      unit="GB/s", frac=round(algo / (xms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if xms > 0 else None,
                      classes=[k for k in HBM_CLASSES if k in per_step])
    gms = sum(per_step[k]["ms"] for k in GEMM_CLASSES if k in per_step)
    gfl = sum(per_step[k]["flops"] for k in GEMM_CLASSES if k in per_step)
    gemms = dict(flops=gfl, ms=round(gms, 4), achieved=round(gfl / (gms * 1e-3) / 1e12, 1) if gms > 0 else None,
                 peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                 frac=round(gfl / (gms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4) if gms > 0 else None)
    # the same fractions from rocprofv3 counters (records under profiles/ taken
    # on the layer set with the current sources): bf16 MFMA flops the
    # hardware counted, and HBM bytes (FETCH_SIZE + WRITE_SIZE), per launch,
    # over the event-timed launch duration of this run
    counters = {}
    for k, v in per_step.items():
        if v["launches"] <= 0 or v["ms"] <= 0:
            continue
        avg_s = v["ms"] / v["launches"] * 1e-3
        mf = counter_record("mfma", k, tag) if k in GEMM_CLASSES else None
        if mf:
            a = mf["mfma_flops_per_launch"] / avg_s / 1e12
            counters[k] = dict(bound="mfma", achieved=round(a, 1), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                               frac=round(a / PEAK_BF16_TFLOPS, 4), mfma_busy=mf["mfma_busy_frac"],
                               clock_ghz=round(mf["cu_busy_cycles_per_launch"] / avg_s / 1e9, 3))
        tr = counter_record("traffic", k, tag) if k in HBM_CLASSES else None
        if tr:
            a = tr["hbm_bytes_per_launch"] / avg_s / 1e9
            counters[k] = dict(bound="hbm", achieved=round(a, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                               frac=round(a / PEAK_HBM_GBS, 4))
    breakdown = {}
    for k, v in sorted(per_step.items(), key=lambda kv: -kv[1]["ms"]):
        e = dict(ms=round(v["ms"], 4), launches=round(v["launches"], 2))
        if v["flops"] > 0:
            e["tflops"] = round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 1)
        if v["bytes"] > 0:
            e["gbs"] = round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1)
        breakdown[k] = e

    # ---- merge of the whole layer set (periodic: not part of a step)
    for lay in layers:
        lay.workspace(P.OP_MERGE)
    torch.cuda.synchronize()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record(stream)
    for lay in layers:
        lay.merge()
    e3.record(stream)
    torch.cuda.synchronize()
    merge_ms = e2.elapsed_time(e3)

    result = {
        "metric": "POET-X layer fwd+bwd tokens/sec and % of MFMA/HBM roofline, 1 GPU",
        "value": round(N / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian inputs with the workload's shapes)",
        "config": {"workload": cfg["name"] if b_over is None else "%s_b%d" % (cfg["name"], b_over),
                   "tokens": N, "matrices": len(mats), "b": b_over or cfg["b"],
                   "shapes": ["%dx%d" % s for s in shapes],
                   "block_builds": "per layer call" if args.per_layer_builds else
                   "batched per pass (Cayley builds and chain rule over all matrices)",
                   "streams": 1 if args.per_layer_builds else max(args.streams, 1),
                   "activations": "z2' kept from the forward pass (no recompute)" if args.keep_z2 else
                   "recomputed in the backward pass (POET-Xmem)",
                   "inputs": "gathered into the working layout once per step beside the forward build and kept "
                   "for the backward pass (POETX_X_PERMUTED)" if args.x_permuted else
                   "gathered by every forward and backward call",
                   "base_weights": "INT8 codes with per-row fp32 scales, dequantized inside the GEMMs "
                   "(POET-XQ)" if args.w0_int8 else "bf16 with a transposed copy (POETX_W0_TRANSPOSED)"
                   if args.w0_transposed else "bf16"},
        "roofline": roof,
        "roofline_classes": classes,
        "roofline_gemms": gemms,
        "roofline_transforms": transforms,
        "roofline_counters": counters or None,
        "kernels_per_step": breakdown,
        "merge_ms": round(merge_ms, 3),
    }

    if args.calibrate_copy:
        # one plain copy kernel of known size: reads and writes CALIBRATION_BYTES
        src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()

    # ---- float64 oracle on the host cores, bounded token sample
    if not args.no_cpu:
        ntok = args.cpu_tokens or {"square": 4096, "mlp7b": 2048}.get(args.workload, 3072)
        result["cpu_baseline"] = cpu_baseline(c, mats, b_over, ntok)
    print(json.dumps(result), flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(c, mats, b_over, ntok):
    """The float64 oracle (bf16 contract mode) on the host cores: forward and
    backward of the workload's matrices on its first ntok tokens."""
    import numpy as np

    import oracle
    import workloads as WL
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = None
    cfg = WL.CONFIGS[c]
    ntok = min(ntok, cfg["N"])
    rows = np.arange(ntok)
    # time only the oracle calls (input generation excluded)
    tot = 0.0
    for j in mats:
        inp = WL.matrix_inputs(c, j, rows=rows, b=b_over)
        s = oracle.make_permutation(inp["perm_seed"], 0, 0, inp["m"])
        t = oracle.make_permutation(inp["perm_seed"], 0, 1, inp["n"])
        a = (inp["W0"][1], inp["thR"][1], inp["thP"][1], s, t, inp["X"][1])
        ts = time.perf_counter()
        oracle.forward(*a, inp["b"], contract=True)
        oracle.backward(*a, inp["gY"][1], inp["b"], contract=True)
        tot += time.perf_counter() - ts
    return {"value": round(ntok / tot, 2), "unit": "tokens/s", "cores": int(threads or os.cpu_count() or 1),
            "kind": "oracle", "cpu_count": os.cpu_count(), "blas_threads": threads, "cpu_model": cpu_model(),
            "sample": "float64 oracle (bf16 contract mode), fwd+bwd of the %d matrices of %s on the first %d of the "
                      "%d tokens; %.1f s; block builds and chain rule included once"
                      % (len(mats), cfg["name"], ntok, cfg["N"], tot)}


if __name__ == "__main__":
    main()
