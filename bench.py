"""Benchmark: POET-X layer fwd+bwd tokens/s on one MI355X.

Workload (default): the LLaMA-1B-shaped layer set -- q, k, v, o 2048x2048,
gate, up 5632x2048, down 2048x5632 -- bf16 W0, block size 256, 8192 tokens,
generators ~N(0, 1e-3).  One step is the hot path over one batch: forward of
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
# MFMA-bound classes and the dense peak of the arithmetic they carry: the
# weight products run on bf16 MFMA; the Cayley solve and the chain rule are
# fp32 computations (emulated with split bf16 products), so they take the
# fp32 peak
MFMA_CLASSES = {"gemm_nt": 2500.0, "gemm_nn": 2500.0, "cayley_build": 157.3, "chain_rule": 157.3}

# kernel name (demangled, as rocprofv3 prints it) -> timing class of the library,
# and the dispatches one timed launch of the class makes
KERNEL_CLASSES = [
    ("permute_gather_kernel", "xform_permute", 1),
    ("permute_scatter_kernel", "xform_permute", 1),
    ("permute_stream_kernel", "xform_permute", 1),
    ("blockdiag_kernel", "xform_blockmul", 1),
    ("gemm_bf16_kernel<false, true,", "xform_blockmul", 1),
    ("gemm_bf16_kernel<false, false,", "gemm_nt", 1),
    ("gemm_wide_kernel<false>", "gemm_nt", 1),
    ("gemm_wide_kernel<true>", "gemm_nn", 1),
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
    ap.add_argument("--cpu-tokens", type=int, default=3072, help="token sample of the oracle baseline")
    ap.add_argument("--profile-steps", type=int, default=3)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="end with one plain copy kernel of %d MiB (read and write) for counter calibration"
                         % (CALIBRATION_BYTES >> 20))
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of "
                         "'bench.py --calibrate-copy' into profiles/traffic_<class>.json")
    ap.add_argument("--kernel-stats", metavar="CSV",
                    help="no GPU: summarize by kernel class a rocprofv3 kernel_stats.csv (whole run) or a "
                         "kernel_trace.csv (only the marked, serialized per-kernel timing pass)")
    ap.add_argument("--workload", choices=("layerset", "stack24"), default="layerset",
                    help="layerset: fwd+bwd of the LLaMA-1B layer set (default); stack24: one training step of the "
                         "24-layer stack with Adam and the global merge")
    ap.add_argument("--streams", type=int, default=3,
                    help="HIP streams the seven independent matrices are spread over (batched mode)")
    ap.add_argument("--chain", choices=["batched", "per-matrix"], default="batched",
                    help="layer set: one chain-rule call for all matrices after the backward pass, or one per "
                         "matrix on its stream")
    ap.add_argument("--w0-int8", action="store_true",
                    help="layer set: base weights stored as per-row INT8 codes and scales (POET-XQ), dequantized "
                         "by every pass")
    ap.add_argument("--keep-z2", action="store_true",
                    help="layer set: the variant without activation recompute (the forward keeps z2' for the "
                         "backward, N*m*2 bytes per matrix); the default recomputes it (POET-Xmem)")
    ap.add_argument("--per-layer-builds", action="store_true",
                    help="let every forward / backward call build its own blocks (one builder launch per call) "
                         "instead of one batched build per pass")
    return ap.parse_args()


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "orthogonal_reparameterized_poetx_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_record(cls):
    """HBM bytes per launch from a committed rocprofv3 counter record, if its
    kernel source hash still matches the current source."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % cls)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != kernel_source_hash(rec.get("source_files", [])):
        return None
    return rec


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
        for name, v in tab.values():
            cls, per = kernel_class(name)
            if cls is None:
                continue
            a = agg.setdefault(cls, dict(fetch=0.0, write=0.0, dispatches_fetch=0, dispatches_write=0, per=per,
                                         kernels=set()))
            a[key] += v * 1024.0 * k
            a["dispatches_" + key] += 1
            a["kernels"].add(name.split("(")[0])
    src_files = ["api.hip", "build.hip", "chain.hip", "transform.hip", "blockdiag.hip", "gemm.hip", "gram.hip",
                 "merge.hip", "common.h", "kernels.h"]
    h = kernel_source_hash(src_files)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for cls, a in agg.items():
        launches_f = a["dispatches_fetch"] / a["per"]
        launches_w = a["dispatches_write"] / a["per"]
        rec = dict(kernel_class=cls, source_hash=h, source_files=src_files,
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

    def __init__(self, P, WL, torch, dev, N, nlayers=24, exact=(), streams=3, w0_int8=False):
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
        # matrices run on `streams` streams (matrix i on stream i % streams);
        # each stream has its own workspace pool
        self.nstreams = max(int(streams), 1)
        pools = [{} for _ in range(self.nstreams)]
        self.layers, self.X, self.gY, self.out = [], {}, [], []
        mats_done = []
        off = 0
        bf = torch.bfloat16
        for l, idx, m, n in mats:
            j = 7 * l + idx
            lay = P.PoetxLayer(m, n, b, "bf16", dev, perm_seed=WL.perm_seed(5, j),
                               ws_pool=pools[len(mats_done) % self.nstreams], w0_int8=w0_int8)
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
            lay.workspace(P.OP_MERGE_BLOCKS)
            lay.dq_buffers()
        self.adam_steps = 0

    def _fan_out(self, main, idx_items, fn):
        for w in self.workers[1:]:
            w.wait_stream(main)
        for i, item in idx_items:
            with self.torch.cuda.stream(self.workers[i % self.nstreams]):
                fn(*item)
        for w in self.workers[1:]:
            main.wait_stream(w)

    def forward_backward(self):
        P, torch = self.P, self.torch
        main = torch.cuda.current_stream()
        if not hasattr(self, "side"):
            self.side = torch.cuda.Stream()      # all streams at the default priority
            self.bwd_ready = torch.cuda.Event()
            self.workers = [main] + [torch.cuda.Stream() for _ in range(self.nstreams - 1)]
        # the backward blocks depend only on the generators: build them on a
        # second stream while the forward pass runs (enqueued after the forward
        # build, so that build gets the CUs first)
        self.side.wait_stream(main)
        P.build_layer_blocks(self.layers, "forward")
        with torch.cuda.stream(self.side):
            P.build_layer_blocks(self.layers, "backward")
            self.bwd_ready.record(self.side)
        n = len(self.layers)
        self._fan_out(main, [(i, (self.layers[i], self.out[i])) for i in range(n)],
                      lambda lay, o: lay.forward_blocks(self.X[lay.x_key], Y=o["Y"]))
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
        if not hasattr(self, "workers"):
            self.workers = [main] + [self.torch.cuda.Stream() for _ in range(self.nstreams - 1)]
        self._fan_out(main, list(enumerate((lay,) for lay in self.layers)), lambda lay: lay.merge_blocks())

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
    st = Stack(P, WL, torch, dev, N, streams=args.streams, w0_int8=args.w0_int8)
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
    print(json.dumps({
        "metric": "POET-X 24-layer stack training step (fwd+bwd, Adam, global merge), 1 GPU",
        "value": round(N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": k, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded Gaussian inputs with the stack's shapes)",
        "config": {"workload": WL.CONFIGS[5]["name"], "tokens": N, "matrices": len(st.layers), "b": WL.CONFIGS[5]["b"],
                   "base_weights": "INT8 codes with per-row fp32 scales (POET-XQ)" if args.w0_int8 else "bf16"},
        "phases_ms": {"fwd_bwd": round(fb / k, 3), "adam": round(ad / k, 3), "merge": round(mg / k, 3)},
        "generators": st.theta.numel(),
        "resident_gb": round(resident / 1e9, 3),
        "peak_hbm_gb": round(torch.cuda.max_memory_allocated() / 1e9, 3),
    }), flush=True)


def main():
    args = parse()
    if args.workload == "stack24":
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
    if args.keep_z2 and args.per_layer_builds:
        print("--keep-z2 uses the prebuilt-block calls; drop --per-layer-builds", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    cfg = WL.CONFIGS[3]
    N = args.tokens or cfg["N"]

    def up(pair, dt):
        a = np.ascontiguousarray(pair[0])
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a.astype(np.float32)).to(dev)

    # ---- resident inputs: seven packed layers, their inputs and upstream grads
    layers, Xs, gYs, outs = [], {}, [], []
    for j in range(len(cfg["mats"])):
        inp = WL.matrix_inputs(3, j, N=N)
        lay = P.PoetxLayer(inp["m"], inp["n"], inp["b"], "bf16", dev, perm_seed=inp["perm_seed"],
                           w0_int8=args.w0_int8)
        lay.pack(up(inp["W0"], "bf16"))
        lay.thR.copy_(up(inp["thR"], "f32"))
        lay.thP.copy_(up(inp["thP"], "f32"))
        owner = WL.input_owner(cfg, j)
        if owner not in Xs:
            Xs[owner] = up(inp["X"], "bf16")
        lay.x_key = owner
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
    # streams (all at the default priority) so one matrix's kernel tails and
    # small launches overlap another's work
    workers = [stream] + [torch.cuda.Stream() for _ in range(max(args.streams, 1) - 1)]

    active = {"workers": workers, "side": side}

    def fan_out(items, fn):
        ws = active["workers"]
        for w in ws[1:]:
            w.wait_stream(stream)
        for i, item in enumerate(items):
            with torch.cuda.stream(ws[i % len(ws)]):
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
        bs.wait_stream(stream)
        # the forward build is enqueued first, so its workgroups take the CUs
        # before the backward build's
        P.build_layer_blocks(layers, "forward")
        with torch.cuda.stream(bs):
            P.build_layer_blocks(layers, "backward")
            bwd_blocks_ready.record(bs)
        if args.keep_z2:
            fan_out(list(zip(layers, outs)),
                    lambda lay, o: lay.forward_blocks_z2(Xs[lay.x_key], Y=o["Y"], Z2=o["Z2"]))
        else:
            fan_out(list(zip(layers, outs)), lambda lay, o: lay.forward_blocks(Xs[lay.x_key], Y=o["Y"]))
        stream.wait_event(bwd_blocks_ready)
        def bwd(lay, g, o):
            if args.keep_z2:
                lay.backward_blocks_dq_z2(Xs[lay.x_key], g, o["Z2"], dX=o["dX"])
            else:
                lay.backward_blocks_dq(Xs[lay.x_key], g, dX=o["dX"])
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
    active["workers"], active["side"] = [stream], stream
    P.timing_enable(True)
    for _ in range(args.profile_steps):
        step()
    torch.cuda.synchronize()
    kern = P.timing_summary()
    P.timing_enable(False)
    active["workers"], active["side"] = workers, side
    torch.sigmoid_(marker)
    torch.cuda.synchronize()
    per_step = {k: dict(v, ms=v["ms"] / args.profile_steps, launches=v["launches"] / args.profile_steps,
                        flops=v["flops"] / args.profile_steps, bytes=v["bytes"] / args.profile_steps)
                for k, v in kern.items()}
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
    rec = traffic_record(dom)
    roof["traffic"] = None if rec is None else rec["hbm_bytes_per_launch"]
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
        "data": "synthetic (seeded Gaussian inputs with the layer set's shapes)",
        "config": {"workload": cfg["name"], "tokens": N, "matrices": len(cfg["mats"]), "b": cfg["b"],
                   "shapes": ["%dx%d" % (m, n) for _, m, n in cfg["mats"]],
                   "block_builds": "per layer call" if args.per_layer_builds else
                   "batched per pass (Cayley builds and chain rule over all seven matrices)",
                   "streams": 1 if args.per_layer_builds else max(args.streams, 1),
                   "activations": "z2' kept from the forward pass (no recompute)" if args.keep_z2 else
                   "recomputed in the backward pass (POET-Xmem)",
                   "base_weights": "INT8 codes with per-row fp32 scales, dequantized per pass (POET-XQ)"
                   if args.w0_int8 else "bf16"},
        "roofline": roof,
        "kernels_per_step": breakdown,
        "merge_ms_layer_set": round(merge_ms, 3),
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
        result["cpu_baseline"] = cpu_baseline(args.cpu_tokens)
    print(json.dumps(result), flush=True)


def cpu_baseline(ntok):
    import numpy as np

    import oracle
    import workloads as WL
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cfg = WL.CONFIGS[3]
    rows = np.arange(ntok)
    # time only the oracle calls (input generation excluded)
    tot = 0.0
    for j in range(len(cfg["mats"])):
        inp = WL.matrix_inputs(3, j, rows=rows)
        s = oracle.make_permutation(inp["perm_seed"], 0, 0, inp["m"])
        t = oracle.make_permutation(inp["perm_seed"], 0, 1, inp["n"])
        a = (inp["W0"][1], inp["thR"][1], inp["thP"][1], s, t, inp["X"][1])
        ts = time.perf_counter()
        oracle.forward(*a, inp["b"], contract=True)
        oracle.backward(*a, inp["gY"][1], inp["b"], contract=True)
        tot += time.perf_counter() - ts
    return {"value": round(ntok / tot, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": "float64 oracle (bf16 contract mode), fwd+bwd of all 7 layer-set matrices on the first %d "
                      "of the 8192 tokens; %.1f s; per-step block builds and chain rule included once" % (ntok, tot)}


if __name__ == "__main__":
    main()
