"""Benchmark of the EQ-Linear hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5]

One step = one pass of the whole path over one batch of resident synthetic input:
pack the weight spectrum (forward and input-gradient packings), forward, input
gradient, weight gradient.  By default (--step train) the three passes are the
training-step entry points, which share the weight-gradient workspace: the forward
and the input gradient leave the half spectra of x and dy there and the weight
gradient runs its GEMMs on them; the same step through the plain entry points is
timed beside it (`plain_step`).  The default workload is the p4 (T=4) fp16 large
square layer, N=65536 rows, C=D=4096 (C'=D'=1024), forward + backward.

Prints ONE JSON line.  `value` is the dense-equivalent throughput of the step,
3 passes x 2*N*D*C FLOPs per step time.  `roofline` covers the step's dominant
kernel (the fused forward kernel, launched once by the forward pass and once by the
input gradient), timed with HIP events on the stream the library launches on
(torch's current stream).  `cpu_baseline` times the fp64 CPU oracle on a bounded row
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

MFMA_PEAK = {"f16": 2516.6, "f32": 157.3}   # dense TFLOP/s: 256 CU x 2.4 GHz x (4096 | 256) FLOP/clk
HBM_PEAK = 8000.0                            # GB/s
METRIC = "EQ-Linear dense-equivalent TFLOP/s + % MFMA peak, p4 fp16 fwd/bwd, 1 MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c5", choices=sorted(W.WORKLOADS))
    ap.add_argument("--step", default="train", choices=["train", "plain"],
                    help="train: eqlinear_fwd_train / eqlinear_bwd_x_train / eqlinear_bwd_w_train (the "
                         "forward and the input gradient leave the spectra in the weight-gradient workspace); "
                         "plain: eqlinear_fwd / eqlinear_bwd_x / eqlinear_bwd_w")
    ap.add_argument("--burn-in-ms", type=int, default=300,
                    help="untimed steps run back to back for at least this long before the warm-up "
                         "steps, so that the timed region starts at the GPU's steady clocks")
    ap.add_argument("--no-plain", action="store_true",
                    help="with --step train, skip timing the plain step beside it (for profiler runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip timing the unrolled dense GEMM comparator")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the same step captured once in a HIP graph and replayed")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip timing the fused epilogue (bias, GELU, residual; and its backward) against torch ops")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of the CPU-oracle sample (0: sized to about 12 s of work)")
    ap.add_argument("--rotate-mib", type=int, default=512,
                    help="rotate through enough copies of every buffer that one round of steps touches at "
                         "least this many MiB (above the 256 MiB Infinity Cache); 0: one resident set")
    ap.add_argument("--group", default="cyclic", choices=["cyclic", "p4m"],
                    help="p4m: time the layer over p4m's point group (dihedral D4, 8 elements) on the "
                         "workload's feature widths C and D (C' = C/8, D' = D/8), instead of the C_T layer")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this size (a reference for "
                         "profiler traffic counters)")
    return ap.parse_args()


def bwdw_fused_path(N, Cp, Dp, T, elt) -> bool:
    """Whether the library's weight gradient takes its fused path for this shape (the
    rule include/eqlinear.h documents for eqlinear_bwd_w, with its EQL_BWDW_PATH override)."""
    if N == 0 or T not in (1, 2, 4) or (Dp * T * elt) % 16 or N * Dp * T * elt >= 2**32:
        return False
    forced = os.environ.get("EQL_BWDW_PATH")
    if forced in ("fused", "separate"):
        return forced == "fused"
    planes = {1: 1, 2: 2, 4: 6}[T]
    return 2.0 * planes * N * Dp * Cp / (elt * T * N * (Cp + Dp)) < 400.0


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "group_circulant_linear_p4_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        table = json.load(f)
    ent = table.get("%s/%s" % (kernel, workload))
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the EQ-Linear path has no multi-GPU mode in this "
              "library (rows shard independently; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import group_circulant_linear_p4_amd as eql

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    eql.lib()  # fail loudly if the HIP library is missing
    wl = W.WORKLOADS[args.workload]
    if args.group == "p4m":
        return bench_p4m(args, torch, eql, wl)
    T, N, Cp, Dp = wl.T, wl.N, wl.Cp, wl.Dp
    code = eql.EQL_F16 if wl.dtype == "f16" else eql.EQL_F32
    tdt = torch.float16 if wl.dtype == "f16" else torch.float32
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("bench: generating %s" % wl.name, file=sys.stderr, flush=True)

    x_h, w_h, dy_h = W.make_x(wl), W.make_w(wl), W.make_dy(wl)
    elt = 2 if wl.dtype == "f16" else 4
    ws_bytes = eql.eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, code)
    # Rotating buffer sets: every step reads and writes its own copy of every buffer,
    # so that the working set of consecutive steps exceeds the 256 MiB Infinity Cache
    # (twice over) and each step starts cold, as the large workloads do by their size.
    set_bytes = (elt * (2 * N * Cp * T + 2 * N * Dp * T + 2 * Dp * Cp * T) + ws_bytes
                 + eql.eqlinear_packed_weight_bytes(Dp, Cp, T, code)
                 + eql.eqlinear_packed_weight_bytes(Cp, Dp, T, code))
    n_sets = max(1, -(-(args.rotate_mib << 20) // set_bytes)) if args.rotate_mib > 0 else 1
    sets = []
    for i in range(n_sets):
        b = {"x": torch.from_numpy(x_h).to(dev), "w": torch.from_numpy(w_h).to(dev),
             "dy": torch.from_numpy(dy_h).to(dev),
             "y": torch.empty((N, Dp * T), dtype=tdt, device=dev), "dx": torch.empty((N, Cp * T), dtype=tdt, device=dev),
             "dw": torch.empty((Dp, Cp, T), dtype=tdt, device=dev),
             "wp": torch.empty(eql.eqlinear_packed_weight_bytes(Dp, Cp, T, code), dtype=torch.uint8, device=dev),
             "wpb": torch.empty(eql.eqlinear_packed_weight_bytes(Cp, Dp, T, code), dtype=torch.uint8, device=dev),
             "ws": torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)}
        sets.append(b)
    s0 = sets[0]
    x, w, dy, y, dx, dw, wp, wpb, ws = (s0[k] for k in ("x", "w", "dy", "y", "dx", "dw", "wp", "wpb", "ws"))
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def make_calls(sp, b=s0, mode=None):
        mode = mode or args.step
        calls = {
            "pack": lambda: (eql.eqlinear_pack_weight(b["w"], b["wp"], Dp, Cp, T, code, eql.EQL_PACK_FWD, sp),
                             eql.eqlinear_pack_weight(b["w"], b["wpb"], Dp, Cp, T, code, eql.EQL_PACK_BWDX, sp)),
        }
        if mode == "train":
            calls["pack"] = lambda: eql.eqlinear_pack_weight_both(b["w"], b["wp"], b["wpb"], Dp, Cp, T, code, sp)
            calls["fwd"] = lambda: eql.eqlinear_fwd_train(b["x"], b["wp"], b["y"], b["ws"], ws_bytes, N, Cp, Dp, T,
                                                          code, sp)
            calls["bwd_x"] = lambda: eql.eqlinear_bwd_x_train(b["dy"], b["wpb"], b["dx"], b["ws"], ws_bytes, N, Cp,
                                                              Dp, T, code, sp)
            calls["bwd_w"] = lambda: eql.eqlinear_bwd_w_train(b["dy"], b["dw"], b["ws"], ws_bytes, N, Cp, Dp, T,
                                                              code, sp)
        else:
            calls["fwd"] = lambda: eql.eqlinear_fwd(b["x"], b["wp"], b["y"], N, Cp, Dp, T, code, sp)
            calls["bwd_x"] = lambda: eql.eqlinear_bwd_x(b["dy"], b["wpb"], b["dx"], N, Cp, Dp, T, code, sp)
            calls["bwd_w"] = lambda: eql.eqlinear_bwd_w(b["x"], b["dy"], b["dw"], b["ws"], ws_bytes, N, Cp, Dp, T,
                                                        code, sp)
        return calls

    set_calls = [make_calls(sptr, b) for b in sets]
    order = ["pack", "fwd", "bwd_x", "bwd_w"]

    def step(i, calls, events=None):
        for k in order:
            if events is not None:
                events[k][0].record(stream)
            calls[k]()
            if events is not None:
                events[k][1].record(stream)

    def timed(calls_of):
        """args.warmup untimed steps, then args.steps timed ones; step i runs calls_of(i)."""
        for i in range(args.warmup):
            step(i, calls_of(i))
        torch.cuda.synchronize()
        evs = [{k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in order}
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, calls_of(args.warmup + i), evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = {k: float(np.mean([e[k][0].elapsed_time(e[k][1]) for e in evs])) for k in order}
        # Device time of each step (the sum of its passes' event windows): spread across steps.
        step_dev = [sum(e[k][0].elapsed_time(e[k][1]) for k in order) for e in evs]
        return wall * 1e3 / args.steps, per, step_dev

    # Burn-in: a few milliseconds of warm-up steps leave the first timed region at a lower
    # clock than the rest (measured: c4 0.89 ms per step after 5 warm-up steps, 0.81 ms
    # after 200).
    t_burn = time.perf_counter()
    i = 0
    while args.burn_in_ms > 0:
        step(i, set_calls[i % n_sets])
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t_burn >= args.burn_in_ms * 1e-3:
                break
    torch.cuda.synchronize()
    ms_per_step, per, step_dev = timed(lambda i: set_calls[i % n_sets])
    plain_step = None
    if args.step == "train" and not args.no_plain:
        # The same step through the plain entry points (each pass on its own inputs; the
        # weight gradient transforms x and dy itself), for comparison.
        plain_calls = [make_calls(sptr, b, "plain") for b in sets]
        pms, pper, _ = timed(lambda i: plain_calls[i % n_sets])
        plain_step = {"ms_per_step": round(pms, 4), "passes_ms": {k: round(v, 4) for k, v in pper.items()},
                      "kind": "pack(fwd)+pack(bwd_x)+eqlinear_fwd+eqlinear_bwd_x+eqlinear_bwd_w on the same buffers"}
        del plain_calls
    warm = None
    if n_sets > 1:
        wms, wper, _ = timed(lambda i: set_calls[0])
        warm = {"ms_per_step": round(wms, 4), "passes_ms": {k: round(v, 4) for k, v in wper.items()},
                "kind": "one resident buffer set (inputs partly served from the Infinity Cache)"}

    dense_eq = 2.0 * N * (Dp * T) * (Cp * T)
    actual = 2.0 * (2 * T - 2 if T % 2 == 0 else 2 * T - 1) * N * Dp * Cp if T > 1 else 2.0 * N * Dp * Cp
    n_passes = 3
    value = n_passes * dense_eq / (ms_per_step * 1e-3) / 1e12
    bytes_pass = {
        "fwd": elt * (N * Cp * T + N * Dp * T + Dp * Cp * T),
        "bwd_x": elt * (N * Dp * T + N * Cp * T + Dp * Cp * T),
        "bwd_w": elt * (N * Cp * T + N * Dp * T + Dp * Cp * T),
    }
    if args.step == "train":
        # The training forward also writes x's half spectrum (the size of x); the training
        # input gradient writes dy's where the weight gradient takes the separate path.  The
        # weight gradient then reads the spectra instead of x and dy (the same bytes).
        bytes_pass["fwd"] += elt * N * Cp * T
        if not bwdw_fused_path(N, Cp, Dp, T, elt):
            bytes_pass["bwd_x"] += elt * N * Dp * T
    passes = {}
    for k in ("fwd", "bwd_x", "bwd_w"):
        t = per[k] * 1e-3
        passes[k] = {
            "ms": round(per[k], 4),
            "dense_eq_tflops": round(dense_eq / t / 1e12, 1),
            "actual_tflops": round(actual / t / 1e12, 1),
            "mfma_frac": round(actual / t / 1e12 / MFMA_PEAK[wl.dtype], 4),
            "hbm_gbs": round(bytes_pass[k] / t / 1e9, 1),
        }
    # Dominant kernel: the forward kernel runs twice per step (forward and input
    # gradient, one launch each: every workload here fits one launch's tile range),
    # the weight gradient is four launches (two transforms, the GEMM, the reduce).
    fwd_kernel_ms = per["fwd"] + per["bwd_x"]
    # T <= 4 with 16-byte rows runs the ring kernel eql_fwd4_kernel, other shapes eql_fwd_kernel.
    fwd_name = "eql_fwd4_kernel" if T <= 4 and (Cp * T * elt) % 16 == 0 and (Dp * T * elt) % 16 == 0 \
        else "eql_fwd_kernel"
    # The forward kernel's launches and their time.  In the training step at p4 fp16 the
    # forward (and, on the separate weight-gradient path, the input gradient) run the launch
    # whose column-0 tiles also store the spectrum; on other shapes the training passes add
    # a separate transform launch, so the kernel's own time is the plain pass's.
    spec_kernel = args.step == "train" and fwd_name == "eql_fwd4_kernel" and T == 4 and elt == 2
    fk_times = per
    if spec_kernel:
        fwd_name = "eql_fwd4_kernel_spec"
        fk_passes = ["fwd"] if bwdw_fused_path(N, Cp, Dp, T, elt) else ["fwd", "bwd_x"]
    else:
        fk_passes = ["fwd", "bwd_x"]
        if args.step == "train" and plain_step is not None:
            fk_times = plain_step["passes_ms"]
    t_fk = float(np.mean([fk_times[k] for k in fk_passes])) * 1e-3
    fk_bytes = elt * (N * Cp * T + N * Dp * T + Dp * Cp * T) + (elt * N * Cp * T if spec_kernel else 0)
    if fwd_kernel_ms >= per["bwd_w"]:
        dom, kname, t_dom, b_dom = "fwd", fwd_name, t_fk, fk_bytes
    else:
        dom, kname, t_dom, b_dom = "bwd_w", "eqlinear_bwd_w", per["bwd_w"] * 1e-3, bytes_pass["bwd_w"]
    flop_bound = actual / MFMA_PEAK[wl.dtype] / 1e12 >= b_dom / HBM_PEAK / 1e9
    if flop_bound:
        roofline = {"bound": "mfma", "achieved": round(actual / t_dom / 1e12, 1), "peak": MFMA_PEAK[wl.dtype],
                    "unit": "TFLOP/s"}
    else:
        roofline = {"bound": "hbm", "achieved": round(b_dom / t_dom / 1e9, 1), "peak": HBM_PEAK,
                    "unit": "GB/s"}
    roofline["frac"] = round(roofline["achieved"] / roofline["peak"], 4)
    roofline["traffic"] = traffic_for(kname, wl.key)
    roofline["kernel"] = kname
    roofline["ms_per_launch"] = round(t_dom * 1e3, 4)
    roofline["algorithmic"] = ("%.4g FLOP (%s real GEMMs of N x D' x C') and %.4g bytes (x, y, weight%s) per launch"
                               % (actual, (2 * T - 2) if T % 2 == 0 else (2 * T - 1), b_dom,
                                  ", x's spectrum" if spec_kernel and dom == "fwd" else ""))

    # The same step captured once in a HIP graph and replayed (the library records only
    # kernel launches on the caller's stream).  Reported beside the eager figure.
    graph = None
    if not args.no_graph:
        try:
            # One captured step per buffer set, in rotation order.
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for b_set in sets:
                    cap = make_calls(torch.cuda.current_stream().cuda_stream, b_set)  # the capturing stream
                    for k in order:
                        cap[k]()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            replays = max(1, -(-args.steps // n_sets))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(replays):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            gms = a.elapsed_time(b) / (replays * n_sets)
            graph = {"ms_per_step": round(gms, 4),
                     "value": round(n_passes * dense_eq / (gms * 1e-3) / 1e12, 2), "unit": "TFLOP/s"}
            del g
        except Exception as e:  # reported, never fatal: the eager line above is the result
            graph = {"error": "%s: %s" % (type(e).__name__, e)}

    if args.copy_probe_mib > 0:
        nbytes = args.copy_probe_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    dense = None
    if not args.no_dense:
        dense = dense_comparator(torch, [b["x"] for b in sets], w, [b["dy"] for b in sets], T,
                                 reps=max(5, min(args.steps, 20)))
        dense["speedup_fwd"] = round(dense["fwd_ms"] / per["fwd"], 3)
        dense["speedup_bwd_x"] = round(dense["bwd_x_ms"] / per["bwd_x"], 3)
        dense["speedup_bwd_w"] = round(dense["bwd_w_ms"] / per["bwd_w"], 3)
        total = dense["fwd_ms"] + dense["bwd_x_ms"] + dense["bwd_w_ms"]
        dense["speedup_fwd_bwd"] = round(total / (per["fwd"] + per["bwd_x"] + per["bwd_w"]), 3)
        if plain_step is not None:
            pp = plain_step["passes_ms"]
            dense["plain_speedup_fwd"] = round(dense["fwd_ms"] / pp["fwd"], 3)
            dense["plain_speedup_bwd_x"] = round(dense["bwd_x_ms"] / pp["bwd_x"], 3)
            dense["plain_speedup_bwd_w"] = round(dense["bwd_w_ms"] / pp["bwd_w"], 3)
            dense["plain_speedup_fwd_bwd"] = round(total / (pp["fwd"] + pp["bwd_x"] + pp["bwd_w"]), 3)

    fused = None
    if not args.no_fused:
        b = torch.from_numpy(W.make_bias(wl)).to(dev)
        fused = fused_epilogue(torch, eql, x, wp, b, dy, y, N, Cp, Dp, T, code, sptr,
                               reps=max(5, min(args.steps, 20)))
        # The plain forward (eqlinear_fwd) the fused epilogue is compared with.
        fused["plain_fwd_ms"] = round(plain_step["passes_ms"]["fwd"] if plain_step is not None else per["fwd"], 4)
        fused["mlp_train_step"] = mlp_train_step(torch, eql, x, w, wp, wpb, b, dy, y, dx, dw, ws, ws_bytes,
                                                 N, Cp, Dp, T, code, sptr, reps=max(5, min(args.steps, 20)),
                                                 train=args.step == "train")
        del b

    cpu = None
    if not args.no_cpu_baseline:
        del x, dy, y, dx, sets, set_calls, s0
        torch.cuda.empty_cache()
        cpu = cpu_baseline(wl, x_h, w_h, dy_h, args.cpu_rows, n_passes)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "burn_in_ms": args.burn_in_ms,
        "ms_per_step": round(ms_per_step, 4),
        "device_ms_per_step_p10_p50_p90": [round(float(np.percentile(step_dev, q)), 4) for q in (10, 50, 90)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; x,dy ~ N(0,1), w ~ N(0,1/C)%s)" % (
            ", %g%% of rows x%g" % (100 * wl.hot_rows_frac, wl.hot_rows_scale) if wl.hot_rows_frac else ""),
        "config": {"workload": wl.name, "T": T, "N": N, "C": Cp * T, "D": Dp * T,
                   "step": ("pack_both+fwd_train+bwd_x_train+bwd_w_train" if args.step == "train"
                            else "pack(fwd)+pack(bwd_x)+fwd+bwd_x+bwd_w"), "buffer_sets": n_sets,
                   "set_mib": round(set_bytes / 2**20, 1)},
        "warm": warm,
        "passes": passes,
        "pack_ms": round(per["pack"], 4),
        "mfma_frac_step": round(n_passes * actual / (ms_per_step * 1e-3) / 1e12 / MFMA_PEAK[wl.dtype], 4),
        "roofline": roofline,
        "plain_step": plain_step,
        "graph_step": graph,
        "dense_baseline": dense,
        "fused_epilogue": fused,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def fused_epilogue(torch, eql, x, wp, b, r, y, N, Cp, Dp, T, code, sptr, reps):
    """eqlinear_fwd_fused against the forward followed by the same epilogue as
    separate torch ops, on the benchmark's workload: bias + GELU (the MLP expansion)
    and bias + residual (the MLP projection back; dy's buffer serves as the residual)."""
    F = torch.nn.functional
    bb = b.repeat_interleave(T)

    def timeit(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return a.elapsed_time(e) / reps

    def unfused(gelu, res):
        eql.eqlinear_fwd(x, wp, y, N, Cp, Dp, T, code, sptr)
        z = y + bb
        if gelu:
            z = F.gelu(z)
        if res:
            z = z + r
        return z

    res = {
        "bias_gelu_ms": timeit(lambda: eql.eqlinear_fwd_fused(x, wp, b, None, y, None, N, Cp, Dp, T, code,
                                                              eql.EQL_ACT_GELU, sptr)),
        "bias_gelu_torch_ms": timeit(lambda: unfused(True, False)),
        "bias_residual_ms": timeit(lambda: eql.eqlinear_fwd_fused(x, wp, b, r, y, None, N, Cp, Dp, T, code,
                                                                  eql.EQL_ACT_NONE, sptr)),
        "bias_residual_torch_ms": timeit(lambda: unfused(False, True)),
    }
    # Training: the forward also keeps the activation's input, and the backward of the
    # epilogue (dpre = dy * GELU'(pre), dbias) runs before the layer's input and weight
    # gradients.  Torch's counterpart: its GELU backward and a channel sum.
    pre = torch.empty_like(y)
    dpre = torch.empty_like(y)
    db = torch.empty_like(b)
    ws_bytes = eql.eqlinear_fused_epilogue_bwd_workspace_bytes(N, Dp, T, code)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=y.device)
    res["bias_gelu_pre_out_ms"] = timeit(lambda: eql.eqlinear_fwd_fused(x, wp, b, None, y, pre, N, Cp, Dp, T, code,
                                                                        eql.EQL_ACT_GELU, sptr))

    def torch_epi_bwd():
        g = torch.ops.aten.gelu_backward(r, pre)
        return g, g.view(N, Dp, T).sum(dim=(0, 2))

    res["epilogue_bwd_ms"] = timeit(lambda: eql.eqlinear_fused_epilogue_bwd(r, pre, dpre, db, ws, ws_bytes, N, Dp, T,
                                                                            code, eql.EQL_ACT_GELU, sptr))
    res["epilogue_bwd_torch_ms"] = timeit(torch_epi_bwd)
    # dy and pre read, dpre written once each (the bias partials are 1/64 of that).
    epi_bytes = 3 * N * Dp * T * y.element_size()
    del pre, dpre, db, ws
    res = {k: round(v, 4) for k, v in res.items()}
    res["speedup_bias_gelu"] = round(res["bias_gelu_torch_ms"] / res["bias_gelu_ms"], 3)
    res["speedup_bias_residual"] = round(res["bias_residual_torch_ms"] / res["bias_residual_ms"], 3)
    res["speedup_epilogue_bwd"] = round(res["epilogue_bwd_torch_ms"] / res["epilogue_bwd_ms"], 3)
    res["epilogue_bwd_GBps"] = round(epi_bytes / (res["epilogue_bwd_ms"] * 1e-3) / 1e9, 1)
    res["kind"] = ("eqlinear_fwd_fused vs eqlinear_fwd + torch (y + b), F.gelu, + residual; "
                   "eqlinear_fused_epilogue_bwd vs torch gelu_backward + channel sum")
    torch.cuda.empty_cache()
    return res


def mlp_train_step(torch, eql, x, w, wp, wpb, b, dy, y, dx, dw, ws, ws_bytes, N, Cp, Dp, T, code, sptr, reps,
                   train=True):
    """One training step of the layer as an MLP expansion, y = GELU(x W^T + b): the
    library's pack (both forms), fused forward keeping pre, epilogue backward (dpre,
    dbias), input and weight gradients on dpre (train: through eqlinear_fwd_fused_train,
    eqlinear_bwd_x_train and eqlinear_bwd_w_train); against the unrolled dense layer in
    torch (F.linear with the repeated bias, F.gelu, gelu_backward, the bias sum, the two
    gradient matmuls, and the fold of the dense weight gradient onto the T tied entries
    of each (d, c)).  Both produce y, dx, dw and db."""
    F = torch.nn.functional
    g = torch.arange(T, device=w.device)
    idx = (g.view(T, 1) - g.view(1, T)) % T          # idx[g][h] = (g - h) mod T
    Wd = w[:, :, idx].permute(0, 2, 1, 3).reshape(Dp * T, Cp * T).contiguous()
    bb = b.repeat_interleave(T)
    # dw[d, c, t] = sum_g dWd[(d, g), (c, (g - t) mod T)]: gather along the last axis
    # with idx[g][t] = (g - t) mod T, then sum over g.
    fold = idx.view(1, T, 1, T).expand(Dp, T, Cp, T)
    pre, dpre = torch.empty_like(y), torch.empty_like(y)
    db = torch.empty_like(b)
    ebytes = eql.eqlinear_fused_epilogue_bwd_workspace_bytes(N, Dp, T, code)
    ews = torch.empty(max(ebytes, 16), dtype=torch.uint8, device=y.device)

    def lib_step():
        if not train:
            eql.eqlinear_pack_weight(w, wp, Dp, Cp, T, code, eql.EQL_PACK_FWD, sptr)
            eql.eqlinear_pack_weight(w, wpb, Dp, Cp, T, code, eql.EQL_PACK_BWDX, sptr)
        if train:
            eql.eqlinear_pack_weight_both(w, wp, wpb, Dp, Cp, T, code, sptr)
            eql.eqlinear_fwd_fused_train(x, wp, b, None, y, pre, ws, ws_bytes, N, Cp, Dp, T, code, eql.EQL_ACT_GELU,
                                         sptr)
        else:
            eql.eqlinear_fwd_fused(x, wp, b, None, y, pre, N, Cp, Dp, T, code, eql.EQL_ACT_GELU, sptr)
        eql.eqlinear_fused_epilogue_bwd(dy, pre, dpre, db, ews, ebytes, N, Dp, T, code, eql.EQL_ACT_GELU, sptr)
        if train:
            eql.eqlinear_bwd_x_train(dpre, wpb, dx, ws, ws_bytes, N, Cp, Dp, T, code, sptr)
            eql.eqlinear_bwd_w_train(dpre, dw, ws, ws_bytes, N, Cp, Dp, T, code, sptr)
        else:
            eql.eqlinear_bwd_x(dpre, wpb, dx, N, Cp, Dp, T, code, sptr)
            eql.eqlinear_bwd_w(x, dpre, dw, ws, ws_bytes, N, Cp, Dp, T, code, sptr)

    def torch_step():
        pre_t = F.linear(x, Wd, bb)
        y_t = F.gelu(pre_t)
        gr = torch.ops.aten.gelu_backward(dy, pre_t)
        db_t = gr.view(N, Dp, T).sum(dim=(0, 2))
        dx_t = torch.mm(gr, Wd)
        dWd = torch.mm(gr.t(), x)
        dw_t = torch.gather(dWd.view(Dp, T, Cp, T), 3, fold).sum(dim=1)
        return y_t, db_t, dx_t, dw_t

    def timeit(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return a.elapsed_time(e) / reps

    res = {"lib_ms": round(timeit(lib_step), 4), "torch_dense_ms": round(timeit(torch_step), 4)}
    res["speedup"] = round(res["torch_dense_ms"] / res["lib_ms"], 3)
    lib_kind = ("pack_both + eqlinear_fwd_fused_train(bias, GELU, pre) + eqlinear_fused_epilogue_bwd + "
                "bwd_x_train + bwd_w_train" if train else
                "pack x2 + eqlinear_fwd_fused(bias, GELU, pre) + eqlinear_fused_epilogue_bwd + bwd_x + bwd_w")
    res["kind"] = lib_kind + (", vs torch on the unrolled dense weight (F.linear, F.gelu, gelu_backward, bias sum, "
                              "mm x2, weight-gradient fold)")
    del Wd, pre, dpre, ews
    torch.cuda.empty_cache()
    return res


def dense_comparator(torch, xs, w, dys, T, reps):
    """The unrolled ("replicate and multiply dense") layer on the same GPU: torch
    F.linear and matmuls on the dense (D'T) x (C'T) weight (built outside the timed
    region), rotating over the same buffer sets as the library's step (xs, dys)."""
    Dp, Cp, _ = w.shape
    g = torch.arange(T, device=w.device)
    idx = (g.view(T, 1) - g.view(1, T)) % T
    Wd = w[:, :, idx].permute(0, 2, 1, 3).reshape(Dp * T, Cp * T).contiguous()
    F = torch.nn.functional
    n = len(xs)

    def timeit(fn):
        for i in range(3):
            fn(i % n)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            fn(i % n)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    dyTs = [dy.t().contiguous() for dy in dys]
    res = {
        "fwd_ms": timeit(lambda i: F.linear(xs[i], Wd)),
        "bwd_x_ms": timeit(lambda i: torch.matmul(dys[i], Wd)),
        "bwd_w_ms": timeit(lambda i: torch.matmul(dyTs[i], xs[i])),
    }
    res = {k: round(v, 4) for k, v in res.items()}
    res["kind"] = "torch F.linear / matmul on the unrolled dense weight (hipBLASLt)"
    res["buffer_sets"] = n
    del Wd, dyTs
    return res


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform's description."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(wl, x_h, w_h, dy_h, rows, n_passes, target_s=12.0, min_s=10.0, max_reps=6):
    """The fp64 oracle on the first `rows` rows of the workload, all three passes.
    rows == 0: a 1024-row probe sizes the sample to about `target_s` seconds; a run
    that still falls short of `min_s` is resized (or, once it covers the whole
    workload, repeated) until the timed work reaches `min_s`."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))

    def run(r):
        xs, dys = x_h[:r], dy_h[:r]
        t0 = time.perf_counter()
        oracle.fwd(xs, w_h)
        oracle.bwd_x(dys, w_h)
        oracle.bwd_w(xs, dys, wl.T)
        return time.perf_counter() - t0

    if rows <= 0:
        probe = min(1024, wl.N)
        t_probe = run(probe)
        rows = int(min(wl.N, max(probe, probe * target_s / max(t_probe, 1e-3))))
        dt = run(rows)
        if dt < min_s and rows < wl.N:
            rows = int(min(wl.N, rows * target_s / max(dt, 1e-3)))
            dt = run(rows)
    else:
        dt = run(rows)
    total, reps = dt, 1
    while total < min_s and rows == wl.N and reps < max_reps:
        total += run(rows)
        reps += 1
    flops = n_passes * 2.0 * rows * wl.D * wl.C * reps
    what = "rows 0..%d" % (rows - 1) if rows < wl.N else "all %d rows" % rows
    return {"value": round(flops / total / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores), "cpu": cpu_model(),
            "kind": "oracle",
            "sample": "%s of the same workload x %d run(s), forward + input gradient + weight gradient, "
                      "fp64 dense unroll (%.1f s)" % (what, reps, total)}


def bench_p4m(args, torch, eql, wl):
    """The p4m layer's training step on the workload's feature widths: weight expansion and
    both packings, forward, input gradient, weight gradient and its fold; all on the C_4 view
    (2C' x 2D' channels, T = 4) the library runs p4m as.  One JSON line like main()'s."""
    C, D, N = wl.Cp * wl.T, wl.Dp * wl.T, wl.N
    if C % 8 or D % 8:
        print("p4m needs feature widths divisible by 8", file=sys.stderr)
        sys.exit(2)
    Cp, Dp = C // 8, D // 8
    code = eql.EQL_F16 if wl.dtype == "f16" else eql.EQL_F32
    tdt = torch.float16 if wl.dtype == "f16" else torch.float32
    elt = 2 if wl.dtype == "f16" else 4
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("bench: generating %s as a p4m layer (C'=%d, D'=%d)" % (wl.name, Cp, Dp), file=sys.stderr, flush=True)
    x_h, dy_h = W.make_x(wl), W.make_dy(wl)
    g = np.random.default_rng(wl.seed + 101)
    w_h = (g.standard_normal((Dp, Cp, 8), dtype=np.float32) / np.sqrt(C)).astype(x_h.dtype)
    x, dy, w = (torch.from_numpy(a).to(dev) for a in (x_h, dy_h, w_h))
    w4 = torch.empty((2 * Dp, 2 * Cp, 4), dtype=tdt, device=dev)
    wp = torch.empty(eql.eqlinear_packed_weight_bytes(2 * Dp, 2 * Cp, 4, code), dtype=torch.uint8, device=dev)
    wpb = torch.empty(eql.eqlinear_packed_weight_bytes(2 * Cp, 2 * Dp, 4, code), dtype=torch.uint8, device=dev)
    y = torch.empty((N, D), dtype=tdt, device=dev)
    dx = torch.empty((N, C), dtype=tdt, device=dev)
    dw4 = torch.empty_like(w4)
    dw = torch.empty_like(w)
    ws_bytes = eql.eqlinear_bwd_w_workspace_bytes(N, 2 * Cp, 2 * Dp, 4, code)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    calls = {
        "pack": lambda: (eql.eqlinear_p4m_expand_weight(w, w4, Dp, Cp, code, sp),
                         eql.eqlinear_pack_weight(w4, wp, 2 * Dp, 2 * Cp, 4, code, eql.EQL_PACK_FWD, sp),
                         eql.eqlinear_pack_weight(w4, wpb, 2 * Dp, 2 * Cp, 4, code, eql.EQL_PACK_BWDX, sp)),
        "fwd": lambda: eql.eqlinear_fwd(x, wp, y, N, 2 * Cp, 2 * Dp, 4, code, sp),
        "bwd_x": lambda: eql.eqlinear_bwd_x(dy, wpb, dx, N, 2 * Cp, 2 * Dp, 4, code, sp),
        "bwd_w": lambda: (eql.eqlinear_bwd_w(x, dy, dw4, ws, ws_bytes, N, 2 * Cp, 2 * Dp, 4, code, sp),
                          eql.eqlinear_p4m_fold_weight_grad(dw4, dw, Dp, Cp, code, sp)),
    }
    if args.step == "train":
        calls["pack"] = lambda: (eql.eqlinear_p4m_expand_weight(w, w4, Dp, Cp, code, sp),
                                 eql.eqlinear_pack_weight_both(w4, wp, wpb, 2 * Dp, 2 * Cp, 4, code, sp))
        calls["fwd"] = lambda: eql.eqlinear_fwd_train(x, wp, y, ws, ws_bytes, N, 2 * Cp, 2 * Dp, 4, code, sp)
        calls["bwd_x"] = lambda: eql.eqlinear_bwd_x_train(dy, wpb, dx, ws, ws_bytes, N, 2 * Cp, 2 * Dp, 4, code, sp)
        calls["bwd_w"] = lambda: (eql.eqlinear_bwd_w_train(dy, dw4, ws, ws_bytes, N, 2 * Cp, 2 * Dp, 4, code, sp),
                                  eql.eqlinear_p4m_fold_weight_grad(dw4, dw, Dp, Cp, code, sp))
    order = ["pack", "fwd", "bwd_x", "bwd_w"]
    t_burn = time.perf_counter()
    while args.burn_in_ms > 0 and time.perf_counter() - t_burn < args.burn_in_ms * 1e-3:
        for _ in range(8):
            for k in order:
                calls[k]()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        for k in order:
            calls[k]()
    torch.cuda.synchronize()
    evs = [{k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in order}
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        for k in order:
            evs[i][k][0].record(stream)
            calls[k]()
            evs[i][k][1].record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    per = {k: float(np.mean([e[k][0].elapsed_time(e[k][1]) for e in evs])) for k in order}
    dense_eq = 2.0 * N * D * C
    actual = 2.0 * 6 * N * (2 * Dp) * (2 * Cp)            # the C_4 view's six real GEMMs
    value = 3 * dense_eq / (ms_step * 1e-3) / 1e12
    bytes_pass = elt * (N * C + N * D + D * C // 4)        # x, y once; w4 (2D' x 2C' x 4: twice the parameters)
    passes = {k: {"ms": round(per[k], 4), "dense_eq_tflops": round(dense_eq / (per[k] * 1e-3) / 1e12, 1),
                  "actual_tflops": round(actual / (per[k] * 1e-3) / 1e12, 1)} for k in ("fwd", "bwd_x", "bwd_w")}
    t_dom = 0.5 * (per["fwd"] + per["bwd_x"]) * 1e-3
    if actual / MFMA_PEAK[wl.dtype] / 1e12 >= bytes_pass / HBM_PEAK / 1e9:
        roofline = {"bound": "mfma", "achieved": round(actual / t_dom / 1e12, 1), "peak": MFMA_PEAK[wl.dtype],
                    "unit": "TFLOP/s"}
    else:
        roofline = {"bound": "hbm", "achieved": round(bytes_pass / t_dom / 1e9, 1), "peak": HBM_PEAK, "unit": "GB/s"}
    roofline["frac"] = round(roofline["achieved"] / roofline["peak"], 4)
    roofline["traffic"] = None
    roofline["kernel"] = ("eql_fwd4_kernel (C_4 view; in the training step the forward's launch also stores x's "
                          "spectrum, the input gradient's is the plain kernel where the weight gradient reads dy itself)"
                          if args.step == "train" else "eql_fwd4_kernel (C_4 view)")
    roofline["ms_per_launch"] = round(t_dom * 1e3, 4)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import p4m_oracle as P
        rows = args.cpu_rows if args.cpu_rows > 0 else N
        xs, dys = x_h[:rows], dy_h[:rows]
        total, reps = 0.0, 0
        while reps == 0 or (total < 10.0 and reps < 6):  # about 10 s of oracle work
            t0 = time.perf_counter()
            P.fwd(xs, w_h)
            P.bwd_x(dys, w_h)
            P.bwd_w(xs, dys)
            total += time.perf_counter() - t0
            reps += 1
        cpu = {"value": round(3 * 2.0 * rows * D * C * reps / total / 1e12, 5), "unit": "TFLOP/s",
               "cores": len(os.sched_getaffinity(0)), "cpu": cpu_model(), "kind": "oracle",
               "sample": "rows 0..%d x %d run(s), p4m oracle forward + input gradient + weight gradient, "
                         "fp64 dense unroll (%.1f s)" % (rows - 1, reps, total)}
    line = {"metric": "p4m EQ-Linear dense-equivalent TFLOP/s, %s fwd/bwd, 1 MI355X" % wl.dtype,
            "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": wl.dtype, "data": "synthetic (seeded; x, dy ~ N(0,1), w ~ N(0,1/C))",
            "config": {"workload": "p4m layer on %s's widths: N=%d, C=%d (C'=%d x 8), D=%d (D'=%d x 8)"
                                   % (wl.key, N, C, Cp, D, Dp),
                       "group": "p4m (D4)",
                       "step": ("expand+pack_both, fwd_train, bwd_x_train, bwd_w_train+fold" if args.step == "train"
                                else "expand+pack x2, fwd, bwd_x, bwd_w+fold")},
            "passes": passes, "pack_ms": round(per["pack"], 4), "roofline": roofline, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
