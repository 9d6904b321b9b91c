"""Benchmark of the EQ-Linear hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5]

One step = one pass of the whole path over one batch of resident synthetic input:
pack the weight spectrum (forward and input-gradient packings), forward, input
gradient, weight gradient.  The default workload is the p4 (T=4) fp16 large square
layer, N=65536 rows, C=D=4096 (C'=D'=1024), forward + backward.

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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip timing the unrolled dense GEMM comparator")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the same step captured once in a HIP graph and replayed")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip timing the fused epilogue (bias, GELU, residual; and its backward) against torch ops")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of the CPU-oracle sample (0: sized to about 12 s of work)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this size (a reference for "
                         "profiler traffic counters)")
    return ap.parse_args()


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
    T, N, Cp, Dp = wl.T, wl.N, wl.Cp, wl.Dp
    code = eql.EQL_F16 if wl.dtype == "f16" else eql.EQL_F32
    tdt = torch.float16 if wl.dtype == "f16" else torch.float32
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("bench: generating %s" % wl.name, file=sys.stderr, flush=True)

    x_h, w_h, dy_h = W.make_x(wl), W.make_w(wl), W.make_dy(wl)
    x = torch.from_numpy(x_h).to(dev)
    w = torch.from_numpy(w_h).to(dev)
    dy = torch.from_numpy(dy_h).to(dev)
    y = torch.empty((N, Dp * T), dtype=tdt, device=dev)
    dx = torch.empty((N, Cp * T), dtype=tdt, device=dev)
    dw = torch.empty((Dp, Cp, T), dtype=tdt, device=dev)
    wp = torch.empty(eql.eqlinear_packed_weight_bytes(Dp, Cp, T, code), dtype=torch.uint8, device=dev)
    wpb = torch.empty(eql.eqlinear_packed_weight_bytes(Cp, Dp, T, code), dtype=torch.uint8, device=dev)
    ws_bytes = eql.eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, code)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def make_calls(sp):
        return {
            "pack": lambda: (eql.eqlinear_pack_weight(w, wp, Dp, Cp, T, code, eql.EQL_PACK_FWD, sp),
                             eql.eqlinear_pack_weight(w, wpb, Dp, Cp, T, code, eql.EQL_PACK_BWDX, sp)),
            "fwd": lambda: eql.eqlinear_fwd(x, wp, y, N, Cp, Dp, T, code, sp),
            "bwd_x": lambda: eql.eqlinear_bwd_x(dy, wpb, dx, N, Cp, Dp, T, code, sp),
            "bwd_w": lambda: eql.eqlinear_bwd_w(x, dy, dw, ws, ws_bytes, N, Cp, Dp, T, code, sp),
        }

    calls = make_calls(sptr)
    order = ["pack", "fwd", "bwd_x", "bwd_w"]

    def step(events=None):
        for i, k in enumerate(order):
            if events is not None:
                events[k][0].record(stream)
            calls[k]()
            if events is not None:
                events[k][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [{k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in order}
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    per = {k: float(np.mean([e[k][0].elapsed_time(e[k][1]) for e in evs])) for k in order}
    # Device time of each step (the sum of its passes' event windows): spread across steps.
    step_dev = [sum(e[k][0].elapsed_time(e[k][1]) for k in order) for e in evs]

    dense_eq = 2.0 * N * (Dp * T) * (Cp * T)
    actual = 2.0 * (2 * T - 2 if T % 2 == 0 else 2 * T - 1) * N * Dp * Cp if T > 1 else 2.0 * N * Dp * Cp
    n_passes = 3
    value = n_passes * dense_eq / (ms_per_step * 1e-3) / 1e12
    elt = 2 if wl.dtype == "f16" else 4
    bytes_pass = {
        "fwd": elt * (N * Cp * T + N * Dp * T + Dp * Cp * T),
        "bwd_x": elt * (N * Dp * T + N * Cp * T + Dp * Cp * T),
        "bwd_w": elt * (N * Cp * T + N * Dp * T + Dp * Cp * T),
    }
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
    if fwd_kernel_ms >= per["bwd_w"]:
        dom, kname, t_dom = "fwd", "eql_fwd_kernel", 0.5 * fwd_kernel_ms * 1e-3
    else:
        dom, kname, t_dom = "bwd_w", "eqlinear_bwd_w", per["bwd_w"] * 1e-3
    flop_bound = actual / MFMA_PEAK[wl.dtype] / 1e12 >= bytes_pass[dom] / HBM_PEAK / 1e9
    if flop_bound:
        roofline = {"bound": "mfma", "achieved": round(actual / t_dom / 1e12, 1), "peak": MFMA_PEAK[wl.dtype],
                    "unit": "TFLOP/s"}
    else:
        roofline = {"bound": "hbm", "achieved": round(bytes_pass[dom] / t_dom / 1e9, 1), "peak": HBM_PEAK,
                    "unit": "GB/s"}
    roofline["frac"] = round(roofline["achieved"] / roofline["peak"], 4)
    roofline["traffic"] = traffic_for(kname, wl.key)
    roofline["kernel"] = kname
    roofline["ms_per_launch"] = round(t_dom * 1e3, 4)
    roofline["algorithmic"] = ("%.4g FLOP (%s real GEMMs of N x D' x C') and %.4g bytes (x, y, weight) per launch"
                               % (actual, (2 * T - 2) if T % 2 == 0 else (2 * T - 1), bytes_pass[dom]))

    # The same step captured once in a HIP graph and replayed (the library records only
    # kernel launches on the caller's stream).  Reported beside the eager figure.
    graph = None
    if not args.no_graph:
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cap = make_calls(torch.cuda.current_stream().cuda_stream)  # the capturing stream
                for k in order:
                    cap[k]()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(args.steps):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            gms = a.elapsed_time(b) / args.steps
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
        dense = dense_comparator(torch, x, w, dy, T, reps=max(5, min(args.steps, 20)))
        dense["speedup_fwd"] = round(dense["fwd_ms"] / per["fwd"], 3)
        dense["speedup_bwd_x"] = round(dense["bwd_x_ms"] / per["bwd_x"], 3)
        dense["speedup_bwd_w"] = round(dense["bwd_w_ms"] / per["bwd_w"], 3)
        total = dense["fwd_ms"] + dense["bwd_x_ms"] + dense["bwd_w_ms"]
        dense["speedup_fwd_bwd"] = round(total / (per["fwd"] + per["bwd_x"] + per["bwd_w"]), 3)

    fused = None
    if not args.no_fused:
        b = torch.from_numpy(W.make_bias(wl)).to(dev)
        fused = fused_epilogue(torch, eql, x, wp, b, dy, y, N, Cp, Dp, T, code, sptr,
                               reps=max(5, min(args.steps, 20)))
        fused["plain_fwd_ms"] = round(per["fwd"], 4)
        fused["mlp_train_step"] = mlp_train_step(torch, eql, x, w, wp, wpb, b, dy, y, dx, dw, ws, ws_bytes,
                                                 N, Cp, Dp, T, code, sptr, reps=max(5, min(args.steps, 20)))
        del b

    cpu = None
    if not args.no_cpu_baseline:
        del x, dy, y, dx
        torch.cuda.empty_cache()
        cpu = cpu_baseline(wl, x_h, w_h, dy_h, args.cpu_rows, n_passes)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "device_ms_per_step_p10_p50_p90": [round(float(np.percentile(step_dev, q)), 4) for q in (10, 50, 90)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; x,dy ~ N(0,1), w ~ N(0,1/C)%s)" % (
            ", %g%% of rows x%g" % (100 * wl.hot_rows_frac, wl.hot_rows_scale) if wl.hot_rows_frac else ""),
        "config": {"workload": wl.name, "T": T, "N": N, "C": Cp * T, "D": Dp * T,
                   "step": "pack(fwd)+pack(bwd_x)+fwd+bwd_x+bwd_w"},
        "passes": passes,
        "pack_ms": round(per["pack"], 4),
        "mfma_frac_step": round(n_passes * actual / (ms_per_step * 1e-3) / 1e12 / MFMA_PEAK[wl.dtype], 4),
        "roofline": roofline,
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


def mlp_train_step(torch, eql, x, w, wp, wpb, b, dy, y, dx, dw, ws, ws_bytes, N, Cp, Dp, T, code, sptr, reps):
    """One training step of the layer as an MLP expansion, y = GELU(x W^T + b): the
    library's pack (both forms), fused forward keeping pre, epilogue backward (dpre,
    dbias), input and weight gradients on dpre; against the unrolled dense layer in
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
        eql.eqlinear_pack_weight(w, wp, Dp, Cp, T, code, eql.EQL_PACK_FWD, sptr)
        eql.eqlinear_pack_weight(w, wpb, Dp, Cp, T, code, eql.EQL_PACK_BWDX, sptr)
        eql.eqlinear_fwd_fused(x, wp, b, None, y, pre, N, Cp, Dp, T, code, eql.EQL_ACT_GELU, sptr)
        eql.eqlinear_fused_epilogue_bwd(dy, pre, dpre, db, ews, ebytes, N, Dp, T, code, eql.EQL_ACT_GELU, sptr)
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
    res["kind"] = ("pack x2 + eqlinear_fwd_fused(bias, GELU, pre) + eqlinear_fused_epilogue_bwd + bwd_x + bwd_w, "
                   "vs torch on the unrolled dense weight (F.linear, F.gelu, gelu_backward, bias sum, mm x2, "
                   "weight-gradient fold)")
    del Wd, pre, dpre, ews
    torch.cuda.empty_cache()
    return res


def dense_comparator(torch, x, w, dy, T, reps):
    """The unrolled ("replicate and multiply dense") layer on the same GPU: torch
    F.linear and matmuls on the dense (D'T) x (C'T) weight (built outside the timed
    region)."""
    Dp, Cp, _ = w.shape
    g = torch.arange(T, device=w.device)
    idx = (g.view(T, 1) - g.view(1, T)) % T
    Wd = w[:, :, idx].permute(0, 2, 1, 3).reshape(Dp * T, Cp * T).contiguous()
    F = torch.nn.functional

    def timeit(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    dyT = dy.t().contiguous()
    res = {
        "fwd_ms": timeit(lambda: F.linear(x, Wd)),
        "bwd_x_ms": timeit(lambda: torch.matmul(dy, Wd)),
        "bwd_w_ms": timeit(lambda: torch.matmul(dyT, x)),
    }
    res = {k: round(v, 4) for k, v in res.items()}
    res["kind"] = "torch F.linear / matmul on the unrolled dense weight (hipBLASLt)"
    del Wd, dyT
    return res


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
    return {"value": round(flops / total / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": "%s of the same workload x %d run(s), forward + input gradient + weight gradient, "
                      "fp64 dense unroll (%.1f s)" % (what, reps, total)}


if __name__ == "__main__":
    main()
