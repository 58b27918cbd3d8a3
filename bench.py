"""Benchmark: dropless MoE layer forward + backward on one MI355X.

One step = one pass of the whole hot path over one batch: top-k routing, dispatch
(index build), gate/up GEMM + SwiGLU, down GEMM, combine, and the backward (dA GEMM +
SwiGLU backward, dW_down, dX GEMM, dW_gate/dW_up, unpermute-sum, router backward).
Inputs are seeded synthetic tensors of the Qwen3-30B-A3B MoE layer shape (T=4096
tokens, H=2048, I=768, 128 experts, top-8, Gaussian router logits) already resident
in HBM.  value = algorithmic TFLOP/s of the step (6RHI forward + 12RHI backward over
the R routed rows; tile padding is not counted).

Prints one JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
[--workload NAME]: the default is the Qwen3-30B-A3B layer; the other names time the
235B-A22B EP=8 share, the Zipf-skewed routing, the fp8_bwd mode and the mxfp8 mode
(MXFP8 forward and backward GEMMs) for the design notes.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 / MXFP8 MFMA
WORKLOADS = {
    "qwen3_30b": "Qwen3-30B-A3B MoE layer, one GPU: T=4096 H=2048 I=768 E=128 top-8, Gaussian router logits, bf16",
    "qwen3_235b_ep8": "Qwen3-235B-A22B MoE layer, one GPU's EP=8 share: 16 of 128 experts, T=16384 H=4096 I=1536 "
                      "top-8, Gaussian router logits, bf16",
    "skew_zipf": "Zipf(1.2)-skewed routing at the 30B shape: T=16384 H=2048 I=768 E=128 top-8, 8 experts empty, bf16",
    "qwen3_235b_ep8_fp8bwd": "fp8_bwd mode at the 235B-A22B EP=8 share: bf16 forward, MXFP8 backward GEMMs",
    "qwen3_235b_ep8_mxfp8": "mxfp8 mode at the 235B-A22B EP=8 share: MXFP8 forward and backward GEMMs",
    "qwen3_30b_mxfp8": "mxfp8 mode at the Qwen3-30B-A3B layer: MXFP8 forward and backward GEMMs",
}
GEMMS = ("fwd_gateup", "fwd_down", "bwd_dA", "bwd_dWd", "bwd_dX", "bwd_dWgu",
         "fwd_gateup_mx", "fwd_down_mx", "bwd_dA_mx", "bwd_dWd_mx", "bwd_dX_mx", "bwd_dWgu_mx")


def kernel_work(name, T, H, I, k, R, El, E_all=0):
    """Algorithmic bytes and flops of one launch of a hot-path kernel (bf16 data).

    Per routed row and per expert weights, as in the design notes: each kernel's
    bytes are the operands it must read and the results it must write once.  The dX
    unpermute also reads the row-dot partials of d_topk_w (WN = 4 per 256 columns of I,
    fp32) and writes d_topk_w."""
    b = 2
    W_gu = 2 * El * H * I * b
    W_d = El * I * H * b
    row_h, row_i, row_2i = R * H * b, R * I * b, R * 2 * I * b
    q = 1 + 1 / 32                       # an MXFP8 element: one byte plus its share of a scale
    table = {
        "fwd_gateup": (row_h + W_gu + row_2i + row_i, 4.0 * R * H * I),
        "fwd_down": (row_i + W_d + row_h, 2.0 * R * H * I),
        "bwd_dA": (row_h + W_d + row_2i + row_i + row_2i, 2.0 * R * H * I),
        "bwd_dWd": (row_i + row_h + W_d, 2.0 * R * H * I),
        "bwd_dX": (row_2i + W_gu + row_h, 4.0 * R * H * I),
        "bwd_dWgu": (row_h + row_2i + W_gu, 4.0 * R * H * I),
        "gather": (T * H * b + row_h, 0.0),
        # router GEMM (E = all experts): x, W_r, fp32 logits / d_logits
        "router_logits": (T * H * b + H * E_all * b + T * E_all * 4, 2.0 * T * H * E_all),
        "router_dx": (T * E_all * 4 + H * E_all * b + 2 * T * H * b, 2.0 * T * H * E_all),
        "combine": (row_h + T * H * b, 0.0),
        "unpermute_dx": (row_h + T * H * b + R * 4 * ((I + 255) // 256) * 4 + T * k * 4, 0.0),
        # MXFP8 GEMMs: fp8 operands, bf16 side inputs and outputs
        "fwd_gateup_mx": ((row_h + W_gu) / b * q + row_2i + row_i, 4.0 * R * H * I),
        "fwd_down_mx": ((row_i + W_d) / b * q + row_h, 2.0 * R * H * I),
        "bwd_dA_mx": ((row_h + W_d) / b * q + row_2i + row_i + row_2i, 2.0 * R * H * I),
        "bwd_dWd_mx": ((row_i + row_h) / b * q + W_d, 2.0 * R * H * I),
        "bwd_dX_mx": ((row_2i + W_gu) / b * q + row_h, 4.0 * R * H * I),
        "bwd_dWgu_mx": ((row_h + row_2i) / b * q + W_gu, 4.0 * R * H * I),
    }
    return table.get(name, (0.0, 0.0))


def sources_sha256():
    """Hash of the library's kernel sources (names and contents of csrc/*)."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "combine_top_router_amd", "csrc", "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` measured with the FETCH_SIZE / WRITE_SIZE counters
    (scaled by a plain copy of known size), as recorded in profiles/hbm_bytes_<workload>.md,
    or None when there is no record or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_bytes_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^sources-sha256 ([0-9a-f]{64})$", text, re.M)
    if not m or m.group(1) != sources_sha256():
        return None
    m = re.search(rf"^traffic-bytes {re.escape(kernel)} (\d+)$", text, re.M)
    return int(m.group(1)) if m else None


def graph_kernel_ms(step_on, stream, names, reps=40, passes=3, warmup=3):
    """Each kernel's marginal time inside a graph replay of the step.

    The step launches its kernels on one stream, so its captured graph is one chain of
    kernel nodes in launch order (`names`, from the library's timing records).  For
    j = 1..n the chain is captured again and cut after its j-th node; each cut graph is
    replayed `reps` times between two events on `stream`, in `passes` interleaved passes
    over j (median per j), and kernel j's time is the difference of the j- and
    (j-1)-node medians.  The prefixes run the same kernels on the buffers of earlier
    full steps, so each reads valid data."""
    import ctypes
    import torch
    hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD)   # torch's HIP runtime, already loaded
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    sh = vp(stream.cuda_stream)

    def ck(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: hipError_t {rc}")

    def chain(graph):
        n = sz(1)
        node = (vp * 1)()
        ck(hip.hipGraphGetRootNodes(graph, node, ctypes.byref(n)), "hipGraphGetRootNodes")
        nodes = [node[0]] if n.value == 1 else []
        while nodes:
            n = sz(0)
            ck(hip.hipGraphNodeGetDependentNodes(vp(nodes[-1]), None, ctypes.byref(n)), "dependents")
            if n.value == 0:
                break
            if n.value != 1:
                raise RuntimeError("the captured step is not one chain")
            nxt = (vp * 1)()
            ck(hip.hipGraphNodeGetDependentNodes(vp(nodes[-1]), nxt, ctypes.byref(n)), "dependents")
            nodes.append(nxt[0])
        return nodes

    def prefix(j):
        graph, gexec = vp(), vp()
        torch.cuda.synchronize()
        ck(hip.hipStreamBeginCapture(sh, 1), "hipStreamBeginCapture")   # thread-local mode
        try:
            with torch.cuda.stream(stream):
                step_on()
        finally:
            ck(hip.hipStreamEndCapture(sh, ctypes.byref(graph)), "hipStreamEndCapture")
        try:
            nodes = chain(graph)
            if len(nodes) != len(names):
                raise RuntimeError(f"captured {len(nodes)} kernels, the step launches {len(names)}")
            for node in reversed(nodes[j:]):
                ck(hip.hipGraphDestroyNode(vp(node)), "hipGraphDestroyNode")
            ck(hip.hipGraphInstantiateWithFlags(ctypes.byref(gexec), graph, ctypes.c_ulonglong(0)),
               "hipGraphInstantiateWithFlags")
        finally:
            hip.hipGraphDestroy(graph)
        return gexec

    def replay_ms(gexec):
        for _ in range(warmup):
            ck(hip.hipGraphLaunch(gexec, sh), "hipGraphLaunch")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            ck(hip.hipGraphLaunch(gexec, sh), "hipGraphLaunch")
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    execs = []
    try:
        for j in range(1, len(names) + 1):
            execs.append(prefix(j))
        runs = [[replay_ms(g) for g in execs] for _ in range(passes)]
    finally:
        for g in execs:
            hip.hipGraphExecDestroy(g)
    t = [0.0] + [float(np.median([r[j] for r in runs])) for j in range(len(names))]
    return [(names[j], t[j + 1] - t[j]) for j in range(len(names))], t[-1]


def cpu_baseline(cfg, inp, budget_s=20.0):
    """The oracle as it stands, on the host cores, over a bounded sample: routing and
    index of all tokens, then the forward of the first n local experts (all their rows),
    then their backward, each timed on its own; n is the whole layer when a first pass
    over one expert says it fits the time budget, else the share that does."""
    from oracle import moe as om
    threads = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        # one GPU's share of the host: 16 threads (the OMP_NUM_THREADS of one-GPU jobs)
        limit = min(16, os.cpu_count() or 1)
        ctx = threadpool_limits(limits=limit)
        threads = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:  # pragma: no cover - threadpoolctl missing
        ctx = None
    try:
        t0 = time.perf_counter()
        idx, w = om.route_topk(inp["logits"], cfg.k, cfg.renorm)
        ix = om.build_index(idx, cfg.e_begin, cfg.e_local)
        t_route = time.perf_counter() - t0
        rel = np.asarray(idx) - cfg.e_begin

        def run(n):
            sub = dict(inp, w_gate=inp["w_gate"][:n], w_up=inp["w_up"][:n], w_down=inp["w_down"][:n])
            f0 = time.perf_counter()
            _, saved = om.layer_forward(sub, cfg.k, 0, n, rel, w)
            f1 = time.perf_counter()
            om.layer_backward(sub, cfg.k, 0, n, rel, w, saved)
            f2 = time.perf_counter()
            return f1 - f0, f2 - f1, int(saved["index"]["offsets"][-1])

        tf1, tb1, r1 = run(1)
        n = cfg.e_local if (tf1 + tb1) * cfg.e_local < budget_s else max(1, int(budget_s / (tf1 + tb1)))
        tf, tb, rows = run(n) if n > 1 else (tf1, tb1, r1)
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    hi = cfg.H * cfg.I
    mx = " (the unquantised oracle; the MXFP8 modes' oracle adds the quantise-dequantise passes)" \
        if "mxfp8" in (cfg.fwd, cfg.bwd) else ""
    return {"value": 18.0 * rows * hi / (tf + tb) / 1e12, "unit": "TFLOP/s", "cores": threads or 1,
            "host_cpus": os.cpu_count(), "kind": "oracle",
            "fwd_TFLOP/s": 6.0 * rows * hi / tf / 1e12, "bwd_TFLOP/s": 12.0 * rows * hi / tb / 1e12,
            "fwd_s": round(tf, 2), "bwd_s": round(tb, 2), "route_index_s": round(t_route, 2),
            "sample": f"fp64 numpy oracle on {threads or 1} BLAS threads of {os.cpu_count()} host CPUs: routing + "
                      f"index of all {cfg.T} tokens, then the forward ({tf:.1f} s) and the backward ({tb:.1f} s) of "
                      f"{n} of {cfg.e_local} local experts ({rows} of {int(ix['counts'].sum())} rows), timed "
                      f"apart{mx}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_30b", choices=list(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of one captured HIP graph per step")
    ap.add_argument("--recompute", action="store_true",
                    help="activation checkpointing: the forward keeps nothing, the backward recomputes the "
                         "gate/up GEMM (value still counts the 18RHI of the layer, not the 4RHI recomputed)")
    ap.add_argument("--router", action="store_true",
                    help="logits from the router GEMM x W_r inside the step (and its backward into dx and dW_r)")
    ap.add_argument("--gather-copy", action="store_true",
                    help="the dispatch writes the gathered token rows Xp, which the GEMMs then read densely "
                         "(default: the GEMM loaders read x through row_src)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run three plain 256 MiB device copies (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {args.gpus} is not supported "
              f"(the path is single-GPU: no collectives)", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    import combine_top_router_amd.lib as L
    from combine_top_router_amd.layer import MoeLayer, stream_handle

    cfg = wl.CONFIGS[args.workload]
    mx = cfg.bwd == "mxfp8"
    mxf = cfg.fwd == "mxfp8"
    inp = wl.make_inputs(cfg)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    bf = torch.bfloat16
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(bf)
    logits = torch.from_numpy(inp["logits"]).to(dev)
    x, wg, wu, wd, dy = t(inp["x"]), t(inp["w_gate"]), t(inp["w_up"]), t(inp["w_down"]), t(inp["dy"])
    layer = MoeLayer(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.e_begin, cfg.e_local, L.MOE_BF16,
                     L.MOE_BWD_MXFP8 if mx else L.MOE_BWD_SAME, cfg.renorm, device=dev,
                     fwd=L.MOE_FWD_MXFP8 if mxf else L.MOE_FWD_SAME, recompute=int(args.recompute),
                     fuse_gather=not args.gather_copy)
    stream = torch.cuda.current_stream()
    if args.router:
        w_r = t(wl.make_router_weight(cfg))
        router_logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=dev)
        dw_r = torch.empty(cfg.H, cfg.E, dtype=bf, device=dev)
        sh, scr = layer.shape, layer.scratch.data_ptr()

    def fwd(st=None):
        if not args.router:
            return layer.forward(logits, x, wg, wu, wd, st)
        h = stream_handle(st)
        L.moe_router_fwd(sh, x.data_ptr(), w_r.data_ptr(), router_logits.data_ptr(), layer.topk_idx.data_ptr(),
                         layer.topk_w.data_ptr(), scr, h)
        layer.inputs = (router_logits, x, wg, wu, wd)
        layer.dispatch(x, st)
        layer.experts(x, wg, wu, wd, st)
        layer.combine(st)
        return layer.y

    def bwd(st=None):
        g = layer.backward(dy, st)
        if args.router:   # x feeds the router too: dx += d_logits W_r^T, and dW_r
            L.moe_router_bwd(sh, x.data_ptr(), w_r.data_ptr(), layer.d_logits.data_ptr(), layer.dx.data_ptr(),
                             layer.dx.data_ptr(), dw_r.data_ptr(), scr, stream_handle(st))
        return g

    def step():
        fwd(stream)
        bwd(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    R = int(layer.offsets[-1].item())

    def timed(run):
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(torch.cuda.current_stream())
        for _ in range(args.steps):
            run()
        stop.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps, time.perf_counter() - t0

    # the step's launches (no allocation, no host synchronisation inside) captured
    # once as a HIP graph and replayed: the same kernels without per-launch gaps
    graph = None
    if not args.eager:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_on = lambda: (fwd(), bwd())
            step_on()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fwd()
            bwd()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
    eager_ms, eager_wall = timed(step)
    if graph is not None:
        ms, wall = timed(graph.replay)
    else:
        ms, wall = eager_ms, eager_wall

    # cold-cache steps: a 1 GiB buffer written before each step evicts L2 and the 256 MB
    # Infinity Cache, and HIP events bracket the step alone (median of five)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    run = graph.replay if graph is not None else step
    for _ in range(5):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(torch.cuda.current_stream())
        run()
        e1.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    cold_ms = float(np.median(cold))
    del flush

    # per-kernel durations from HIP events that each kernel's dispatch stamps (the library's
    # opt-in timing), on the stream the kernels are launched on
    L.moe_timing_enable(True)
    per = {}
    nrep = max(3, min(args.steps, 10))
    part_ms = {"fwd": 0.0, "bwd": 0.0}
    # one untimed step counts the forward's launches; then each step is read once (no host
    # wait between its forward and backward) and split at that count
    fwd(stream)
    n_fwd = len(L.moe_timing_read())
    bwd(stream)
    L.moe_timing_read()
    order = []
    for _ in range(nrep):
        fwd(stream)
        bwd(stream)
        recs = L.moe_timing_read()
        order = [name for name, _ in recs]
        for i, (name, kms) in enumerate(recs):
            per.setdefault(name, []).append(kms)
            part_ms["fwd" if i < n_fwd else "bwd"] += kms / nrep
    L.moe_timing_enable(False)
    # the same kernels' marginal times inside graph replays (prefixes of the captured step)
    in_graph, graph_sum = {}, None
    if graph is not None:
        try:
            marg, graph_sum = graph_kernel_ms(step_on, side, order)
        except RuntimeError as err:   # a step whose captured graph is not one chain of kernels
            print(f"graph prefixes not timed: {err}", file=sys.stderr)
            marg = []
        for name, gms in marg:
            in_graph.setdefault(name, []).append(gms)
    kernels = {}
    for name, v in per.items():
        avg = float(np.mean(v))
        byts, flops = kernel_work(name, cfg.T, cfg.H, cfg.I, cfg.k, R, cfg.e_local, cfg.E)
        kernels[name] = {"ms": round(avg, 4), "launches_per_step": len(v) // nrep,
                         "GB/s": round(byts / avg / 1e6, 1) if byts else None,
                         "TFLOP/s": round(flops / avg / 1e9, 1) if flops else None}
        if name in in_graph:
            kernels[name]["graph_ms"] = round(float(np.mean(in_graph[name])), 4)
    gemm = {n: kernels[n] for n in GEMMS if n in kernels}
    # each GEMM against the dense MFMA peak of its own operand type (bf16 or MXFP8)
    gemm_flops = sum(kernel_work(n, cfg.T, cfg.H, cfg.I, cfg.k, R, cfg.e_local)[1] * v["launches_per_step"]
                     for n, v in gemm.items())
    gemm_peak_ms = sum(v["ms"] * v["launches_per_step"] * (FP8_PEAK_TFLOPS if n.endswith("_mx") else BF16_PEAK_TFLOPS)
                       for n, v in gemm.items())
    dom = max(gemm, key=lambda n: gemm[n]["ms"])
    byts, flops = kernel_work(dom, cfg.T, cfg.H, cfg.I, cfg.k, R, cfg.e_local)
    avg_ms = gemm[dom]["ms"]
    achieved = byts / avg_ms / 1e6
    mfma_peak = FP8_PEAK_TFLOPS if dom.endswith("_mx") else BF16_PEAK_TFLOPS
    # the roofline that bounds the kernel: HBM when its arithmetic intensity is below the ridge
    hbm_bound = flops / byts < mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    traffic = counted_traffic(args.workload, dom)
    if hbm_bound:
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        tf = flops / avg_ms / 1e9
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(tf, 1), "peak": mfma_peak,
                    "unit": "TFLOP/s", "frac": round(tf / mfma_peak, 4), "traffic": traffic}
    roofline.update({"algorithmic_bytes": int(byts), "algorithmic_flops": flops, "avg_ms": avg_ms,
                     "mfma_frac": round(flops / avg_ms / 1e9 / mfma_peak, 4),
                     "hbm_frac": round(achieved / HBM_PEAK_GBS, 4)})

    flops_step = 18.0 * R * cfg.H * cfg.I + (6.0 * cfg.T * cfg.H * cfg.E if args.router else 0.0)
    fwd_ms, bwd_ms = part_ms["fwd"], part_ms["bwd"]
    out = {
        "metric": "MoE layer fwd+bwd ms & TFLOPS at Qwen3-30B-A3B shape, 1 MI355X; % MFMA peak",
        "value": round(flops_step / ms / 1e9, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "launch": "eager" if graph is None else "hip_graph",
        "eager_ms_per_step": round(eager_ms, 4),
        "cold_ms_per_step": round(cold_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("mxfp8" if mxf and mx else "mxfp8+bf16" if mxf else "bf16+mxfp8" if mx else "bf16"),
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload] + (", activation checkpointing (backward recomputes "
                                                            "the gate/up GEMM)" if args.recompute else "")
                   + (", router GEMM x W_r in the step" if args.router else "")
                   + (", gathered rows Xp written by the dispatch" if args.gather_copy else ""),
                   "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "k": cfg.k, "e_local": cfg.e_local, "rows": R},
        # the layer's algorithmic flops (router GEMM included with --router) over the step
        # time, against the dense bf16 peak
        "mfma_frac_step": round(flops_step / ms / 1e9 / BF16_PEAK_TFLOPS, 4),
        # the expert GEMMs only: their flops over the sum of their kernel times, each kernel
        # against its own operand type's dense peak (bf16 2.5, MXFP8 5.0 PFLOP/s)
        "mfma_frac_gemms": round(gemm_flops / gemm_peak_ms / 1e9, 4),
        "kernel_timing": "HIP events stamped by each kernel's own dispatch (hipExtLaunchKernel, no "
                         f"system-scope fence) over {nrep} eagerly launched steps (mean per launch); "
                         "ms_per_step is the graph replay",
        "graph_kernel_timing": "each kernel's marginal time in graph replays: the step's captured chain cut "
                               "after kernel j, minus the chain cut before it (median of 3 passes of 40 replays)",
        "graph_prefix_ms": round(graph_sum, 4) if graph_sum is not None else None,
        "fwd_ms_kernels": round(fwd_ms, 4),
        "bwd_ms_kernels": round(bwd_ms, 4),
        "hbm_frac_combine": round(kernels["combine"]["GB/s"] / HBM_PEAK_GBS, 4) if "combine" in kernels else None,
        "hbm_frac_unpermute_dx": (round(kernels["unpermute_dx"]["GB/s"] / HBM_PEAK_GBS, 4)
                                  if "unpermute_dx" in kernels else None),
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "kernels": kernels,
    }
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = 256 << 20
        del src, dst
    del layer, x, wg, wu, wd, dy, logits
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
