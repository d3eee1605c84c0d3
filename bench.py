#!/usr/bin/env python3
"""Benchmark of the weight-quantized decode GEMV on one MI355X.

Default workload (the decode configuration the metric is quoted on):
W8A8 INT8, N=17408, K=5120.  One step = the whole INT8 decode linear layer
(qlin_linear_i8: per-token quantisation + GEMV with its bf16 epilogue; one
kernel for one token, quantiser + GEMV kernels otherwise) once at every
M in {1, 2, 4, 8, 16}.  Weights are cold: each call reads the next of B
rotating weight copies (B * |W| >= 2 x the 256 MB Infinity Cache).
The same line also carries `fp8_m1`: the E4M3 weight-only GEMV at M=1 on the
same shape, per-channel and per-tensor scales, timed the same way.

Prints ONE JSON line.  `value` = algorithmic bytes moved by the timed steps /
their wall time on the GPU (GB/s, inputs already in HBM).  `roofline`
describes the dominant kernel (the GEMV): algorithmic bytes per launch /
mean launch duration, from HIP events recorded on the stream the kernel runs
on around a batch of back-to-back launches (rotating weight copies) per M.
All timed launches are replayed from HIP graphs, so the host's per-call
overhead is not in the measurement.  The whole-step region replays graphs of
--graph-steps consecutive steps (default 10, as a decode step's graph holds
many layers); each replay of a graph adds a fixed cost of several
microseconds, which --graph-steps 1 charges to every step.
`cpu_baseline` times the CPU oracle (oracle/, plain C, OpenMP over rows) on
the host on the same workload.

Other workloads (--workload fp8_decode | fp8_w8a8 | fp8_blk | moe_mxfp4 |
moe_ffn_mxfp4) time the other
entry points the same way; they are used for profiling, the default run is
the int8 one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
PEAK_INT8_TOPS = 5000.0  # MI355X dense int8 matrix-core peak
MALL_BYTES = 256 << 20  # Infinity Cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ----------------------------------------------------------------------------- byte counts

def bytes_gemv_i8(M, N, K):
    return N * K + 4 * N + M * K + 4 * M + 2 * M * N          # W, ws, xq, xs, y


def bytes_act_quant_i8(M, K):
    return 2 * M * K + M * K + 4 * M                           # x, xq, xs


def bytes_gemv_fp8(M, N, K, per_tensor=False):
    return N * K + (4 if per_tensor else 4 * N) + 2 * M * K + 2 * M * N   # W, ws, x, y


def bytes_act_quant_fp8(M, K):
    return 2 * M * K + M * K + 4 * M                           # x, xq, xs


def bytes_gemv_fp8_w8a8(M, N, K):
    return N * K + 4 * N + M * K + 4 * M + 2 * M * N          # W, ws, xq, xs, y


def bytes_blk_call(M, N, K, bn=128, bk=128):
    return N * K + ((N + bn - 1) // bn) * (K // bk) + 2 * M * K + 2 * M * N   # W, ws, x, y


def bytes_blk_gemv(M, N, K):
    return N * K + ((N + 127) // 128) * (K // 128) + M * K + M * (K // 128) + 2 * M * N


def bytes_moe_call(M, N, K, topk, live):
    return live * (N * K // 2 + N * K // 32) + 2 * M * K + 2 * M * N + 8 * M * topk


def bytes_moe_ffn_call(M, H, I, E, topk, live):
    # router rows, live experts' gate/up and down codes + scales, x, y, ids + weights
    return (2 * E * H + live * (2 * I * (H // 2 + H // 32) + H * (I // 2 + I // 32))
            + 2 * M * H + 2 * M * H + 8 * M * topk)


# ----------------------------------------------------------------------------- workloads

# translation units of the kernels the roofline's traffic figure covers (the
# dominant kernel of each workload; the whole call for block FP8, the MoE
# and the expert FFN)
KERNEL_SOURCES = {
    "int8_decode": ("gemv.hip", "ks_i8.hip"),
    "int8_prefill": ("gemm.hip",),
    "int8_prefill_smalln": ("gemv.hip",),
    "fp8_prefill": ("gemm.hip",),
    "fp8_decode": ("gemv.hip", "ks_f8.hip"),
    "fp8_w8a8": ("gemv.hip", "ks_w8a8_e4m3.hip"),
    "fp8_blk": ("act_quant.hip", "gemv.hip"),
    "moe_mxfp4": ("moe.hip",),
    "moe_prefill": ("moe.hip", "moe_prefill.hip"),
    "moe_ffn_mxfp4": ("moe.hip", "routing.hip"),
}


def src_hash(workload, read=None):
    """Hash of the device code behind a workload's traffic figure: its
    translation units and the local headers they include, transitively.
    qlin_launch.hpp (host-side declarations of every launcher) is left out,
    so that adding an entry point elsewhere does not invalidate the counters.
    `read(name) -> bytes` reads a source file (default: the working tree)."""
    csrc = os.path.join(ROOT, "skinny_gemm_qlin_amd", "csrc")
    if read is None:
        def read(name):
            with open(os.path.join(csrc, name), "rb") as fh:
                return fh.read()
    todo, seen, h = list(KERNEL_SOURCES[workload]), set(), hashlib.sha256()
    while todo:
        f = todo.pop()
        if f in seen or f == "qlin_launch.hpp":
            continue
        seen.add(f)
        todo += re.findall(r'^#include "([A-Za-z0-9_.]+)"', read(f).decode(), re.M)
    for f in sorted(seen):
        h.update(f.encode())
        h.update(read(f))
    return h.hexdigest()[:16]


def load_traffic(workload):
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p)).get(workload)
    except Exception:
        return None
    if not t or t.get("src_hash") != src_hash(workload):
        return None  # counters were taken on other kernel code
    return t.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--graph-steps", type=int, default=10,
                    help="steps captured in one HIP graph for the timed region (one replay per graph)")
    ap.add_argument("--workload", default="int8_decode",
                    choices=["int8_decode", "fp8_decode", "fp8_w8a8", "fp8_blk", "moe_mxfp4", "moe_ffn_mxfp4",
                             "int8_prefill", "int8_prefill_smalln", "fp8_prefill", "moe_prefill"])
    ap.add_argument("--ms", default=None, help="comma list of M values (default: the workload's)")
    ap.add_argument("--rotate", type=int, default=0, help="weight copies (0 = enough to defeat the MALL)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--per-tensor", action="store_true", help="fp8_decode: per-tensor weight scale")
    ap.add_argument("--block", default="128,128", help="fp8_blk: block_n,block_k of the weight scales")
    ap.add_argument("--no-fp8", action="store_true", help="int8_decode: skip the fp8_m1 measurement")
    ap.add_argument("--bias", action="store_true", help="INT8 workloads: add a bf16 bias (seeded N(0, 1))")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(one GPU measures the per-GPU kernel at a shard's shape).", file=sys.stderr)
        sys.exit(1)

    import numpy as np
    import torch

    import skinny_gemm_qlin_amd as ql
    from skinny_gemm_qlin_amd import inputs

    ql.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def tb(b):
        return t(b.view(np.int16)).view(torch.bfloat16)

    wl = args.workload
    spec = inputs.WORKLOADS[wl]
    Ms = [int(m) for m in args.ms.split(",")] if args.ms else list(spec["Ms"])
    Mmax = max(Ms)
    N, K = spec.get("N", spec.get("H")), spec.get("K", spec.get("H"))  # the FFN maps H -> H

    # ---------------------------------------------------------------- inputs (seed 0)
    log(f"bench: generating {wl} inputs N={N} K={K} Ms={Ms}")
    if wl in ("int8_decode", "int8_prefill", "int8_prefill_smalln"):
        d = inputs.gen_int8(Mmax, N, K, seed=0)
        wbytes = N * K
    elif wl in ("fp8_decode", "fp8_prefill"):
        d = inputs.gen_fp8(Mmax, N, K, seed=0, per_tensor=args.per_tensor)
        wbytes = N * K
    elif wl == "fp8_w8a8":
        d = inputs.gen_fp8_w8a8(Mmax, N, K, w_fmt=0, seed=0)
        wbytes = N * K
    elif wl == "fp8_blk":
        bn, bk = (int(v) for v in args.block.split(","))
        d = inputs.gen_fp8_blk(Mmax, N, K, seed=0, block_n=bn, block_k=bk)
        wbytes = N * K
    elif wl in ("moe_mxfp4", "moe_prefill"):
        E, topk = spec["E"], spec["topk"]
        d = inputs.gen_moe(Mmax, E, N, K, topk, seed=0)
        wbytes = E * N * K // 2
    else:
        E, topk, I = spec["E"], spec["topk"], spec["I"]
        d = inputs.gen_moe_ffn(Mmax, E, N, I, topk, seed=0)
        wbytes = E * 3 * I * N // 2
    B = args.rotate or max(1, -(-2 * MALL_BYTES // wbytes))
    log(f"bench: {B} rotating weight copies ({B * wbytes / 1e6:.0f} MB)")

    x = tb(d["x"])
    if wl == "moe_ffn_mxfp4":
        wr = tb(d["wr"])
        ffn = [(t(d["w13"]), t(d["s13"]), t(d["w2"]), t(d["s2"]))]
        for i in range(1, B):
            ffn.append(tuple(a.clone() for a in ffn[0]))
        ws_copies = [None] * B
    elif wl in ("moe_mxfp4", "moe_prefill"):
        ws_copies = [t(d["w"])] + [None] * (B - 1)
        s_copies = [t(d["s"])] + [None] * (B - 1)
        for i in range(1, B):
            ws_copies[i] = ws_copies[0].clone()
            s_copies[i] = s_copies[0].clone()
    else:
        w0 = t(d["w"])
        ws_copies = [w0] + [w0.clone() for _ in range(B - 1)]
    sc = t(d["ws"]) if "ws" in d else None
    bias = None
    if args.bias:
        if not wl.startswith("int8"):
            raise SystemExit("--bias applies to the INT8 workloads only")
        bias = tb(inputs.bf16_bits(np.random.default_rng(1).standard_normal(N, dtype=np.float32)))
    bias_bytes = 2 * N if args.bias else 0

    # ---------------------------------------------------------------- per-call launch lists
    xq_buf = torch.empty((Mmax, K), dtype=torch.int8 if wl.startswith("int8") else torch.uint8, device=dev)
    xs_buf = torch.empty((Mmax,), dtype=torch.float32, device=dev)
    xsb_buf = torch.empty((Mmax, K // (bk if wl == "fp8_blk" else 128)), dtype=torch.uint8, device=dev)
    y_buf = torch.empty((Mmax, N), dtype=torch.bfloat16, device=dev)
    if wl in ("moe_mxfp4", "moe_prefill"):
        ids, gw = t(d["ids"]), t(d["gw"])
        ws_moe = torch.empty((ql.qlin_moe_mxfp4_workspace_bytes(Mmax, N, spec["topk"], spec["E"]),),
                             dtype=torch.uint8, device=dev)
        live = len(np.unique(d["ids"]))
        live_of = {M: len(np.unique(d["ids"][:M])) for M in Ms}
    if wl == "moe_ffn_mxfp4":
        ws_ffn = torch.empty((ql.qlin_moe_ffn_mxfp4_workspace_bytes(Mmax, N, spec["I"], spec["topk"], spec["E"]),),
                             dtype=torch.uint8, device=dev)
        ids_buf = torch.empty((Mmax, spec["topk"]), dtype=torch.int32, device=dev)
        gw_buf = torch.empty((Mmax, spec["topk"]), dtype=torch.float32, device=dev)
        # live experts of the device's own routing (the same for every call)
        ql.qlin_moe_ffn_mxfp4(x, wr, *ffn[0], spec["topk"], y=torch.empty((Mmax, N), dtype=torch.bfloat16, device=dev),
                              workspace=ws_ffn, ids=ids_buf, gw=gw_buf)
        torch.cuda.synchronize()
        live_of = {M: len(np.unique(ids_buf[:M].cpu().numpy())) for M in Ms}
        live = live_of[Mmax]

    def launches(M, ci):
        """[(kernel, bytes, fn)] for one call of the workload's entry point."""
        w = ws_copies[ci]
        xm = x[:M]
        if wl == "int8_decode":
            return [("linear_i8", bytes_act_quant_i8(M, K) + bytes_gemv_i8(M, N, K) + bias_bytes,
                     lambda: ql.qlin_linear_i8(xm, w, sc, bias=bias, xq=xq_buf[:M], xs=xs_buf[:M], y=y_buf[:M]))]
        if wl in ("int8_prefill", "int8_prefill_smalln"):
            return [("act_quant_i8", bytes_act_quant_i8(M, K),
                     lambda: ql.qlin_act_quant_i8(xm, xq_buf[:M], xs_buf[:M])),
                    ("gemv_i8", bytes_gemv_i8(M, N, K) + bias_bytes,
                     lambda: ql.qlin_gemv_i8(xq_buf[:M], xs_buf[:M], w, sc, bias=bias, y=y_buf[:M]))]
        if wl in ("fp8_decode", "fp8_prefill"):
            return [("gemv_fp8", bytes_gemv_fp8(M, N, K), lambda: ql.qlin_gemv_fp8(xm, w, sc, y=y_buf[:M]))]
        if wl == "fp8_w8a8":
            return [("act_quant_fp8", bytes_act_quant_fp8(M, K),
                     lambda: ql.qlin_act_quant_fp8(xm, 0, True, xq_buf[:M], xs_buf[:M])),
                    ("gemv_fp8_w8a8", bytes_gemv_fp8_w8a8(M, N, K),
                     lambda: ql.qlin_gemv_fp8_w8a8(xq_buf[:M], xs_buf[:M], w, sc, 0, 0, y=y_buf[:M]))]
        if wl == "fp8_blk":
            return [("act_quant_blk+gemv_fp8_blk", bytes_blk_call(M, N, K, bn, bk),
                     lambda: ql.qlin_gemv_fp8_blk_ex(xm, w, sc, bn, bk, xq=xq_buf[:M], xs=xsb_buf[:M], y=y_buf[:M]))]
        if wl in ("moe_mxfp4", "moe_prefill"):
            return [("moe_mxfp4", bytes_moe_call(M, N, K, spec["topk"], live_of[M]),
                     lambda: ql.qlin_moe_mxfp4(xm, w, s_copies[ci], ids[:M], gw[:M], y=y_buf[:M],
                                               workspace=ws_moe))]
        return [("moe_ffn_mxfp4", bytes_moe_ffn_call(M, N, spec["I"], spec["E"], spec["topk"], live_of[M]),
                 lambda: ql.qlin_moe_ffn_mxfp4(xm, wr, *ffn[ci], spec["topk"], y=y_buf[:M], workspace=ws_ffn,
                                               ids=ids_buf[:M], gw=gw_buf[:M]))]

    def measured(M, ci):
        """[(kernel, bytes, fn)] timed one by one (region B): the step's launches,
        and for the INT8 decode layer also its quantiser and GEMV alone."""
        if wl != "int8_decode":
            return launches(M, ci)
        w = ws_copies[ci]
        xm = x[:M]
        return [("act_quant_i8", bytes_act_quant_i8(M, K),
                 lambda: ql.qlin_act_quant_i8(xm, xq_buf[:M], xs_buf[:M])),
                ("gemv_i8", bytes_gemv_i8(M, N, K) + bias_bytes,
                 lambda: ql.qlin_gemv_i8(xq_buf[:M], xs_buf[:M], w, sc, bias=bias, y=y_buf[:M]))] + launches(M, ci)

    dominant = {"int8_decode": "gemv_i8", "fp8_decode": "gemv_fp8", "fp8_w8a8": "gemv_fp8_w8a8",
                "int8_prefill": "gemv_i8", "int8_prefill_smalln": "gemv_i8", "fp8_prefill": "gemv_fp8",
                "fp8_blk": "act_quant_blk+gemv_fp8_blk", "moe_mxfp4": "moe_mxfp4", "moe_prefill": "moe_mxfp4",
                "moe_ffn_mxfp4": "moe_ffn_mxfp4"}[wl]

    def run_step(step):
        for i, M in enumerate(Ms):
            ci = (step * len(Ms) + i) % B
            for _, _, fn in launches(M, ci):
                fn()

    def capture(fns):
        """Record the launches into one HIP graph (replayed without host overhead).
        The kernels are enqueued on torch's current stream, which is the capture
        stream inside the context."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for fn in fns:
                fn()
        return g

    log(f"bench: warmup {args.warmup} steps (eager)")
    for s in range(args.warmup):
        run_step(s)
    torch.cuda.synchronize()

    # step s uses weight copies (s*len(Ms)+i) % B.  The timed steps are replayed
    # from graphs of `graph_steps` consecutive steps each (the last graph holds
    # the remainder), one graph per distinct starting copy offset.
    S = max(1, min(args.graph_steps, args.steps))

    def step_fns(s):
        fns = []
        for i, M in enumerate(Ms):
            fns += [fn for _, _, fn in launches(M, (s * len(Ms) + i) % B)]
        return fns

    graphs = {}

    def chunk_graph(s0, n):
        key = ((s0 * len(Ms)) % B, n)
        if key not in graphs:
            fns = []
            for s in range(s0, s0 + n):
                fns += step_fns(s)
            graphs[key] = capture(fns)
        return graphs[key]

    chunks = [(s0, min(S, args.steps - s0)) for s0 in range(0, args.steps, S)]
    plan = [chunk_graph(s0, n) for s0, n in chunks]
    for g in plan[:max(1, -(-args.warmup // S))]:
        g.replay()
    torch.cuda.synchronize()

    # timed region A: the whole job, args.steps steps
    log(f"bench: timing {args.steps} steps ({len(plan)} graph replays of up to {S} steps)")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for g in plan:
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps

    # timed region B: per M and kernel, `reps` back-to-back launches (rotating
    # weight copies) in one graph, between two events on the replay stream
    # -> mean launch duration of that kernel.
    reps = max(20, args.steps)
    per_m = {}
    dom_bytes, dom_ms, dom_n, dom_flops = 0, 0.0, 0, 0
    for i, M in enumerate(Ms):
        ent = per_m.setdefault(str(M), {})
        for kidx in range(len(measured(M, 0))):
            kname, nb, _ = measured(M, 0)[kidx]
            g = capture([measured(M, (i + r) % B)[kidx][2] for r in range(reps)])
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            us = ms * 1e3
            ent[kname] = {"us": round(us, 3), "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                          "frac": round(nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            if kname == dominant:
                dom_flops += 2 * M * N * K * reps
                ent[kname]["TFLOPs"] = round(2 * M * N * K / (us * 1e-6) / 1e12, 1)
                dom_bytes += nb * reps
                dom_ms += ms * reps
                dom_n += reps
            del g
        ent["call_us"] = round(sum(ent[k]["us"] for k, _, _ in launches(M, 0)), 3)

    step_bytes = 0
    for M in Ms:
        step_bytes += sum(nb for _, nb, _ in launches(M, 0))
    value = step_bytes * args.steps / (ms_total * 1e-3) / 1e9

    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic = load_traffic(wl)
    if wl in ("int8_prefill", "int8_prefill_smalln", "fp8_prefill"):
        # compute-bound: algorithmic MACs x 2 per launch / launch duration, against
        # the dense matrix-core peak of the instruction's type (int8 5.0 POP/s,
        # bf16 2.5 PFLOP/s)
        peak = PEAK_INT8_TOPS if wl.startswith("int8") else PEAK_BF16_TFLOPS
        tf = dom_flops / (dom_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dominant, "achieved": round(tf, 1), "peak": peak,
                    "unit": "TOP/s" if wl.startswith("int8") else "TFLOP/s", "frac": round(tf / peak, 4),
                    "traffic": traffic, "launches": dom_n}
    else:
        roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "launches": dom_n}

    # ---------------------------------------------------------------- FP8 weight-only, one token
    fp8_m1 = None
    if wl == "int8_decode" and not args.no_fp8:
        fp8_m1 = {}
        for pt in (False, True):
            f = inputs.gen_fp8(1, N, K, seed=0, per_tensor=pt)
            w8 = [t(f["w"])]
            w8 += [w8[0].clone() for _ in range(B - 1)]
            x8, s8 = tb(f["x"]), t(f["ws"])
            y8 = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
            fns = [(lambda wc=w8[r % B]: ql.qlin_gemv_fp8(x8, wc, s8, y=y8)) for r in range(reps)]
            g = capture(fns)
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / reps * 1e3
            nb = bytes_gemv_fp8(1, N, K, per_tensor=pt)
            fp8_m1["per_tensor" if pt else "per_channel"] = {
                "us": round(us, 3), "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                "frac": round(nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "bytes": nb}
            del g, w8
        log(f"bench: fp8 M=1 {fp8_m1}")

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        oracle.set_threads(threads)
        used = oracle.max_threads()
        log(f"bench: cpu_baseline with {used} threads")

        def oracle_step():
            for M in Ms:
                xm = d["x"][:M]
                if wl in ("int8_decode", "int8_prefill", "int8_prefill_smalln"):
                    xq, xs = oracle.act_quant_i8(xm)
                    oracle.gemv_i8(xq, xs, d["w"], d["ws"])
                elif wl in ("fp8_decode", "fp8_prefill"):
                    oracle.gemv_fp8(xm, d["w"], d["ws"])
                elif wl == "fp8_w8a8":
                    xq, xs = oracle.act_quant_fp8(xm, 0, True)
                    oracle.gemv_fp8_w8a8(xq, xs, 0, d["w"], d["ws"], 0)
                elif wl == "fp8_blk":
                    oracle.fp8_blk(xm, d["w"], d["ws"], bn, bk)
                else:
                    if wl in ("moe_mxfp4", "moe_prefill"):
                        oracle.moe_mxfp4(xm, d["w"], d["s"], d["ids"][:M], d["gw"][:M])
                    else:
                        oracle.moe_ffn_route_mxfp4(xm, d["wr"], spec["topk"], d["w13"], d["s13"], d["w2"], d["s2"])

        # a bounded sample: full steps until about 10 s of CPU work (at least
        # 3 steps; no new step starts after 30 s), median step time
        times = []
        t_begin = time.perf_counter()
        while (len(times) < 3 or time.perf_counter() - t_begin < 10.0) and time.perf_counter() - t_begin < 30.0:
            t0 = time.perf_counter()
            oracle_step()
            times.append(time.perf_counter() - t0)
        med = statistics.median(times)
        cpu = {"value": round(step_bytes / med / 1e9, 3), "unit": "GB/s", "cores": used, "kind": "oracle",
               "sample": f"{len(times)} full step(s) of the same workload (Ms={Ms}, N={N}, K={K}), "
                         f"{sum(times):.1f} s of CPU work, median {med:.3f} s per step",
               "cpu_model": cpu_model()}
        # the same oracle on one thread: up to 3 steps, no new step after 20 s
        # (skipped when one step would take longer than that)
        if med * used <= 20.0:
            oracle.set_threads(1)
            t1, t_begin = [], time.perf_counter()
            while len(t1) < 3 and time.perf_counter() - t_begin < 20.0:
                t0 = time.perf_counter()
                oracle_step()
                t1.append(time.perf_counter() - t0)
            oracle.set_threads(used)
            med1 = statistics.median(t1)
            cpu["single_thread"] = {"value": round(step_bytes / med1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                                    "sample": f"{len(t1)} full step(s), median {med1:.3f} s per step"}
        else:
            cpu["single_thread"] = None

    cfg = {"workload": {
        "int8_decode": f"W8A8 INT8 decode linear (qlin_linear_i8: act quant + GEMV, bf16 out) N={N} K={K}, one call per M",
        "fp8_decode": f"E4M3 weight-only GEMV ({'per-tensor' if args.per_tensor else 'per-channel'}) N={N} K={K}",
        "int8_prefill": f"W8A8 INT8 prefill linear (act quant + tiled GEMM, bf16 out) N={N} K={K}, one call per M",
        "int8_prefill_smalln": f"W8A8 INT8 prefill linear on a few-row matrix (act quant + split-K over "
                               f"16-token blocks, bf16 out) N={N} K={K}, one call per M",
        "fp8_prefill": f"E4M3 weight-only prefill GEMM (per-channel) N={N} K={K}, one call per M",
        "fp8_w8a8": f"FP8 W8A8 E4M3 x E4M3 (per-token act quant + GEMV, per-channel ws) N={N} K={K}",
        "fp8_blk": f"{args.block.replace(',', 'x')} block-scaled FP8 (act quant + GEMV) N={N} K={K}",
        "moe_mxfp4": f"MXFP4 top-{spec.get('topk')} expert GEMV E={spec.get('E')} N={N} K={K}",
        "moe_prefill": f"MXFP4 top-{spec.get('topk')} expert GEMM, prefill (pair sort + grouped GEMM + combine) "
                       f"E={spec.get('E')} N={N} K={K}",
        "moe_ffn_mxfp4": f"MXFP4 top-{spec.get('topk')} expert FFN with routing E={spec.get('E')} "
                         f"H={N} I={spec.get('I')} (router, gate/up+SwiGLU, down, combine)",
    }[wl], "N": N, "K": K, "Ms": Ms, "weight_copies": B, "cold_weights": B * wbytes >= 2 * MALL_BYTES,
           "graph_steps": S}
    if wl in ("moe_mxfp4", "moe_ffn_mxfp4", "moe_prefill"):
        cfg["live_experts"] = int(live)
    if args.bias:
        cfg["bias"] = "bf16 [N]"

    out = {
        "metric": "us/call + achieved HBM GB/s (% of peak) for quantized decode GEMV, M=1..16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"int8_decode": "int8", "fp8_decode": "fp8e4m3*bf16->f32", "fp8_w8a8": "fp8e4m3*fp8e4m3->f32",
                  "int8_prefill": "int8", "int8_prefill_smalln": "int8", "fp8_prefill": "fp8e4m3*bf16->f32",
                  "fp8_blk": "fp8e4m3->f32", "moe_mxfp4": "fp4e2m1*bf16->f32", "moe_prefill": "fp4e2m1*bf16->f32",
                  "moe_ffn_mxfp4": "fp4e2m1*bf16->f32"}[wl],
        "data": "synthetic",
        "config": cfg,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fp8_m1": fp8_m1,
        "per_m": per_m,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
