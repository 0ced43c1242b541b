#!/usr/bin/env python3
"""Benchmark of the quantized-GEMM hot path on one MI355X.

Headline workload (one JSON line on stdout): the W4A16 decode GEMV sweep,
K=4096, N=11008, G=128 (a 7B-class MLP up-projection), fp16 activations with
M = 1, 4 and 8.  One step = one launch at each M.  Every launch reads a
different one of 16 weight sets (16 x 23.2 MB > the 256 MB Infinity Cache),
so the weights stream from HBM.  Steps are recorded once as HIP graphs (the
library's launches on torch's current stream are captured) and replayed,
16 consecutive steps per graph, so host and graph launch overhead does not
pace the GPU (as in a decode loop).

value      = algorithmic bytes of a step / time of a step (GB/s, HBM-bound)
roofline   = the M=1 decode kernel: algorithmic bytes per launch / its mean
             duration, timed with HIP events around a graph of 48 launches;
             peak 8000 GB/s (MI355X HBM3E)
cpu_baseline = the CPU oracle on the same step (all host threads the oracle
             uses), repeated for about 10 s
rows       = every other hot-path row, each timed the same way on its own
             inputs (prefill GEMM, W8A8 GEMM + epilogue, per-token int8
             quantization, KV-cache quant/dequant, INT4 MoE layer, the FP8
             E4M3 path: per-tensor quantization, FP8 GEMM, FP8 KV cache,
             weight-only int8 (W8A16) decode and prefill, and the INT8
             attention chain)

Usage: python bench.py [--steps K] [--warmup W] [--no-rows] [--no-cpu]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 flop/clk (dense)
I8_MFMA_PEAK_TOPS = 5033.2     # 256 CU x 2.4 GHz x 8192 op/clk (dense)
FP8_MFMA_PEAK_TFLOPS = 5000.0  # dense E4M3 MFMA, AMD's published MI355X figure

DEC_K, DEC_N, DEC_G = 4096, 11008, 128
DEC_MS = (1, 4, 8)
MHA_SHAPE = (8, 512, 32, 128)  # batch, tokens (queries = keys), heads, head_dim
ROT = 16


def w4a16_bytes(M, N, K, G):
    return K * N // 2 + 2 * (K // G) * N + 2 * M * K + 2 * M * N


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--no-rows", action="store_true", help="skip the other hot-path rows")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--profile", default=None,
                    choices=["decode1", "decode4", "decode8", "prefill", "w8a8", "quant_act",
                             "kvquant", "kvdequant", "moe", "mha", "copy", "stream",
                             "w8a16_decode1", "w8a16_decode8", "fp8", "fp8kv"],
                    help="launch one workload's kernels --launches times (eagerly) and exit; "
                         "for rocprofv3 runs")
    ap.add_argument("--launches", type=int, default=20)
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="print per-kernel duration statistics (markdown) of a rocprofv3 kernel-trace CSV "
                         "and exit: all dispatches, and each run of at least 40 consecutive dispatches of "
                         "one kernel (the timed graph replays)")
    ap.add_argument("--summarize-pmc", metavar="DIR", nargs="+",
                    help="print per-kernel means (markdown) of rocprofv3 --pmc counter CSVs found under "
                         "the given directories and exit")
    return ap.parse_args()


def _kernel_short(name):
    import re
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", name)


def summarize_trace(path):
    """Markdown statistics of a rocprofv3 kernel-trace CSV (durations in us)."""
    import csv
    import statistics as st
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    by, runs = {}, []
    for r in rows:
        k = _kernel_short(r["Kernel_Name"])
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        by.setdefault(k, []).append(d)
        if runs and runs[-1][0] == k:
            runs[-1][1].append(d)
            runs[-1][3] = int(r["End_Timestamp"])
        else:
            runs.append([k, [d], int(r["Start_Timestamp"]), int(r["End_Timestamp"])])
    q = lambda v, f: sorted(v)[min(len(v) - 1, int(f * len(v)))]
    print("| kernel | dispatches | mean us | median us | p10 us | p90 us |")
    print("|---|---|---|---|---|---|")
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{k}` | {len(v)} | {st.mean(v):.3f} | {st.median(v):.3f} | {q(v, 0.1):.3f} | {q(v, 0.9):.3f} |")
    print()
    print("Runs of at least 40 consecutive dispatches of one kernel (graph replays of one workload):")
    print()
    print("| kernel | dispatches | mean us | median us | p10 us | p90 us | span / dispatch us |")
    print("|---|---|---|---|---|---|---|")
    for k, v, t0, t1 in runs:
        if len(v) >= 40:
            print(f"| `{k}` | {len(v)} | {st.mean(v):.3f} | {st.median(v):.3f} | {q(v, 0.1):.3f} | "
                  f"{q(v, 0.9):.3f} | {(t1 - t0) / 1000.0 / len(v):.3f} |")


def summarize_pmc(dirs):
    """Markdown per-kernel means of rocprofv3 --pmc counter CSVs (one row per kernel and run)."""
    import csv
    import glob
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            agg = {}
            for r in csv.DictReader(open(f)):
                k = _kernel_short(r["Kernel_Name"])
                agg.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            for k, cs in agg.items():
                vals = ", ".join(f"{c} {sum(v) / len(v):.6g}" for c, v in sorted(cs.items()))
                print(f"| {os.path.relpath(f, d)} | `{k}` | {len(next(iter(cs.values())))} | {vals} |")


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_pmc:
        print("| file | kernel | dispatches | mean per dispatch |")
        print("|---|---|---|---|")
        summarize_pmc(args.summarize_pmc)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(each operation would shard by columns, heads or experts); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_quantized_gemm_qgemm_amd as qg
    import qgemm_inputs as qi

    if not os.path.exists(qg.LIB_PATH):
        from bit_quantized_gemm_qgemm_amd import build
        build.build()
    qg.lib()
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if args.profile:
        profile_one(args.profile, args.launches, qg, qi, np, torch, to_dev)
        return

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    def graph_of(fns):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in fns:
                f()
        return g

    def settle(g, warm_s=0.05):
        # untimed replays for at least warm_s seconds: the shader clock takes
        # tens of milliseconds of load to settle (an MFMA-bound GEMM ran 15 %
        # slower in its first 50 ms than afterwards)
        t0, n = time.perf_counter(), 0
        while n < 3 or time.perf_counter() - t0 < warm_s:
            g.replay()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()

    def time_graph(g, launches, reps, warm_s=0.05):
        settle(g, warm_s)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / (reps * launches)  # seconds per launch

    # ------------------------------------------------------------ decode inputs
    log(f"[bench] device {props.name}, {props.multi_processor_count} CUs; building 16 weight sets")
    sets = []
    for r in range(ROT):
        Wb, S = qi.w4a16_weights(DEC_K, DEC_N, DEC_G, 101 + 1000 * r)
        Wf = qg.qgemm_w4a16_prepack(to_dev(Wb), DEC_K, DEC_N)
        sets.append((Wf, to_dev(S)))
    acts = {M: [to_dev(qi.activations(M, DEC_K, 1010 + M + 7919 * r)) for r in range(ROT)]
            for M in DEC_MS}
    outs = {M: torch.empty((M, DEC_N), dtype=torch.float16, device=dev) for M in DEC_MS}
    torch.cuda.synchronize()

    def decode_launch(M, r):
        Wf, S = sets[r % ROT]
        return lambda: qg.qgemm_w4a16(acts[M][r % ROT], Wf, S, DEC_G, Y=outs[M])

    # Step k runs M = 1, 4, 8 on weight sets 3k, 3k+1, 3k+2 (mod ROT).  Steps
    # are replayed from HIP graphs: one graph holds ROT consecutive steps (all
    # rotation offsets, 3 * ROT launches) so that graph-launch overhead is
    # shared as in a decode loop; a remainder of steps uses one-step graphs.
    step_graphs = []
    for k in range(ROT):
        fns = [decode_launch(M, 3 * k + i) for i, M in enumerate(DEC_MS)]
        step_graphs.append(graph_of(fns))
    block_graph = graph_of([decode_launch(M, 3 * k + i) for k in range(ROT)
                            for i, M in enumerate(DEC_MS)])
    step_bytes = sum(w4a16_bytes(M, DEC_N, DEC_K, DEC_G) for M in DEC_MS)
    step_flops = sum(2 * M * DEC_N * DEC_K for M in DEC_MS)

    def run_steps(n):
        for _ in range(n // ROT):
            block_graph.replay()
        for k in range(n % ROT):
            step_graphs[k].replay()

    run_steps(args.warmup)
    settle(block_graph)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    run_steps(args.steps)
    e1.record()
    torch.cuda.synchronize()
    step_s = e0.elapsed_time(e1) * 1e-3 / args.steps
    value = step_bytes / step_s / 1e9
    log(f"[bench] decode step {step_s * 1e6:.2f} us, {value:.1f} GB/s")

    # per-kernel mean durations: graphs of 48 launches of one M, rotating sets
    per_m = {}
    for M in DEC_MS:
        g = graph_of([decode_launch(M, r) for r in range(3 * ROT)])
        t = time_graph(g, 3 * ROT, reps=max(4, args.steps // 16))
        b = w4a16_bytes(M, DEC_N, DEC_K, DEC_G)
        per_m[M] = {"us": round(t * 1e6, 3), "GB/s": round(b / t / 1e9, 1),
                    "hbm_frac": round(b / t / 1e9 / HBM_PEAK_GBS, 4),
                    "TFLOP/s": round(2 * M * DEC_N * DEC_K / t / 1e12, 3)}
        log(f"[bench] decode M={M}: {per_m[M]}")

    b1 = w4a16_bytes(1, DEC_N, DEC_K, DEC_G)
    # achievable read bandwidth at the decode working set: the library's plain
    # streaming-read kernel over 16 rotated buffers of one M=1 launch's bytes,
    # timed like the decode kernel (graph of 48 launches)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    bufs = [torch.empty(b1, dtype=torch.uint8, device=dev).fill_(r) for r in range(ROT)]
    g = graph_of([(lambda r=r: qg.qgemm_stream_read(bufs[r % ROT], sink)) for r in range(3 * ROT)])
    t_s = time_graph(g, 3 * ROT, reps=max(4, args.steps // 16))
    stream_23 = b1 / t_s / 1e9
    del bufs
    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(3)
    g = graph_of([lambda: qg.qgemm_stream_read(big, sink)] * 8)
    t_b = time_graph(g, 8, reps=4)
    stream_1g = (1 << 30) / t_b / 1e9
    del big
    log(f"[bench] stream read: {b1} B x16 rotated {t_s * 1e6:.2f} us {stream_23:.1f} GB/s; "
        f"1 GiB {stream_1g:.1f} GB/s")
    achieved = b1 / (per_m[1]["us"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": read_traffic(), "kernel": "wq_decode_kernel<WB=4,MT=1,NSW=1,KCW=4,G=128,BAL=false> (M=1)",
                "bytes_per_launch": b1, "us_per_launch": per_m[1]["us"],
                "measured_read_ceiling": {"GB/s": round(stream_23, 1), "us": round(t_s * 1e6, 3),
                                          "kernel": "stream_read_kernel, 16-B non-temporal loads",
                                          "working_set": f"{b1} B per launch, 16 rotated buffers"},
                "frac_of_measured_ceiling": round(achieved / stream_23, 4),
                "read_1GiB_GB/s": round(stream_1g, 1),
                "rocprof_trace": read_trace()}
    for M in DEC_MS:
        per_m[M]["frac_of_measured_ceiling"] = round(per_m[M]["GB/s"] / stream_23, 4)

    rows = {}
    if not args.no_rows:
        rows = bench_rows(qg, qi, np, torch, to_dev, graph_of, time_graph, log)
        # every HBM-bound row beside the streaming-read ceiling measured above
        for v in rows.values():
            if "hbm_frac" in v:
                v["frac_of_read_ceiling"] = round(v["GB/s"] / stream_23, 4)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(np, qi, step_bytes, args.cpu_seconds, log)

    line = {
        "metric": "W4A16 qGEMM TFLOP/s & HBM GB/s (% roofline) at decode M=1 and prefill M=2048",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "W4A16 decode GEMV sweep M in {1,4,8}, K=4096 N=11008 G=128, "
                               "16 rotated weight sets",
                   "M": list(DEC_MS), "K": DEC_K, "N": DEC_N, "G": DEC_G,
                   "rotation_sets": ROT, "steps_per_graph": ROT, "step_flops": step_flops,
                   "step_bytes": step_bytes,
                   "device": props.name, "cus": props.multi_processor_count},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "decode": {str(M): v for M, v in per_m.items()},
        "rows": rows,
    }
    print(json.dumps(line), flush=True)


def profile_one(name, launches, qg, qi, np, torch, to_dev):
    """Eager launches of one workload, for counter collection.  Weight sets
    rotate as in the timed runs so reads come from HBM."""
    dev = torch.device("cuda:0")
    if name.startswith("decode"):
        M = int(name[len("decode"):])
        sets = []
        for r in range(ROT):
            Wb, S = qi.w4a16_weights(DEC_K, DEC_N, DEC_G, 101 + 1000 * r)
            sets.append((qg.qgemm_w4a16_prepack(to_dev(Wb), DEC_K, DEC_N), to_dev(S)))
        A = to_dev(qi.activations(M, DEC_K, 1010 + M))
        Y = torch.empty((M, DEC_N), dtype=torch.float16, device=dev)
        torch.cuda.synchronize()
        for i in range(launches):
            Wf, S = sets[i % ROT]
            qg.qgemm_w4a16(A, Wf, S, DEC_G, Y=Y)
    elif name == "prefill":
        M, K, N, G = 2048, 4096, 4096, 128
        probs = []
        for r in range(4):
            A, Wb, S = qi.w4a16_problem(M, K, N, G, 102 + 1000 * r)
            probs.append((to_dev(A), qg.qgemm_w4a16_prepack(to_dev(Wb), K, N), to_dev(S)))
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)
        torch.cuda.synchronize()
        for i in range(launches):
            p = probs[i % len(probs)]
            qg.qgemm_w4a16(p[0], p[1], p[2], G, Y=Y)
    elif name in ("w8a8", "quant_act"):
        M = N = K = 4096
        RQ = 8
        X, Wf16, bias, om = qi.w8a8_problem(M, N, K, 103)
        Xs = [to_dev(X)] + [to_dev(qi.activations(M, K, 1103 + r)) for r in range(1, RQ)]
        qws = [qg.quant_sym_int8(to_dev(Wf16))]
        qws += [qg.quant_sym_int8(to_dev(qi.activations(N, K, 1203 + r))) for r in range(1, RQ)]
        qas = [qg.quant_sym_int8(x) for x in Xs]
        biasd = to_dev(bias)
        Yqs = [torch.empty((M, N), dtype=torch.int8, device=dev) for _ in range(RQ)]
        torch.cuda.synchronize()
        for i in range(launches):
            r = i % RQ
            if name == "w8a8":
                qg.qgemm_w8a8_epilogue(qas[r][0], qws[r][0], qas[r][1], qws[r][1], biasd, float(om), 3,
                                       Y=Yqs[r])
            else:
                qg.quant_sym_int8(Xs[r], Q=qas[r][0], scales=qas[r][1])
    elif name == "stream":
        # the streaming-read reference over 16 rotated buffers of one M=1 decode launch's bytes
        b1 = w4a16_bytes(1, DEC_N, DEC_K, DEC_G)
        bufs = [torch.empty(b1, dtype=torch.uint8, device=dev).fill_(r) for r in range(ROT)]
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        for i in range(launches):
            qg.qgemm_stream_read(bufs[i % ROT], sink)
    elif name in ("kvquant", "kvdequant"):
        kvs = [to_dev(qi.kv_problem(32, 2048, 128, 103 + 1000 * r)) for r in range(16)]
        Q = torch.empty((32, 2048, 128), dtype=torch.int8, device=dev)
        Sk = torch.empty(32 * 2048, dtype=torch.float32, device=dev)
        Xo = torch.empty((32, 2048, 128), dtype=torch.float16, device=dev)
        qs = [qg.quant_sym_int8(kv) for kv in kvs]
        torch.cuda.synchronize()
        for i in range(launches):
            if name == "kvquant":
                qg.quant_sym_int8(kvs[i % 16], Q=Q, scales=Sk)
            else:
                qg.dequant_sym_int8(qs[i % 16][0], qs[i % 16][1], X=Xo)
    elif name == "moe":
        T, H, I, E, topK, G = 256, 4096, 14336, 8, 2, 128
        X, logits, Wg, Wu, Wd, Sg, Su, Sd = qi.moe_problem(T, H, I, E, G, 104)
        pg = torch.cat([qg.qgemm_w4a16_prepack(to_dev(Wg[e]), H, I) for e in range(E)])
        pu = torch.cat([qg.qgemm_w4a16_prepack(to_dev(Wu[e]), H, I) for e in range(E)])
        pd = torch.cat([qg.qgemm_w4a16_prepack(to_dev(Wd[e]), I, H) for e in range(E)])
        args = [to_dev(a) for a in (X, logits)] + [pg, pu, pd] + [to_dev(a) for a in (Sg, Su, Sd)]
        torch.cuda.synchronize()
        for _ in range(launches):
            qg.moe_w4a16(*args, topK, G)
    elif name == "mha":
        B, L, H, D = MHA_SHAPE
        Q, K, V, bias, alpha, pv, om = qi.mha_problem(B, L, L, H, D, 109)
        Qd, Kd, Vd, bd = (to_dev(a) for a in (Q, K, V, bias))
        O = torch.empty((B, L, H, D), dtype=torch.int8, device=dev)
        torch.cuda.synchronize()
        for _ in range(launches):
            qg.mha_int8(Qd, Kd, Vd, alpha, pv, om, bias=bd, O=O)
    elif name.startswith("w8a16_decode"):
        M = int(name[len("w8a16_decode"):])
        sets = []
        for r in range(ROT):
            _, W, S = qi.w8a16_problem(1, DEC_K, DEC_N, DEC_G, 107 + 1000 * r)
            sets.append((qg.qgemm_w8a16_prepack(to_dev(W), DEC_K, DEC_N), to_dev(S)))
        A = to_dev(qi.activations(M, DEC_K, 1070 + M))
        Y = torch.empty((M, DEC_N), dtype=torch.float16, device=dev)
        torch.cuda.synchronize()
        for i in range(launches):
            Wf, S = sets[i % ROT]
            qg.qgemm_w8a16(A, Wf, S, DEC_G, Y=Y)
    elif name == "fp8":
        # per-tensor activation quant and the FP8 GEMM, 8 rotated sets as in the timed rows
        M = N = K = 4096
        RQ = 8
        X, Wf16, _, _ = qi.w8a8_problem(M, N, K, 106)
        Xs = [to_dev(X)] + [to_dev(qi.activations(M, K, 1106 + r)) for r in range(1, RQ)]
        qws = [qg.quant_fp8_e4m3(to_dev(Wf16), per_row=False)]
        qws += [qg.quant_fp8_e4m3(to_dev(qi.activations(N, K, 1206 + r)), per_row=False) for r in range(1, RQ)]
        qas = [qg.quant_fp8_e4m3(x, per_row=False) for x in Xs]
        Ys = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(RQ)]
        torch.cuda.synchronize()
        for i in range(launches):
            r = i % RQ
            qg.quant_fp8_e4m3(Xs[r], per_row=False, Q=qas[r][0], scales=qas[r][1])
            qg.qgemm_fp8(qas[r][0], qws[r][0], qas[r][1], qws[r][1], Y=Ys[r])
    elif name == "fp8kv":
        # per-row E4M3 KV cache quant then dequant, 16 rotated sets
        kvs = [to_dev(qi.kv_problem(32, 2048, 128, 105 + 1000 * r)) for r in range(16)]
        qs = [qg.quant_fp8_e4m3(kv) for kv in kvs]
        Xo = torch.empty((32, 2048, 128), dtype=torch.float16, device=dev)
        torch.cuda.synchronize()
        for i in range(launches):
            r = i % 16
            qg.quant_fp8_e4m3(kvs[r], Q=qs[r][0], scales=qs[r][1])
            qg.dequant_fp8_e4m3(qs[r][0], qs[r][1], X=Xo)
    elif name == "copy":
        # an elementwise kernel of known traffic (reads 256 MiB, writes 256 MiB),
        # to calibrate the HBM byte counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(launches):
            torch.add(src, 1, out=dst)
    torch.cuda.synchronize()
    print(f"profiled {name} x{launches}", file=sys.stderr, flush=True)


# sources of the decode kernel whose HBM counters profiles/decode_traffic.json
# holds, and the build script whose compiler flags shape its code
DECODE_SOURCES = ("csrc/common.hpp", "csrc/wq_tile.hpp", "csrc/wq_pass.hpp", "csrc/wq_gemm.hpp",
                  "csrc/w4a16.hip", "build.py")


def decode_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "bit_quantized_gemm_qgemm_amd", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_profile_record():
    """The committed counter and trace record of the M=1 decode kernel, if it
    was taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
        if d.get("source_sha256_16") != decode_source_hash():
            return None
        return d
    except (OSError, ValueError):
        return None


def read_traffic():
    """HBM bytes per launch of the M=1 decode kernel (counters), or None."""
    d = read_profile_record()
    return None if d is None else d.get("bytes_per_launch")


def read_trace():
    """rocprofv3 kernel-trace figures of the M=1 decode kernel, or None."""
    d = read_profile_record()
    return None if d is None else d.get("trace")


def bench_rows(qg, qi, np, torch, to_dev, graph_of, time_graph, log):
    rows = {}
    dev = torch.device("cuda:0")

    # cfg0: W4A16 M=16 K=N=512 G=128 (launch-latency sized)
    A, Wb, S = qi.w4a16_problem(16, 512, 512, 128, 100)
    Wf = qg.qgemm_w4a16_prepack(to_dev(Wb), 512, 512)
    Ad, Sd = to_dev(A), to_dev(S)
    Y = torch.empty((16, 512), dtype=torch.float16, device=dev)
    g = graph_of([lambda: qg.qgemm_w4a16(Ad, Wf, Sd, 128, Y=Y)] * 32)
    t = time_graph(g, 32, reps=20)
    b = w4a16_bytes(16, 512, 512, 128)
    rows["w4a16_cfg0_M16_K512_N512"] = {"us": round(t * 1e6, 3), "GB/s": round(b / t / 1e9, 1)}
    log(f"[bench] cfg0 {rows['w4a16_cfg0_M16_K512_N512']}")

    # cfg2: prefill M=2048 K=N=4096 G=128, 12 rotated sets (12 x 25 MB)
    M, K, N, G = 2048, 4096, 4096, 128
    R = 12
    probs = []
    for r in range(R):
        A, Wb, S = qi.w4a16_problem(M, K, N, G, 102 + 1000 * r)
        probs.append((to_dev(A), qg.qgemm_w4a16_prepack(to_dev(Wb), K, N), to_dev(S)))
    Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    g = graph_of([(lambda p=p: qg.qgemm_w4a16(p[0], p[1], p[2], G, Y=Y)) for p in probs])
    t = time_graph(g, R, reps=10)
    fl = 2 * M * N * K
    b = w4a16_bytes(M, N, K, G)
    rows["w4a16_prefill_M2048_K4096_N4096"] = {
        "us": round(t * 1e6, 2), "TFLOP/s": round(fl / t / 1e12, 1),
        "mfma_frac": round(fl / t / 1e12 / F16_MFMA_PEAK_TFLOPS, 4), "GB/s": round(b / t / 1e9, 1)}
    log(f"[bench] prefill {rows['w4a16_prefill_M2048_K4096_N4096']}")
    del probs

    # cfg3a: W8A8 M=N=K=4096: per-token activation quant + GEMM with epilogue.
    # RQ = 8 rotated sets (activation quant: 8 x 50 MB in + out; GEMM: 8 x (A, W,
    # Y) = 8 x 50 MB), past the 256 MB Infinity Cache
    M = N = K = 4096
    RQ = 8
    X, Wf16, bias, om = qi.w8a8_problem(M, N, K, 103)
    Xs = [to_dev(X)] + [to_dev(qi.activations(M, K, 1103 + r)) for r in range(1, RQ)]
    qws = [qg.quant_sym_int8(to_dev(Wf16))]
    qws += [qg.quant_sym_int8(to_dev(qi.activations(N, K, 1203 + r))) for r in range(1, RQ)]
    qas = [torch.empty((M, K), dtype=torch.int8, device=dev) for _ in range(RQ)]
    sas = [torch.empty(M, dtype=torch.float32, device=dev) for _ in range(RQ)]
    biasd = to_dev(bias)
    Yqs = [torch.empty((M, N), dtype=torch.int8, device=dev) for _ in range(RQ)]
    gq = graph_of([(lambda r=r: qg.quant_sym_int8(Xs[r], Q=qas[r], scales=sas[r])) for r in range(RQ)])
    tq = time_graph(gq, RQ, reps=10)
    qb = 3 * M * K + 4 * M
    rows["quant_sym_int8_act_4096x4096"] = {"us": round(tq * 1e6, 2), "GB/s": round(qb / tq / 1e9, 1),
                                            "hbm_frac": round(qb / tq / 1e9 / HBM_PEAK_GBS, 4),
                                            "rotation_sets": RQ}
    for r in range(RQ):
        qg.quant_sym_int8(Xs[r], Q=qas[r], scales=sas[r])
    gg = graph_of([(lambda r=r: qg.qgemm_w8a8_epilogue(qas[r], qws[r][0], sas[r], qws[r][1], biasd,
                                                       float(om), 3, Y=Yqs[r])) for r in range(RQ)])
    tg = time_graph(gg, RQ, reps=10)
    ops = 2 * M * N * K
    rows["w8a8_gemm_gelu_4096"] = {"us": round(tg * 1e6, 2), "TOPS": round(ops / tg / 1e12, 1),
                                   "mfma_frac": round(ops / tg / 1e12 / I8_MFMA_PEAK_TOPS, 4),
                                   "rotation_sets": RQ}
    log(f"[bench] w8a8 {rows['w8a8_gemm_gelu_4096']} quant {rows['quant_sym_int8_act_4096x4096']}")
    del Xs, qws, qas, sas, Yqs

    # cfg3b: KV cache [32, 2048, 128] quant + dequant, 16 rotated sets
    R = 16
    kvs = [to_dev(qi.kv_problem(32, 2048, 128, 103 + 1000 * r)) for r in range(R)]
    Xo = torch.empty((32, 2048, 128), dtype=torch.float16, device=dev)
    Qs = [torch.empty((32, 2048, 128), dtype=torch.int8, device=dev) for _ in range(R)]
    Ss = [torch.empty(32 * 2048, dtype=torch.float32, device=dev) for _ in range(R)]
    for r in range(R):
        qg.quant_sym_int8(kvs[r], Q=Qs[r], scales=Ss[r])
    # codes and scales written over the rotated sets too, like the ceiling's copies
    gk = graph_of([(lambda r=r: qg.quant_sym_int8(kvs[r], Q=Qs[r], scales=Ss[r])) for r in range(R)])
    tk = time_graph(gk, R, reps=10)
    gd = graph_of([(lambda r=r: qg.dequant_sym_int8(Qs[r], Ss[r], X=Xo)) for r in range(R)])
    td = time_graph(gd, R, reps=10)
    kb = 3 * 65536 * 128 + 4 * 65536
    # read+write references of the same traffic shapes over the same rotated
    # buffers: 16.8 MB read / 8.4 MB written, and the reverse (no scales)
    gcq = graph_of([(lambda r=r: qg.qgemm_stream_copy(kvs[r], Qs[r])) for r in range(R)])
    tcq = time_graph(gcq, R, reps=10)
    gcd = graph_of([(lambda r=r: qg.qgemm_stream_copy(Qs[r], Xo)) for r in range(R)])
    tcd = time_graph(gcd, R, reps=10)
    cb = 3 * 65536 * 128
    rw = {"quant": {"us": round(tcq * 1e6, 3), "GB/s": round(cb / tcq / 1e9, 1),
                    "shape": "16.8 MB read, 8.4 MB written, 16 rotated sets"},
          "dequant": {"us": round(tcd * 1e6, 3), "GB/s": round(cb / tcd / 1e9, 1),
                      "shape": "8.4 MB read, 16.8 MB written, 16 rotated sets"}}
    rows["kv_quant_32x2048x128"] = {"us": round(tk * 1e6, 2), "GB/s": round(kb / tk / 1e9, 1),
                                    "hbm_frac": round(kb / tk / 1e9 / HBM_PEAK_GBS, 4),
                                    "rw_ceiling": rw["quant"], "frac_of_rw_ceiling": round(tcq / tk, 4)}
    rows["kv_dequant_32x2048x128"] = {"us": round(td * 1e6, 2), "GB/s": round(kb / td / 1e9, 1),
                                      "hbm_frac": round(kb / td / 1e9 / HBM_PEAK_GBS, 4),
                                      "rw_ceiling": rw["dequant"], "frac_of_rw_ceiling": round(tcd / td, 4)}
    log(f"[bench] kv {rows['kv_quant_32x2048x128']} {rows['kv_dequant_32x2048x128']}")
    del kvs, Qs, Ss

    # cfg4: INT4 MoE T=256 H=4096 I=14336 E=8 top-2 G=128 (760 MB working set)
    T, H, I, E, topK, G = 256, 4096, 14336, 8, 2, 128
    X, logits, Wg, Wu, Wd, Sg, Su, Sd = qi.moe_problem(T, H, I, E, G, 104)
    pg = torch.cat([qg.qgemm_w4a16_prepack(to_dev(Wg[e]), H, I) for e in range(E)])
    pu = torch.cat([qg.qgemm_w4a16_prepack(to_dev(Wu[e]), H, I) for e in range(E)])
    pd = torch.cat([qg.qgemm_w4a16_prepack(to_dev(Wd[e]), I, H) for e in range(E)])
    del Wg, Wu, Wd
    Xd, Ld, Sgd, Sud, Sdd = (to_dev(a) for a in (X, logits, Sg, Su, Sd))
    Ym = torch.empty((T, H), dtype=torch.float16, device=dev)
    ids = torch.empty((T, topK), dtype=torch.int32, device=dev)
    wts = torch.empty((T, topK), dtype=torch.float32, device=dev)
    ws = torch.empty(qg.moe_w4a16_workspace_bytes(T, H, I, E, topK), dtype=torch.uint8, device=dev)
    run = lambda: qg.moe_w4a16(Xd, Ld, pg, pu, pd, Sgd, Sud, Sdd, topK, G, Y=Ym, topk_ids=ids,
                               topk_w=wts, workspace=ws)
    gm = graph_of([run] * 4)
    tm = time_graph(gm, 4, reps=5)
    counts = np.bincount(ids.cpu().numpy().ravel(), minlength=E)
    hit = int((counts > 0).sum())
    P = T * topK
    wbytes = hit * (3 * H * I // 2 + 2 * (2 * (H // G) * I + (I // G) * H))
    abytes = 2 * T * H + 2 * T * E + 2 * 2 * P * I + 2 * 4 * P * H + 2 * T * H
    fl = 6 * P * H * I
    rows["moe_T256_H4096_I14336_E8_top2"] = {
        "us": round(tm * 1e6, 2), "TFLOP/s": round(fl / tm / 1e12, 1),
        "mfma_frac": round(fl / tm / 1e12 / F16_MFMA_PEAK_TFLOPS, 4),
        "GB/s": round((wbytes + abytes) / tm / 1e9, 1),
        "hbm_frac": round((wbytes + abytes) / tm / 1e9 / HBM_PEAK_GBS, 4),
        "tokens_per_expert": counts.tolist()}
    log(f"[bench] moe {rows['moe_T256_H4096_I14336_E8_top2']}")
    del pg, pu, pd, Xd, Ld, Sgd, Sud, Sdd, ws

    # FP8 E4M3: per-tensor activation quant 4096 x 4096, FP8 GEMM M=N=K=4096
    # (fp16 out), per-row KV cache [32, 2048, 128] quant + dequant (16 rotated sets)
    # (8 rotated sets each, as for W8A8: 8 x 50 MB)
    M = N = K = 4096
    X, Wf16, _, _ = qi.w8a8_problem(M, N, K, 106)
    Xs = [to_dev(X)] + [to_dev(qi.activations(M, K, 1106 + r)) for r in range(1, RQ)]
    qw8s = [qg.quant_fp8_e4m3(to_dev(Wf16), per_row=False)]
    qw8s += [qg.quant_fp8_e4m3(to_dev(qi.activations(N, K, 1206 + r)), per_row=False)
             for r in range(1, RQ)]
    qa8s = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _ in range(RQ)]
    sa8s = [torch.empty(1, dtype=torch.float32, device=dev) for _ in range(RQ)]
    Y8s = [torch.empty((M, N), dtype=torch.float16, device=dev) for _ in range(RQ)]
    gq = graph_of([(lambda r=r: qg.quant_fp8_e4m3(Xs[r], per_row=False, Q=qa8s[r], scales=sa8s[r]))
                   for r in range(RQ)])
    tq = time_graph(gq, RQ, reps=10)
    qb = 3 * M * K + 4
    rows["fp8_quant_per_tensor_4096x4096"] = {"us": round(tq * 1e6, 2), "GB/s": round(qb / tq / 1e9, 1),
                                              "hbm_frac": round(qb / tq / 1e9 / HBM_PEAK_GBS, 4),
                                              "rotation_sets": RQ}
    for r in range(RQ):
        qg.quant_fp8_e4m3(Xs[r], per_row=False, Q=qa8s[r], scales=sa8s[r])
    gg = graph_of([(lambda r=r: qg.qgemm_fp8(qa8s[r], qw8s[r][0], sa8s[r], qw8s[r][1], Y=Y8s[r]))
                   for r in range(RQ)])
    tg = time_graph(gg, RQ, reps=10)
    fl = 2 * M * N * K
    rows["fp8_gemm_4096"] = {"us": round(tg * 1e6, 2), "TFLOP/s": round(fl / tg / 1e12, 1),
                             "mfma_frac": round(fl / tg / 1e12 / FP8_MFMA_PEAK_TFLOPS, 4),
                             "rotation_sets": RQ}
    log(f"[bench] fp8 gemm {rows['fp8_gemm_4096']} quant {rows['fp8_quant_per_tensor_4096x4096']}")
    del Xs, qw8s, qa8s, sa8s, Y8s
    R = 16
    kvs = [to_dev(qi.kv_problem(32, 2048, 128, 105 + 1000 * r)) for r in range(R)]
    Xo = torch.empty((32, 2048, 128), dtype=torch.float16, device=dev)
    Qs = [torch.empty((32, 2048, 128), dtype=torch.uint8, device=dev) for _ in range(R)]
    Ss = [torch.empty(32 * 2048, dtype=torch.float32, device=dev) for _ in range(R)]
    for r in range(R):
        qg.quant_fp8_e4m3(kvs[r], Q=Qs[r], scales=Ss[r])
    gk = graph_of([(lambda r=r: qg.quant_fp8_e4m3(kvs[r], Q=Qs[r], scales=Ss[r])) for r in range(R)])
    tk = time_graph(gk, R, reps=10)
    gd = graph_of([(lambda r=r: qg.dequant_fp8_e4m3(Qs[r], Ss[r], X=Xo)) for r in range(R)])
    td = time_graph(gd, R, reps=10)
    kb = 3 * 65536 * 128 + 4 * 65536
    rows["fp8_kv_quant_32x2048x128"] = {"us": round(tk * 1e6, 2), "GB/s": round(kb / tk / 1e9, 1),
                                        "hbm_frac": round(kb / tk / 1e9 / HBM_PEAK_GBS, 4),
                                        "rw_ceiling": rw["quant"], "frac_of_rw_ceiling": round(tcq / tk, 4)}
    rows["fp8_kv_dequant_32x2048x128"] = {"us": round(td * 1e6, 2), "GB/s": round(kb / td / 1e9, 1),
                                          "hbm_frac": round(kb / td / 1e9 / HBM_PEAK_GBS, 4),
                                          "rw_ceiling": rw["dequant"], "frac_of_rw_ceiling": round(tcd / td, 4)}
    log(f"[bench] fp8 kv {rows['fp8_kv_quant_32x2048x128']} {rows['fp8_kv_dequant_32x2048x128']}")
    del kvs, Qs, Ss, Xo

    # W8A16 (int8 weights, fp16 activations, G = 128): decode M = 1, 8 on the
    # K = 4096, N = 11008 weights (16 rotated sets of 45 MB) and prefill
    # M = 2048, K = N = 4096 (12 rotated (A, W) sets)
    K, N, G = DEC_K, DEC_N, DEC_G
    sets = []
    for r in range(ROT):
        _, W, S = qi.w8a16_problem(1, K, N, G, 107 + 1000 * r)
        sets.append((qg.qgemm_w8a16_prepack(to_dev(W), K, N), to_dev(S)))
    for M in (1, 8):
        Ad = to_dev(qi.activations(M, K, 1070 + M))
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)
        g = graph_of([(lambda w=w: qg.qgemm_w8a16(Ad, w[0], w[1], G, Y=Y)) for w in sets])
        t = time_graph(g, ROT, reps=20)
        b = K * N + 2 * (K // G) * N + 2 * M * K + 2 * M * N
        rows[f"w8a16_decode_M{M}_K{K}_N{N}"] = {"us": round(t * 1e6, 3), "GB/s": round(b / t / 1e9, 1),
                                                "hbm_frac": round(b / t / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"[bench] w8a16 decode M={M} {rows[f'w8a16_decode_M{M}_K{K}_N{N}']}")
    del sets
    M, K, N, G = 2048, 4096, 4096, 128
    probs = []
    for r in range(12):
        A, W, S = qi.w8a16_problem(M, K, N, G, 108 + 1000 * r)
        probs.append((to_dev(A), qg.qgemm_w8a16_prepack(to_dev(W), K, N), to_dev(S)))
    Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    g = graph_of([(lambda p=p: qg.qgemm_w8a16(p[0], p[1], p[2], G, Y=Y)) for p in probs])
    t = time_graph(g, 12, reps=10)
    fl = 2 * M * N * K
    rows["w8a16_prefill_M2048_K4096_N4096"] = {"us": round(t * 1e6, 2), "TFLOP/s": round(fl / t / 1e12, 1),
                                               "mfma_frac": round(fl / t / 1e12 / F16_MFMA_PEAK_TFLOPS, 4)}
    log(f"[bench] w8a16 prefill {rows['w8a16_prefill_M2048_K4096_N4096']}")
    del probs

    # INT8 attention chain: 8 sequences x 512 tokens, 32 heads of 128 (the W8A8
    # token batch), 4 rotated input sets; algorithmic work 4 B H L^2 D int-ops
    # (Q K^T and P V; the kernel computes Q K^T twice)
    B, L, H, D = MHA_SHAPE
    sets = []
    for r in range(4):
        Q, K, V, bias, alpha, pv, om = qi.mha_problem(B, L, L, H, D, 109 + 1000 * r)
        sets.append(tuple(to_dev(a) for a in (Q, K, V, bias)))
    O = torch.empty((B, L, H, D), dtype=torch.int8, device=dev)
    g = graph_of([(lambda s=s: qg.mha_int8(s[0], s[1], s[2], alpha, pv, om, bias=s[3], O=O)) for s in sets])
    t = time_graph(g, 4, reps=10)
    ops = 4 * B * H * L * L * D
    rows[f"mha_int8_B{B}_L{L}_H{H}_D{D}"] = {"us": round(t * 1e6, 2), "TOPS": round(ops / t / 1e12, 1),
                                            "mfma_frac": round(ops / t / 1e12 / I8_MFMA_PEAK_TOPS, 4)}
    log(f"[bench] mha {rows[f'mha_int8_B{B}_L{L}_H{H}_D{D}']}")
    return rows


def cpu_baseline(np, qi, step_bytes, seconds, log):
    """The oracle, as it stands, on the decode step (full outputs at M=1,4,8)."""
    import oracle
    Wb, S = qi.w4a16_weights(DEC_K, DEC_N, DEC_G, 101)
    acts = {M: qi.activations(M, DEC_K, 1010 + M) for M in DEC_MS}
    reps = 0
    t0 = time.perf_counter()
    while True:
        for M in DEC_MS:
            oracle.w4a16(acts[M], Wb, S, DEC_G)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per_step = el / reps
    log(f"[bench] cpu oracle: {reps} steps in {el:.1f} s")
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(step_bytes / per_step / 1e9, 3), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": model, "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS"),
            "sample": f"{reps} decode steps (M=1,4,8 full outputs, K=4096 N=11008 G=128), "
                      f"{el:.1f} s, fp64 sums, OpenMP over output columns",
            "s_per_step": round(per_step, 4)}


if __name__ == "__main__":
    main()
