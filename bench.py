#!/usr/bin/env python3
"""Decode-layer benchmark of the NVFP4 path on one MI355X.

Workload: the 27B-class dense decode layer at M=1 (one token): the gate and
up projections 5120 -> 2 x 17408 in one fused launch (fp4_gemv_multi) and the
down projection 17408 -> 5120 (fp4_gemv), NVFP4 weights quantised on the GPU
from seeded bf16 N(0, 0.015) with 0.1% x20 outliers, x ~ N(0,1) bf16.
A step is that layer once; it is captured in a HIP graph (via torch.cuda.CUDAGraph)
over `--copies` distinct weight copies (>= 512 MB together, so the 256 MB
Infinity Cache cannot serve repeats) and replayed.

Printed: ONE JSON line with the effective weight bandwidth (NVFP4 weight
bytes / step time, GB/s), the roofline of the dominant kernel (the GEMV
kernel, live HIP-event timing of its launches), and the CPU oracle timed on
the host's cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
HIDDEN, INTER = 5120, 17408


def weight_bytes(N, K):
    return N * K // 2 + N * K // 16


def kernel_source_sha():
    with open(os.path.join(ROOT, "bit_block_scaled_fp4_amd", "csrc", "gemv.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is absent or was taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", "gemv_dense27b_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("gemv_source_sha") != kernel_source_sha():
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_baseline(seconds: float):
    """The oracle's fp64 product on the down projection (M=1), timed on the
    host cores; returns the effective weight GB/s and what was run."""
    import numpy as np
    import oracle
    from workloads import tensor_bits, x_bits, workload

    wl = workload("dense27b_layer")
    t = wl.tensor("down")
    W = tensor_bits(t)
    x = x_bits(wl.x("x_mid"))
    p, s, g = oracle.quantize(W)
    threads = min(16, os.cpu_count() or 1)
    oracle.gemv(x, p, s, g, threads=threads, with_l1=False)      # warm
    calls, t0 = 0, time.perf_counter()
    while True:
        oracle.gemv(x, p, s, g, threads=threads, with_l1=False)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    gbps = weight_bytes(t.N, t.K) * calls / el / 1e9
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "down projection %dx%d, M=1, fp64 oracle product, %d calls in %.2f s on %d threads"
                      % (t.N, t.K, calls, el, threads)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--copies", type=int, default=12, help="rotating weight copies (12 x 150.4 MB; >= 512 MB per kernel)")
    ap.add_argument("--kernel-reps", type=int, default=400, help="launches per kernel for the per-kernel timing")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--all", action="store_true",
                    help="after the main line, print one JSON line per other workload (small-M, LM head, "
                         "prefill, the 28-layer Qwen3-0.6B-shaped decode sequence, the 1024x1024 GEMV)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 10 device-to-device copies of MIB MiB (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (the decode path is single-GPU); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import bit_block_scaled_fp4_amd as fp4
    from workloads import tensor_bits, x_bits, workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "copies": 10}))
        return
    wl = workload("dense27b_layer")

    def gpu_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    base = {}
    for name in ("gate", "up", "down"):
        base[name] = fp4.quantize(gpu_bf16(tensor_bits(wl.tensor(name))), "tiled")
    torch.cuda.synchronize()
    copies = []
    for c in range(args.copies):
        copies.append({k: fp4.NVFP4Weight(w.packed.clone(), None, w.gscale.clone(), w.N, w.K)
                       for k, w in base.items()})
    del base
    x_in = gpu_bf16(x_bits(wl.x("x_in")))
    x_mid = gpu_bf16(x_bits(wl.x("x_mid")))
    gu = torch.empty((1, 2 * INTER), dtype=torch.float32, device=dev)
    yd = torch.empty((1, HIDDEN), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def gate_up(c):
        w = copies[c]
        fp4.gemv_multi(x_in, [w["gate"], w["up"]], [gu, gu[:, INTER:]], [2 * INTER, 2 * INTER])

    def down(c):
        fp4.gemv(x_mid, copies[c]["down"], out=yd)

    def step(c):
        gate_up(c)
        down(c)

    stream = torch.cuda.Stream(device=dev)       # default priority

    def graph_of(fn, n):
        """Capture fn(0..n-1 cyclic over copies) into one graph."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for c in range(args.copies):     # warm-up launches outside capture
                fn(c)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for i in range(n):
                    fn(i % args.copies)
        torch.cuda.synchronize()
        return g

    def timed(run, n_runs):
        with torch.cuda.stream(stream):
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(n_runs):
                run()
            b.record(stream)
            torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3

    # ---- per-kernel timing (same number of launches of each, so the GEMV
    # kernel's average over all launches is the layer's 1:1 mix)
    reps = max(args.copies, args.kernel_reps // args.copies * args.copies)
    if args.eager:
        t_gu = timed(lambda: [gate_up(i % args.copies) for i in range(reps)], 1) / reps
        t_d = timed(lambda: [down(i % args.copies) for i in range(reps)], 1) / reps
    else:
        g_gu, g_d = graph_of(gate_up, reps), graph_of(down, reps)
        g_gu.replay(); g_d.replay()
        t_gu = timed(g_gu.replay, 1) / reps
        t_d = timed(g_d.replay, 1) / reps

    # ---- the timed steps
    per_graph = args.copies
    if args.eager:
        for i in range(args.warmup):
            with torch.cuda.stream(stream):
                step(i % args.copies)
        total = timed(lambda: [step(i % args.copies) for i in range(args.steps)], 1)
        steps = args.steps
    else:
        g_step = graph_of(step, per_graph)
        for _ in range(max(1, args.warmup // per_graph)):
            g_step.replay()
        n_rep = max(1, args.steps // per_graph)
        total = timed(g_step.replay, n_rep)
        steps = n_rep * per_graph
    t_step = total / steps

    B_gu = weight_bytes(2 * INTER, HIDDEN)
    B_d = weight_bytes(HIDDEN, INTER)
    B_step = B_gu + B_d
    # algorithmic bytes per launch: NVFP4 weights + bf16 activations + fp32 outputs
    A_gu = B_gu + 2 * HIDDEN + 4 * 2 * INTER
    A_d = B_d + 2 * INTER + 4 * HIDDEN
    achieved = (A_gu + A_d) / (t_gu + t_d) / 1e9
    value = B_step / t_step / 1e9
    traffic = load_traffic()

    out = {
        "metric": "4-bit GEMV effective HBM GB/s (% of 8 TB/s peak) at M=1; us/decode-layer",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4(e2m1,e4m3)xbf16->f32",
        "data": "synthetic: seeded bf16 N(0,0.015) weights with 0.1% x20 outliers, quantised on the GPU; x ~ N(0,1)",
        "config": {"workload": "27B-class dense decode layer, M=1: NVFP4 gate_up 5120->34816 (one fused launch) "
                               "+ down 17408->5120", "M": 1, "hidden": HIDDEN, "intermediate": INTER,
                   "weight_bytes_per_step": B_step, "rotating_weight_copies": args.copies,
                   "launch": "eager" if args.eager else "hip graph replay"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "us_per_decode_layer": round(t_step * 1e6, 3),
        "kernels": {
            "gate_up_fused": {"us": round(t_gu * 1e6, 3), "weight_GBps": round(B_gu / t_gu / 1e9, 1)},
            "down_5120x17408": {"us": round(t_d * 1e6, 3), "weight_GBps": round(B_d / t_d / 1e9, 1),
                                "pct_of_hbm_peak": round(100 * B_d / t_d / 1e9 / HBM_PEAK_GBPS, 2)},
        },
        "roofline": {"kernel": "k_gemv<1> (both launches of a step: fused gate_up 2x17408x5120, down 5120x17408)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": (A_gu + A_d) / 2,
                     "avg_launch_us": round((t_gu + t_d) / 2 * 1e6, 3)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)
    if args.all:
        other_workloads(fp4, copies, x_in, x_mid, timed, graph_of_fn(stream), gpu_bf16, dev)


def graph_of_fn(stream):
    import torch

    def graph_of(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            fn(0)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for i in range(n):
                    fn(i)
        torch.cuda.synchronize()
        return g
    return graph_of


def other_workloads(fp4, copies, x_in0, x_mid0, timed, graph_of, gpu_bf16, dev):
    """One JSON line per remaining workload, each timed from a HIP graph over
    rotating weight copies of >= 512 MB where the weights are that large."""
    import torch
    from workloads import tensor_bits, x_bits, workload

    def line(d):
        print(json.dumps(d), flush=True)

    ncp = len(copies)
    # ---- small-M batched decode on the 27B-class layer
    sm = workload("dense27b_smallm")
    for M in (2, 4, 8, 16):
        xi = gpu_bf16(x_bits(sm.x("x_in_m%d" % M)))
        xm = gpu_bf16(x_bits(sm.x("x_mid_m%d" % M)))
        gu = torch.empty((M, 2 * INTER), dtype=torch.float32, device=dev)
        yd = torch.empty((M, HIDDEN), dtype=torch.float32, device=dev)

        def step(i, xi=xi, xm=xm, gu=gu, yd=yd):
            w = copies[i % ncp]
            fp4.gemv_multi(xi, [w["gate"], w["up"]], [gu, gu[:, INTER:]], [2 * INTER, 2 * INTER])
            fp4.gemv(xm, w["down"], out=yd)
        g = graph_of(step, ncp)
        g.replay()
        t = timed(g.replay, 20) / (20 * ncp)
        B = weight_bytes(2 * INTER, HIDDEN) + weight_bytes(HIDDEN, INTER)
        flops = 2.0 * M * (2 * INTER * HIDDEN + HIDDEN * INTER)
        line({"workload": "27B-class dense decode layer, small-M batch", "M": M, "us_per_layer": round(t * 1e6, 3),
              "weight_GBps": round(B / t / 1e9, 1), "pct_of_hbm_peak": round(100 * B / t / 1e9 / HBM_PEAK_GBPS, 2),
              "TFLOPs": round(flops / t / 1e12, 2)})
    # ---- LM head 151936 x 1024, M = 1 and 8
    lm = workload("lm_head")
    base = fp4.quantize(gpu_bf16(tensor_bits(lm.tensor("w"))), "tiled")
    lcp = [base] + [fp4.NVFP4Weight(base.packed.clone(), None, base.gscale.clone(), base.N, base.K)
                    for _ in range(6)]
    for M in (1, 8):
        x = gpu_bf16(x_bits(lm.x("x_m%d" % M)))
        y = torch.empty((M, 151936), dtype=torch.float32, device=dev)
        g = graph_of(lambda i, x=x, y=y: fp4.gemv(x, lcp[i % len(lcp)], out=y), len(lcp) * 8)
        g.replay()
        t = timed(g.replay, 5) / (5 * len(lcp) * 8)
        B = weight_bytes(151936, 1024)
        line({"workload": "LM head 151936x1024", "M": M, "us": round(t * 1e6, 3), "weight_GBps": round(B / t / 1e9, 1),
              "pct_of_hbm_peak": round(100 * B / t / 1e9 / HBM_PEAK_GBPS, 2)})
        # the greedy step: the same product, then the per-row argmax of the logits
        idx = torch.empty((M,), dtype=torch.int32, device=dev)
        g = graph_of(lambda i, x=x, y=y, idx=idx: fp4.lm_head_greedy(x, lcp[i % len(lcp)], logits=y, out=idx),
                     len(lcp) * 8)
        g.replay()
        t2 = timed(g.replay, 5) / (5 * len(lcp) * 8)
        line({"workload": "LM head 151936x1024 + greedy choice (logits, then per-row argmax)", "M": M,
              "us": round(t2 * 1e6, 3), "argmax_added_us": round((t2 - t) * 1e6, 3),
              "weight_GBps": round(B / t2 / 1e9, 1), "pct_of_hbm_peak": round(100 * B / t2 / 1e9 / HBM_PEAK_GBPS, 2)})
    del lcp, base
    # ---- prefill: 2048 tokens x gate_up 5120 -> 34816 (gate and up launches)
    xp = gpu_bf16(x_bits(workload("prefill").x("x")))
    yp = torch.empty((2048, INTER), dtype=torch.float32, device=dev)

    def pf(i):
        w = copies[i % ncp]
        fp4.gemm_prefill(xp, w["gate"], out=yp)
        fp4.gemm_prefill(xp, w["up"], out=yp)
    g = graph_of(pf, 4)
    g.replay()
    t = timed(g.replay, 5) / (5 * 4)
    flops = 2.0 * 2048 * 2 * INTER * HIDDEN
    line({"workload": "prefill GEMM, M=2048 tokens x gate_up 5120->34816 (bf16 MFMA)", "us": round(t * 1e6, 2),
          "TFLOPs": round(flops / t / 1e12, 1), "mfma_bf16_peak_TFLOPs": 2500.0,
          "frac_of_mfma_peak": round(flops / t / 1e12 / 2500.0, 4)})
    # the same product as ONE launch over both tensors (columns of one [2048][34816] output)
    yf = torch.empty((2048, 2 * INTER), dtype=torch.float32, device=dev)

    def pff(i):
        w = copies[i % ncp]
        fp4.gemm_prefill_multi(xp, [w["gate"], w["up"]], [yf[:, :INTER], yf[:, INTER:]], [2 * INTER, 2 * INTER])
    g = graph_of(pff, 4)
    g.replay()
    t = timed(g.replay, 5) / (5 * 4)
    line({"workload": "prefill GEMM, M=2048 tokens x gate_up 5120->34816 (bf16 MFMA, one fused launch)",
          "us": round(t * 1e6, 2), "TFLOPs": round(flops / t / 1e12, 1), "mfma_bf16_peak_TFLOPs": 2500.0,
          "frac_of_mfma_peak": round(flops / t / 1e12 / 2500.0, 4)})
    del yp, yf
    # reference only (not this library): the same product as a dense bf16 GEMM in the vendor library
    # (torch.matmul -> hipBLASLt), bf16 weights (4x the bytes of NVFP4), no decode, bf16 and fp32 output
    wd = [torch.randn(2 * INTER, HIDDEN, device=dev, dtype=torch.bfloat16) for _ in range(4)]
    for name, fn in (("bf16 out", lambda i: torch.matmul(xp, wd[i % 4].t())),
                     ("fp32 out", lambda i: torch.mm(xp, wd[i % 4].t(), out_dtype=torch.float32))):
        for i in range(8):
            fn(i)
        tr = timed(lambda c=[0]: (fn(c[0]), c.__setitem__(0, c[0] + 1)), 20) / 20
        line({"workload": "reference: dense bf16 GEMM of the same prefill shape in hipBLASLt (torch.matmul), "
                          "bf16 weights, " + name, "us": round(tr * 1e6, 2), "TFLOPs": round(flops / tr / 1e12, 1)})
    del wd, xp
    # ---- Qwen3-0.6B-shaped decode: 28 layers x (QKV fused, O, gate_up fused, down), M = 1
    wl = workload("qwen3_0p6b_decode")
    layers = []
    for l in range(1, 29):
        ws = {t: fp4.quantize(gpu_bf16(tensor_bits(wl.tensor("L%d.%s" % (l, t)))), "tiled")
              for t in ("q", "k", "v", "o", "gate", "up", "down")}
        xs = {k: gpu_bf16(x_bits(wl.x("L%d.x%d" % (l, k)))) for k in (1024, 2048, 3072)}
        layers.append((ws, xs))
    sets = [layers] + [[({t: fp4.NVFP4Weight(w.packed.clone(), None, w.gscale.clone(), w.N, w.K)
                          for t, w in ws.items()}, xs) for ws, xs in layers] for _ in range(2)]
    qkv = torch.empty((1, 4096), dtype=torch.float32, device=dev)
    o = torch.empty((1, 1024), dtype=torch.float32, device=dev)
    gu = torch.empty((1, 6144), dtype=torch.float32, device=dev)
    d = torch.empty((1, 1024), dtype=torch.float32, device=dev)

    def token(i):
        for ws, xs in sets[i % len(sets)]:
            fp4.gemv_multi(xs[1024], [ws["q"], ws["k"], ws["v"]], [qkv, qkv[:, 2048:], qkv[:, 3072:]], [4096] * 3)
            fp4.gemv(xs[2048], ws["o"], out=o)
            fp4.gemv_multi(xs[1024], [ws["gate"], ws["up"]], [gu, gu[:, 3072:]], [6144] * 2)
            fp4.gemv(xs[3072], ws["down"], out=d)
    g = graph_of(token, len(sets))
    g.replay()
    t = timed(g.replay, 10) / (10 * len(sets) * 28)
    B = 8847360
    line({"workload": "Qwen3-0.6B-shaped decode, 28 layers x (QKV fused, O, gate_up fused, down), M=1, one HIP graph",
          "us_per_decode_layer": round(t * 1e6, 3), "weight_GBps": round(B / t / 1e9, 1),
          "pct_of_hbm_peak": round(100 * B / t / 1e9 / HBM_PEAK_GBPS, 2), "launches_per_layer": 4})
    del sets, layers
    # ---- load-time quantisation of the 27B down projection (5120 x 17408) from bf16 and from an FP8 release.
    # The rule needs the tensor amax before any block can be encoded, so the input is read twice; the
    # algorithmic bytes are 2 input reads + the 9/16 byte per element written.
    from workloads import fp8_release
    Nq, Kq = HIDDEN, INTER
    Wb = gpu_bf16(tensor_bits(workload("dense27b_layer").tensor("down")))
    codes, sc = fp8_release((Nq, Kq), 32, 0.015, outlier_p=0.001, outlier_scale=20)
    Wf = torch.from_numpy(codes).to(dev)
    Sf = torch.tensor([float(sc)], dtype=torch.float32, device=dev)
    for name, ebytes, q in (("bf16", 2, lambda o: fp4.quantize(Wb, "tiled", out=o)),
                            ("fp8 E4M3 + tensor scale", 1, lambda o: fp4.quantize_fp8(Wf, Sf, "tiled", out=o))):
        o = q(None)
        g = graph_of(lambda i, q=q, o=o: q(o), 4)
        g.replay()
        t = timed(g.replay, 5) / (5 * 4)
        alg = 2 * ebytes * Nq * Kq + weight_bytes(Nq, Kq)
        line({"workload": "load-time NVFP4 quantisation, 5120x17408 from %s (tiled output)" % name,
              "us": round(t * 1e6, 2), "input_GBps": round(ebytes * Nq * Kq / t / 1e9, 1),
              "algorithmic_GBps": round(alg / t / 1e9, 1), "pct_of_hbm_peak": round(100 * alg / t / 1e9 / HBM_PEAK_GBPS, 2)})
        del o
    del Wb, Wf
    # ---- single 1024 x 1024 GEMV (latency)
    w0 = workload("gemv_1024")
    base = fp4.quantize(gpu_bf16(tensor_bits(w0.tensor("w"))), "tiled")
    cps = [base] + [fp4.NVFP4Weight(base.packed.clone(), None, base.gscale.clone(), base.N, base.K)
                    for _ in range(899)]
    x = gpu_bf16(x_bits(w0.x("x")))
    y = torch.empty((1, 1024), dtype=torch.float32, device=dev)
    g = graph_of(lambda i: fp4.gemv(x, cps[i % len(cps)], out=y), len(cps))
    g.replay()
    t = timed(g.replay, 3) / (3 * len(cps))
    line({"workload": "single NVFP4 GEMV 1024x1024, M=1 (900 rotating copies)", "us": round(t * 1e6, 3),
          "weight_GBps": round(589824 / t / 1e9, 1)})


if __name__ == "__main__":
    main()
