#!/usr/bin/env python3
"""Decode-layer benchmark of the NVFP4 path on one MI355X.

Headline workload: the 27B-class dense decode layer at M=1 (one token): the
gate and up projections 5120 -> 2 x 17408 in one fused launch
(fp4_gemv_multi) and the down projection 17408 -> 5120 (fp4_gemv), NVFP4
weights quantised on the GPU from seeded bf16 N(0, 0.015) with 0.1% x20
outliers, x ~ N(0,1) bf16. A step is that layer once. The K timed steps are
one HIP graph (captured through torch.cuda.CUDAGraph) of exactly K steps that
cycle over `--copies` distinct weight copies (>= 512 MB together, so the
256 MB Infinity Cache cannot serve repeats); the graph is replayed in 7
timed windows and the median window gives `value` (min and max reported).

Printed: ONE JSON line with
  - value: NVFP4 weight bytes per step / step time (GB/s), ms_per_step;
  - roofline: the dominant kernel (the M <= 4 GEMV kernel, both launches of a
    step) from HIP events on its launch stream, against the 8 TB/s peak,
    with HBM traffic from the committed rocprofv3 counter summary;
  - read_ceiling: a plain streaming read of the same byte counts in the best
    of a few launch shapes (the attainable ceiling of a one-launch read);
  - configs: every workload (the 1024x1024 GEMV, the Qwen3-0.6B-shaped
    28-layer decode sequence, this layer, its small-M batches, the LM head
    with and without the greedy choice, the prefill GEMM, the load-time
    quantiser), each timed the same way;
  - clocks: GPU clock readings around the run;
  - cpu_baseline: the oracle timed on the host's cores on bounded samples.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP4_PEAK_TFLOPS = 10100.0   # dense FP4 matrix-core peak
HIDDEN, INTER = 5120, 17408
REPS = 7            # timed windows per measurement
CPU_THREADS = 16    # the host cores one GPU's job may use


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


def progress(msg):
    """One line on stderr per finished stage (the JSON line stays alone on stdout)."""
    print("[bench] %s" % msg, file=sys.stderr, flush=True)


class _Results(dict):
    """The per-config results; reports each line as it is measured."""

    def __setitem__(self, key, value):
        super().__setitem__(key, value)
        progress("%s measured" % key)


def stats(xs):
    return {"median": round(statistics.median(xs), 4), "min": round(min(xs), 4), "max": round(max(xs), 4)}


def clocks():
    """The GPU's current core and memory clock levels from sysfs (the DPM
    tables with the active level marked), or the reason they are missing.
    Read from files so that no program is started from this process."""
    import glob
    try:
        out = {}
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            try:
                with open(os.path.join(dev, "vendor")) as f:
                    if f.read().strip() != "0x1002":
                        continue
                for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
                    with open(os.path.join(dev, name)) as f:
                        cur = [ln.strip() for ln in f if ln.strip().endswith("*")]
                    out[name] = cur[0] if cur else None
            except OSError:
                continue
            if out:
                out["device"] = dev
                return out
    except Exception:  # noqa: BLE001  (fall through to the library)
        pass
    try:  # the amd-smi library (no subprocess)
        import amdsmi
        amdsmi.amdsmi_init()
        try:
            h = amdsmi.amdsmi_get_processor_handles()[0]
            out = {}
            for name, kind in (("gfx", amdsmi.AmdSmiClkType.GFX), ("mem", amdsmi.AmdSmiClkType.MEM)):
                info = amdsmi.amdsmi_get_clock_info(h, kind)
                out[name + "_mhz"] = {k: info[k] for k in ("clk", "min_clk", "max_clk") if k in info}
            return out
        finally:
            amdsmi.amdsmi_shut_down()
    except Exception as e:  # noqa: BLE001  (missing clocks must not stop the benchmark)
        return {"error": "no clock source: %s" % str(e)[:200]}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(seconds: float):
    """The oracle (plain C, fp64 sums) on the host cores: the down projection
    5120x17408 at M=1 on one thread and on CPU_THREADS threads, the quantiser
    on 640 rows of it, and 2 token rows of the 2048-token prefill product."""
    import numpy as np
    import oracle
    from workloads import tensor_bits, x_bits, workload

    wl = workload("dense27b_layer")
    t = wl.tensor("down")
    W = tensor_bits(t)
    x = x_bits(wl.x("x_mid"))
    p, s, g = oracle.quantize(W)
    B = weight_bytes(t.N, t.K)

    def rate(threads, budget):
        oracle.gemv(x, p, s, g, threads=threads, with_l1=False)     # warm
        calls, t0 = 0, time.perf_counter()
        while True:
            oracle.gemv(x, p, s, g, threads=threads, with_l1=False)
            calls += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return B * calls / el / 1e9, calls, el

    threads = min(CPU_THREADS, os.cpu_count() or 1)
    multi, calls_m, el_m = rate(threads, seconds / 2)
    single, calls_1, el_1 = rate(1, seconds / 4)
    rows = 640
    t0 = time.perf_counter()
    oracle.quantize(np.ascontiguousarray(W[:rows]))
    q_el = time.perf_counter() - t0
    # prefill: 2 token rows of x [2048][5120] against the gate projection
    pf = workload("prefill")
    xp = x_bits(pf.x("x"))[[0, 2047]]
    pg, sg, gg = oracle.quantize(tensor_bits(wl.tensor("gate")))
    t0 = time.perf_counter()
    oracle.gemv(xp, pg, sg, gg, threads=threads, with_l1=False)
    p_el = time.perf_counter() - t0
    return {"value": round(multi, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "down projection %dx%d, M=1, fp64 oracle product: %d calls in %.2f s on %d threads"
                      % (t.N, t.K, calls_m, el_m, threads),
            "host_cores": os.cpu_count(), "threads_used": threads, "cpu_model": cpu_model(),
            "single_thread": {"value": round(single, 3), "unit": "GB/s",
                              "sample": "%d calls in %.2f s on 1 thread" % (calls_1, el_1)},
            "quantiser": {"value": round(rows * t.K / q_el / 1e6, 2), "unit": "Melem/s", "threads": 1,
                          "sample": "oracle quantisation of %d rows x %d of the down projection in %.2f s"
                                    % (rows, t.K, q_el)},
            "prefill": {"value": round(2 * 2 * 17408 * 5120 / p_el / 1e9, 3), "unit": "GFLOP/s",
                        "threads": threads,
                        "sample": "2 token rows x gate 17408x5120 of the 2048-token prefill in %.2f s" % p_el}}


class Timer:
    """HIP graph capture and event timing on one dedicated stream (default
    priority): the events are recorded on the stream the kernels run on."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.Stream()

    def graph(self, fn, n):
        """fn(0..n-1) captured into one graph (fn(0) runs once eagerly first)."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            fn(0)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=self.stream):
                for i in range(n):
                    fn(i)
        torch.cuda.synchronize()
        return g

    def windows(self, g, per, reps=REPS):
        """Replay g once (warm), then `reps` timed replays; microseconds per
        unit (`per` units per replay) of each. Before each window a spin
        kernel keeps the stream busy while the host submits the start event
        and the graph, so the window holds the graph's GPU work and not the
        host's submission latency."""
        torch = self.torch
        g.replay()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(self.stream):
                torch.cuda._sleep(1 << 21)
                a.record(self.stream)
                g.replay()
                b.record(self.stream)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) * 1e3 / per)
        return out

    def time_calls(self, fn, n, reps=REPS):
        g = self.graph(fn, n)
        r = self.windows(g, n, reps)
        del g
        return r


def read_ceiling(fp4, torch, timer, nbytes_list):
    """Best median time of a plain streaming read of each byte count over a
    few launch shapes (workgroups, waves, loads in flight per wave, order,
    non-temporal), rotating over >= 512 MB of distinct buffers."""
    lib = fp4.raw()
    lib.fp4_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.fp4_bench_stream_read.restype = ctypes.c_int
    pool_bytes = 1200 << 20
    pool = torch.full((pool_bytes,), 7, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    shapes = [(1024, 8, 1, 0, 1), (512, 16, 1, 0, 1), (2048, 4, 1, 0, 1), (256, 8, 4, 0, 1)]
    out = {}
    for nbytes in nbytes_list:
        nbuf = pool_bytes // nbytes
        stride = (pool_bytes // nbuf) // 4096 * 4096
        best = None
        for wgs, waves, unroll, mode, nt in shapes:
            def fn(i, wgs=wgs, waves=waves, unroll=unroll, mode=mode, nt=nt):
                rc = lib.fp4_bench_stream_read(pool.data_ptr() + (i % nbuf) * stride, nbytes, wgs, waves, unroll,
                                               mode, nt, sink.data_ptr(), timer.stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError("fp4_bench_stream_read: %d" % rc)
            t = statistics.median(timer.time_calls(fn, 4 * nbuf))
            if best is None or t < best[0]:
                best = (t, {"workgroups": wgs, "waves": waves, "loads_in_flight_per_wave": unroll,
                            "order": "round-robin 1 KB blocks" if mode == 0 else "contiguous per wave",
                            "nontemporal": bool(nt)})
        out[nbytes] = {"us": round(best[0], 3), "GBps": round(nbytes / best[0] / 1e3, 1), "shape": best[1]}
    del pool
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="steps per timed window (exactly this many)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=12, help="rotating weight copies (12 x 150.4 MB; >= 512 MB per kernel)")
    ap.add_argument("--kernel-reps", type=int, default=240, help="launches per kernel for the per-kernel timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="wall time of the oracle product samples")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config lines (headline only)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 10 device-to-device copies of MIB MiB (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (the decode path is single-GPU); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("--steps must be >= 1", file=sys.stderr)
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
    clocks_before = clocks()
    wl = workload("dense27b_layer")

    def gpu_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def clone(w):
        return fp4.NVFP4Weight(w.packed.clone(), None, w.gscale.clone(), w.N, w.K)

    base = {name: fp4.quantize(gpu_bf16(tensor_bits(wl.tensor(name))), "tiled") for name in ("gate", "up", "down")}
    torch.cuda.synchronize()
    copies = [base] + [{k: clone(w) for k, w in base.items()} for _ in range(args.copies - 1)]
    ncp = len(copies)
    x_in = gpu_bf16(x_bits(wl.x("x_in")))
    x_mid = gpu_bf16(x_bits(wl.x("x_mid")))
    gu = torch.empty((1, 2 * INTER), dtype=torch.float32, device=dev)
    yd = torch.empty((1, HIDDEN), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def gate_up(c):
        w = copies[c % ncp]
        fp4.gemv_multi(x_in, [w["gate"], w["up"]], [gu, gu[:, INTER:]], [2 * INTER, 2 * INTER])

    def down(c):
        fp4.gemv(x_mid, copies[c % ncp]["down"], out=yd)

    def step(c):
        gate_up(c)
        down(c)

    timer = Timer(torch)
    # ---- the timed steps: one graph of exactly `steps` steps, REPS windows
    if args.warmup > 0:
        gw = timer.graph(step, args.warmup)
        gw.replay()
        torch.cuda.synchronize()
        del gw
    g_step = timer.graph(step, args.steps)
    win = timer.windows(g_step, args.steps)
    progress("headline steps timed")
    del g_step
    t_step = statistics.median(win) * 1e-6

    # ---- per-kernel timing (graphs of one kernel's launches over the copies)
    reps = max(ncp, args.kernel_reps // ncp * ncp)
    k_gu = timer.time_calls(gate_up, reps)
    k_d = timer.time_calls(down, reps)
    t_gu, t_d = statistics.median(k_gu) * 1e-6, statistics.median(k_d) * 1e-6

    B_gu = weight_bytes(2 * INTER, HIDDEN)
    B_d = weight_bytes(HIDDEN, INTER)
    B_step = B_gu + B_d
    # algorithmic bytes per launch: NVFP4 weights + bf16 activations + fp32 outputs
    A_gu = B_gu + 2 * HIDDEN + 4 * 2 * INTER
    A_d = B_d + 2 * INTER + 4 * HIDDEN
    achieved = (A_gu + A_d) / (t_gu + t_d) / 1e9
    value = B_step / t_step / 1e9
    tiled_d = fp4.layout_bytes(HIDDEN, INTER)[0]
    tiled_gu = 2 * fp4.layout_bytes(INTER, HIDDEN)[0]
    progress("per-kernel launches timed")
    ceil = read_ceiling(fp4, torch, timer, [tiled_d, tiled_gu])
    progress("read ceiling measured")
    c_d, c_gu = ceil[tiled_d]["us"], ceil[tiled_gu]["us"]

    out = {
        "metric": "4-bit GEMV effective HBM GB/s (% of 8 TB/s peak) at M=1; us/decode-layer",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4(e2m1,e4m3)xbf16->f32",
        "data": "synthetic: seeded bf16 N(0,0.015) weights with 0.1% x20 outliers, quantised on the GPU; x ~ N(0,1)",
        "config": {"workload": "27B-class dense decode layer, M=1: NVFP4 gate_up 5120->34816 (one fused launch) "
                               "+ down 17408->5120", "M": 1, "hidden": HIDDEN, "intermediate": INTER,
                   "weight_bytes_per_step": B_step, "rotating_weight_copies": ncp,
                   "launch": "one hip graph of exactly `steps` steps, %d timed windows" % REPS},
        "windows_us_per_step": stats(win),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "us_per_decode_layer": round(t_step * 1e6, 3),
        "kernels": {
            "gate_up_fused": {"us": stats(k_gu), "weight_GBps": round(B_gu / t_gu / 1e9, 1),
                              "pct_of_hbm_peak": round(100 * B_gu / t_gu / 1e9 / HBM_PEAK_GBPS, 2),
                              "read_ceiling_us": c_gu, "pct_of_read_ceiling": round(100 * c_gu / (t_gu * 1e6), 1)},
            "down_5120x17408": {"us": stats(k_d), "weight_GBps": round(B_d / t_d / 1e9, 1),
                                "pct_of_hbm_peak": round(100 * B_d / t_d / 1e9 / HBM_PEAK_GBPS, 2),
                                "read_ceiling_us": c_d, "pct_of_read_ceiling": round(100 * c_d / (t_d * 1e6), 1)},
        },
        "read_ceiling": {str(k): v for k, v in ceil.items()},
        "roofline": {"kernel": "k_gemv<1> (both launches of a step: fused gate_up 2x17408x5120, down 5120x17408)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": load_traffic(),
                     "algorithmic_bytes_per_launch": (A_gu + A_d) / 2,
                     "avg_launch_us": round((t_gu + t_d) / 2 * 1e6, 3)},
    }
    del copies[1:]
    if not args.no_configs:
        out["configs"] = other_configs(fp4, torch, timer, copies[0], gpu_bf16, dev, x_in, x_mid)
    out["clocks"] = {"before": clocks_before, "after": clocks()}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


def other_configs(fp4, torch, timer, w27, gpu_bf16, dev, x_in0, x_mid0):
    """Every workload, timed as the headline is: a graph over rotating weight
    copies (>= 512 MB where the weights are large), median/min/max of REPS
    windows. Products with a K split use a workspace (fp4_*_ws forms)."""
    from workloads import fp8_release, tensor_bits, x_bits, workload

    res = _Results()

    def clone(w):
        return fp4.NVFP4Weight(w.packed.clone(), None, w.gscale.clone(), w.N, w.K)

    def line(us_list, nbytes=None, flops=None, mfma=False):
        t = statistics.median(us_list)
        d = {"us": stats(us_list)}
        if nbytes is not None:
            d["weight_GBps"] = round(nbytes / t / 1e3, 1)
            d["pct_of_hbm_peak"] = round(100 * nbytes / t / 1e3 / HBM_PEAK_GBPS, 2)
        if flops is not None:
            d["TFLOPs"] = round(flops / t / 1e6, 1)
            if mfma:
                d["frac_of_mfma_bf16_peak"] = round(flops / t / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)
        return d

    # ---- config 0: one 1024 x 1024 GEMV, M = 1 (launch latency)
    w0 = workload("gemv_1024")
    b0 = fp4.quantize(gpu_bf16(tensor_bits(w0.tensor("w"))), "tiled")
    cps = [b0] + [clone(b0) for _ in range(899)]
    x0 = gpu_bf16(x_bits(w0.x("x")))
    y0 = torch.empty((1, 1024), dtype=torch.float32, device=dev)
    res["c0_gemv_1024x1024_m1"] = line(timer.time_calls(lambda i: fp4.gemv(x0, cps[i % 900], out=y0), 900),
                                       weight_bytes(1024, 1024))
    del cps
    # ---- config 1: Qwen3-0.6B-shaped decode, 28 layers x (QKV fused, O, gate_up fused, down), M = 1
    wq = workload("qwen3_0p6b_decode")
    layers = []
    for l in range(1, 29):
        ws = {t: fp4.quantize(gpu_bf16(tensor_bits(wq.tensor("L%d.%s" % (l, t)))), "tiled")
              for t in ("q", "k", "v", "o", "gate", "up", "down")}
        xs = {k: gpu_bf16(x_bits(wq.x("L%d.x%d" % (l, k)))) for k in (1024, 2048, 3072)}
        layers.append((ws, xs))
    sets = [layers] + [[({t: clone(w) for t, w in ws.items()}, xs) for ws, xs in layers] for _ in range(2)]
    qkv = torch.empty((1, 4096), dtype=torch.float32, device=dev)
    o = torch.empty((1, 1024), dtype=torch.float32, device=dev)
    gu1 = torch.empty((1, 6144), dtype=torch.float32, device=dev)
    d1 = torch.empty((1, 1024), dtype=torch.float32, device=dev)

    def token(i):
        for ws, xs in sets[i % len(sets)]:
            fp4.gemv_multi(xs[1024], [ws["q"], ws["k"], ws["v"]], [qkv, qkv[:, 2048:], qkv[:, 3072:]], [4096] * 3)
            fp4.gemv(xs[2048], ws["o"], out=o)
            fp4.gemv_multi(xs[1024], [ws["gate"], ws["up"]], [gu1, gu1[:, 3072:]], [6144] * 2)
            fp4.gemv(xs[3072], ws["down"], out=d1)
    us = [u / 28 for u in timer.time_calls(token, 6)]
    res["c1_qwen3_0p6b_decode_28_layers"] = dict(line(us, 8847360), unit="per layer", launches_per_layer=4)
    # the same step with the next projection's weights streamed into the caches during each product: a
    # forked branch of the graph (a second stream of the same priority, joined at the end) runs the
    # streaming-read probe on the next call's weight tiles while the current call computes; the products
    # keep their order on the main stream
    lib = fp4.raw()
    lib.fp4_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    side = torch.cuda.Stream()
    psink = torch.zeros(1 << 12, dtype=torch.int32, device=dev)

    def calls(layer_set):
        out = []
        for ws, xs in layer_set:
            out.append(((lambda ws=ws, xs=xs: fp4.gemv_multi(xs[1024], [ws["q"], ws["k"], ws["v"]],
                                                               [qkv, qkv[:, 2048:], qkv[:, 3072:]], [4096] * 3)),
                        [ws["q"], ws["k"], ws["v"]]))
            out.append(((lambda ws=ws, xs=xs: fp4.gemv(xs[2048], ws["o"], out=o)), [ws["o"]]))
            out.append(((lambda ws=ws, xs=xs: fp4.gemv_multi(xs[1024], [ws["gate"], ws["up"]], [gu1, gu1[:, 3072:]],
                                                               [6144] * 2)), [ws["gate"], ws["up"]]))
            out.append(((lambda ws=ws, xs=xs: fp4.gemv(xs[3072], ws["down"], out=d1)), [ws["down"]]))
        return out
    seqs = [calls(ls) for ls in sets]

    def token_prefetch(i):
        seq = seqs[i % len(seqs)]
        main = torch.cuda.current_stream()
        for k, (call, _) in enumerate(seq):
            if k + 1 < len(seq):
                ev = torch.cuda.Event()
                ev.record(main)
                side.wait_event(ev)
                for w in seq[k + 1][1]:
                    nb = w.packed.numel() // 1024 * 1024
                    rc = lib.fp4_bench_stream_read(w.packed.data_ptr(), nb, 64, 4, 1, 0, 0, psink.data_ptr(),
                                                   side.cuda_stream)
                    if rc != 0:
                        raise RuntimeError("fp4_bench_stream_read: %d" % rc)
            call()
        done = torch.cuda.Event()
        done.record(side)
        main.wait_event(done)
    us = [u / 28 for u in timer.time_calls(token_prefetch, 6)]
    res["c1_qwen3_0p6b_decode_28_layers_next_weights_prefetched"] = dict(line(us, 8847360), unit="per layer",
                                                                        launches_per_layer=4)
    del seqs
    # the same layers with their neighbours fused: RMS norm (eps 1e-6) inside the QKV launch, SwiGLU inside
    # the gate_up launch writing bf16 h, and the down projection reading that h
    from workloads import norm_gain
    gain = gpu_bf16(norm_gain(1024, 55))
    h1 = torch.empty((1, 3072), dtype=torch.bfloat16, device=dev)

    def token_fused(i):
        for ws, xs in sets[i % len(sets)]:
            fp4.gemv_multi_rmsnorm(xs[1024], gain, 1e-6, [ws["q"], ws["k"], ws["v"]],
                                   [qkv, qkv[:, 2048:], qkv[:, 3072:]], [4096] * 3)
            fp4.gemv(xs[2048], ws["o"], out=o)
            fp4.gemv_swiglu(xs[1024], ws["gate"], ws["up"], out=h1)
            fp4.gemv(h1, ws["down"], out=d1)
    us = [u / 28 for u in timer.time_calls(token_fused, 6)]
    res["c1_qwen3_0p6b_decode_28_layers_norm_swiglu_fused"] = dict(line(us, 8847360), unit="per layer",
                                                                   launches_per_layer=4)
    del sets, layers
    # ---- config 2 at M = 1 is the headline; config 3: the same layer with M in {2, 4, 8, 16}
    wcp = [w27] + [{k: clone(w) for k, w in w27.items()} for _ in range(5)]
    sm = workload("dense27b_smallm")
    B27 = weight_bytes(2 * INTER, HIDDEN) + weight_bytes(HIDDEN, INTER)
    for M in (2, 4, 8, 16):
        xi = gpu_bf16(x_bits(sm.x("x_in_m%d" % M)))
        xm = gpu_bf16(x_bits(sm.x("x_mid_m%d" % M)))
        gu = torch.empty((M, 2 * INTER), dtype=torch.float32, device=dev)
        yd = torch.empty((M, HIDDEN), dtype=torch.float32, device=dev)
        work = fp4.new_workspace(max(fp4.workspace_bytes(fp4.OP_GEMV, M, HIDDEN, [INTER, INTER]),
                                     fp4.workspace_bytes(fp4.OP_GEMV, M, INTER, [HIDDEN])), dev)

        def layer(i, xi=xi, xm=xm, gu=gu, yd=yd, work=work):
            w = wcp[i % len(wcp)]
            fp4.gemv_multi(xi, [w["gate"], w["up"]], [gu, gu[:, INTER:]], [2 * INTER, 2 * INTER], workspace=work)
            fp4.gemv(xm, w["down"], out=yd, workspace=work)
        flops = 2.0 * M * (2 * INTER * HIDDEN + HIDDEN * INTER)
        res["c3_dense27b_layer_m%d" % M] = dict(line(timer.time_calls(layer, 24), B27, flops), unit="per layer")
    # ---- config 2 as a real MLP: SwiGLU(gate, up) -> bf16 h -> down(h), M = 1
    hh = torch.empty((1, INTER), dtype=torch.bfloat16, device=dev)
    yd1 = torch.empty((1, HIDDEN), dtype=torch.float32, device=dev)

    def mlp(i):
        w = wcp[i % len(wcp)]
        fp4.gemv_swiglu(x_in0, w["gate"], w["up"], out=hh)
        fp4.gemv(hh, w["down"], out=yd1)
    res["c2_dense27b_mlp_swiglu_then_down_m1"] = dict(line(timer.time_calls(mlp, 24), B27), unit="per layer")
    # ---- config 4a: LM head 151936 x 1024 at M = 1 and 8, product alone and with the greedy choice
    lm = workload("lm_head")
    bl = fp4.quantize(gpu_bf16(tensor_bits(lm.tensor("w"))), "tiled")
    lcp = [bl] + [clone(bl) for _ in range(6)]
    BL = weight_bytes(151936, 1024)
    for M in (1, 8):
        x = gpu_bf16(x_bits(lm.x("x_m%d" % M)))
        y = torch.empty((M, 151936), dtype=torch.float32, device=dev)
        idx = torch.empty((M,), dtype=torch.int32, device=dev)
        work = fp4.new_workspace(fp4.workspace_bytes(fp4.OP_LM_HEAD_GREEDY, M, 1024, [151936]), dev)
        t1 = timer.time_calls(lambda i, x=x, y=y: fp4.gemv(x, lcp[i % 7], out=y), 56)
        t2 = timer.time_calls(lambda i, x=x, y=y, idx=idx, work=work:
                              fp4.lm_head_greedy(x, lcp[i % 7], logits=y, out=idx, workspace=work), 56)
        res["c4_lm_head_m%d" % M] = line(t1, BL, 2.0 * M * 151936 * 1024)
        res["c4_lm_head_greedy_m%d" % M] = dict(line(t2, BL),
                                                greedy_added_us=round(statistics.median(t2) - statistics.median(t1), 3))
    del lcp, bl
    # ---- config 4b: prefill 2048 tokens x gate_up 5120 -> 34816, gate and up in one launch
    xp = gpu_bf16(x_bits(workload("prefill").x("x")))
    yf = torch.empty((2048, 2 * INTER), dtype=torch.float32, device=dev)
    work = fp4.new_workspace(fp4.workspace_bytes(fp4.OP_GEMM_PREFILL, 2048, HIDDEN, [INTER, INTER]), dev)

    def pf(i):
        w = wcp[i % len(wcp)]
        fp4.gemm_prefill_multi(xp, [w["gate"], w["up"]], [yf[:, :INTER], yf[:, INTER:]], [2 * INTER, 2 * INTER],
                               workspace=work)
    res["c4_prefill_2048x34816x5120"] = line(timer.time_calls(pf, 6, reps=5), flops=2.0 * 2048 * 2 * INTER * HIDDEN,
                                             mfma=True)
    del yf, wcp
    # ---- MXFP4 (E8M0 scale per 32 elements): the 27B-class layer at M = 1 (gate, up, down), the LM head at
    # M = 1 and the prefill product of the gate projection
    wl2 = workload("dense27b_layer")
    # gate and up stacked into one 34816 x 5120 weight (the rows are quantised independently, so stacking
    # before or after quantisation gives the same bytes) and read by one launch
    mxb = {n: fp4.quantize_mx(gpu_bf16(tensor_bits(wl2.tensor(n))), "mx_tiled") for n in ("gate", "down")}
    mxb["gate_up"] = fp4.quantize_mx(torch.cat([gpu_bf16(tensor_bits(wl2.tensor(n))) for n in ("gate", "up")]),
                                     "mx_tiled")
    mxc = [mxb] + [{k: fp4.MXFP4Weight(w.packed.clone(), None, w.N, w.K) for k, w in mxb.items()} for _ in range(5)]
    g2 = torch.empty((1, 2 * INTER), dtype=torch.float32, device=dev)

    def mx_layer(i):
        w = mxc[i % len(mxc)]
        fp4.gemv_mx(x_in0, w["gate_up"], out=g2)
        fp4.gemv_mx(x_mid0, w["down"], out=yd1)
    Bmx = lambda N, K: N * K // 2 + N * K // 32   # noqa: E731
    Bmx27 = 2 * Bmx(INTER, HIDDEN) + Bmx(HIDDEN, INTER)
    res["mx_dense27b_layer_m1"] = dict(line(timer.time_calls(mx_layer, 24), Bmx27), unit="per layer", launches=2)
    res["mx_down_5120x17408_m1"] = line(timer.time_calls(lambda i: fp4.gemv_mx(x_mid0, mxc[i % 6]["down"], out=yd1), 48),
                                        Bmx(HIDDEN, INTER))
    lmx = fp4.quantize_mx(gpu_bf16(tensor_bits(workload("lm_head").tensor("w"))), "mx_tiled")
    lmxc = [lmx] + [fp4.MXFP4Weight(lmx.packed.clone(), None, lmx.N, lmx.K) for _ in range(6)]
    xl = gpu_bf16(x_bits(workload("lm_head").x("x_m1")))
    yl = torch.empty((1, 151936), dtype=torch.float32, device=dev)
    res["mx_lm_head_m1"] = line(timer.time_calls(lambda i: fp4.gemv_mx(xl, lmxc[i % 7], out=yl), 56),
                                Bmx(151936, 1024))
    ypm = torch.empty((2048, INTER), dtype=torch.float32, device=dev)
    res["mx_prefill_2048x17408x5120"] = line(timer.time_calls(lambda i: fp4.gemm_prefill_mx(xp, mxc[i % 6]["gate"],
                                                                                          out=ypm), 6, reps=5),
                                             flops=2.0 * 2048 * INTER * HIDDEN, mfma=True)
    # the same product with both operands MXFP4 on the block-scaled FP4 matrix cores; the activations are
    # quantised (fp4_quantize_mx, the activation operand layout) in a launch of their own, timed apart
    xq4 = fp4.quantize_mx(xp, "mx_act")
    fl4 = 2.0 * 2048 * INTER * HIDDEN
    t4 = timer.time_calls(lambda i: fp4.gemm_mx_a4(xq4, mxc[i % 6]["gate"], out=ypm), 6, reps=5)
    res["mx_a4_prefill_2048x17408x5120"] = dict(
        line(t4, flops=fl4), frac_of_mfma_fp4_peak=round(fl4 / statistics.median(t4) / 1e6 / MFMA_FP4_PEAK_TFLOPS, 4))
    res["mx_a4_quantise_x_2048x5120"] = line(timer.time_calls(lambda i: fp4.quantize_mx(xp, "mx_act", out=xq4), 6,
                                                              reps=5))
    del mxb, mxc, lmx, lmxc, ypm, xp, g2, xq4
    # ---- load-time quantisation of the down projection from bf16 and from an FP8 release (the
    # rule reads the input twice: algorithmic bytes = 2 input reads + 9/16 byte per element written)
    Wb = gpu_bf16(tensor_bits(workload("dense27b_layer").tensor("down")))
    codes, sc = fp8_release((HIDDEN, INTER), 32, 0.015, outlier_p=0.001, outlier_scale=20)
    Wf = torch.from_numpy(codes).to(dev)
    Sf = torch.tensor([float(sc)], dtype=torch.float32, device=dev)
    for name, ebytes, q in (("bf16", 2, lambda o: fp4.quantize(Wb, "tiled", out=o)),
                            ("fp8", 1, lambda o: fp4.quantize_fp8(Wf, Sf, "tiled", out=o))):
        o = q(None)
        alg = 2 * ebytes * HIDDEN * INTER + weight_bytes(HIDDEN, INTER)
        t = timer.time_calls(lambda i, q=q, o=o: q(o), 4, reps=5)
        d = line(t)
        d["algorithmic_GBps"] = round(alg / statistics.median(t) / 1e3, 1)
        d["pct_of_hbm_peak"] = round(100 * alg / statistics.median(t) / 1e3 / HBM_PEAK_GBPS, 2)
        res["quantise_5120x17408_from_%s" % name] = d
    return res


if __name__ == "__main__":
    main()
