#!/usr/bin/env python3
"""Benchmark of the fused 4-bit weight-only GEMM on one MI355X.

Workload (one "step" = one pass of the whole decode hot path over one batch):
Llama-2-7B-shaped decode layers in GPTQ layout with act-order -- (K, N) in
{(4096, 4096), (4096, 11008), (11008, 4096)} at M in {1, 4, 16} tokens, group
size 128, fp16 activations ~ N(0, 1), W ~ N(0, 0.02) RTN-quantized on the
device.  Each (shape, M) pair is its own layer with its own weights, and R
rotating copies of the weight set (>= 512 MB in total, twice the 256 MB
Infinity Cache) make every step stream its weights from HBM.  Inputs are
resident in HBM before timing starts.

Printed: ONE JSON line with the weight-stream GB/s of the step (value), the
effective TFLOP/s, the roofline of the dominant kernel (HIP-event durations of
every GEMM launch in the timed region), and the CPU oracle timed on a bounded
sample on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 MFMA
SHAPES = [(4096, 4096), (4096, 11008), (11008, 4096)]   # (K, N)
MS = [1, 4, 16]
G = 128


def weight_bytes(K, N, perm=True):
    return K * N // 2 + 2 * N * K // G + N * K // (2 * G) + (4 * K if perm else 0)


def call_bytes(M, K, N):
    """Algorithmic bytes of the GEMM kernel itself: codes + scales + zeros, the
    (permuted) activations and the output.  The permutation vector is read by
    the separate act-order gather kernel."""
    return weight_bytes(K, N, perm=False) + 2 * M * K + 2 * M * N


def kernel_name(M, K, N):
    """Kernel instantiation the library picks for an act-order call with M
    rows (f16).  Mirrors its rules: the large-M kernel from 32 rows (5 on
    layers of 100 Mi weights; 17 on layers of 24 Mi weights with N < 5120);
    otherwise the
    decode kernel, where M <= 4 rows are gathered in the kernel when the
    staged rows + permutation take at most 72 KB per workgroup and 17 MiB over
    the N/16 workgroups, else a preparation pass permutes them first; one row
    (M = 1) has an instantiation of its own (the one-row form of the fold);
    more rows take the full-row modes."""
    kb = lambda b: (b + 1023) // 1024 * 1024
    w = N * K
    if (M >= 32 or (w >= 100 << 20 and M >= 5)
            or (w >= 24 << 20 and N < 5120 and M >= 17)):
        return "wq_prefill_kernel<f16, INT 4-bit>"      # the large-M kernel
    if M <= 4:
        staged = kb(M * K * 2) + kb(K * 4)
        mode = ("xgather" if staged <= 72 * 1024 and ((N + 15) // 16) * staged <= 17 << 20
                else "packed")
        return "intb_decode_kernel<f16, MT=1, %s, 4-bit%s>" % (mode, ", one row" if M == 1 else "")
    mt = 1 if M <= 16 else (2 if M <= 32 else 4)
    # full rows: direct loads for at most 8 rows on at most 4096 columns, else
    # whole-line loads and a transpose through LDS
    return "intb_decode_kernel<f16, MT=%d, %s, 4-bit>" % (mt, "full" if M <= 8 and N <= 4096
                                                          else "full-t")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-nf4", action="store_true")
    ap.add_argument("--no-qwen", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run each decode call of the workload once, then a 256 MiB device copy "
                         "(for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE), and exit")
    ap.add_argument("--min-rotation-mb", type=float, default=512.0)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_weight_only_gemm_amd as w4
    from bit_weight_only_gemm_amd import synth, _lib

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = _lib.load()
    if args.pmc_probe:
        pmc_probe(L, dev)
        return
    stream = torch.cuda.Stream()          # graphs are captured on a non-default stream
    torch.cuda.set_stream(stream)
    sptr = ctypes.c_void_p(stream.cuda_stream)

    # ---- inputs: weights quantized + repacked on the device, x per M
    base = {}
    for K, N in SHAPES:
        W = torch.from_numpy(synth.weights("C2/W/%dx%d" % (K, N), N, K)).to(dev)
        gi = torch.from_numpy(synth.act_order_gidx("C2/gidx/%dx%d" % (K, N), K, G)).to(dev)
        qw, sc, qz = w4.w4a16_quantize_rtn(W, G, g_idx=gi)
        base[(K, N)] = w4.w4a16_repack(qw, sc, qz, gi)
        del W, qw, sc, qz
    set_bytes = sum(weight_bytes(K, N) for K, N in SHAPES) * len(MS)
    R = max(1, int(np.ceil(args.min_rotation_mb * 1e6 / set_bytes)))
    rot = []
    for r in range(R):
        step_layers = []
        for K, N in SHAPES:
            p = base[(K, N)]
            for M in MS:
                q = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
                step_layers.append((K, N, M, q))
        rot.append(step_layers)
    xs = {}
    outs = {}
    for K, N in SHAPES:
        for M in MS:
            xb = synth.to_f16_bits(synth.activations("C2/x/%dx%d" % (M, K), M, K))
            xs[(M, K)] = torch.from_numpy(xb.view(np.int16)).view(torch.float16).to(dev)
            outs[(M, N, K)] = torch.empty((M, N), dtype=torch.float16, device=dev)
    ws_need = max(w4.w4a16_workspace_bytes(M, N, K) for K, N in SHAPES for M in MS)
    ws = w4.workspace(ws_need, dev)
    ws_ptr = ctypes.c_void_p(ws.data_ptr() if ws is not None else 0)
    ws_len = ws.numel() * 4 if ws is not None else 0

    # pre-bound C calls (argument marshalling done once)
    calls = []
    for step_layers in rot:
        cl = []
        for K, N, M, q in step_layers:
            a = (ctypes.c_void_p(xs[(M, K)].data_ptr()), ctypes.c_void_p(q["codes"].data_ptr()),
                 ctypes.c_void_p(q["scales"].data_ptr()), ctypes.c_void_p(q["zeros"].data_ptr()),
                 ctypes.c_void_p(q["perm"].data_ptr()), G,
                 ctypes.c_void_p(outs[(M, N, K)].data_ptr()), M, N, K, w4.F16, ws_ptr, ws_len,
                 sptr)
            cl.append((a, call_bytes(M, K, N), 2 * M * N * K, weight_bytes(K, N)))
        calls.append(cl)
    torch.cuda.synchronize()

    def run_step(i):
        for a, _, _, _ in calls[i % R]:
            st = L.w4a16_gemm(*a)
            if st != 0:
                raise RuntimeError("w4a16_gemm status %d" % st)

    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()

    # ---- one HIP graph per weight-rotation set: a step is one graph replay
    # (the 9 GEMM calls with their act-order permutation kernels), so host
    # launch overhead is out of the measured step.
    graphs = []
    for r in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            run_step(r)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(max(args.warmup, R)):
        graphs[i % R].replay()
    torch.cuda.synchronize()

    # ---- timed region, part 1: K steps (graph replays), synchronized both sides
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps

    # ---- timed region, part 2: the same K steps launched eagerly with HIP
    # timing events attached to every GEMM kernel's own dispatch
    # (hipExtLaunchKernel start/stop), on the stream the kernels run on.  A
    # dispatch's start event is taken when it is queued, so a kernel queued
    # behind another one would be charged that kernel's tail: calls whose
    # kernel does not gather x itself get their activations already permuted
    # (perm = NULL; the same kernel instantiation on the same data without the
    # library's permutation pass in front of it), and the stream is drained
    # after every call, before the next one is queued.  (The step time above
    # includes the pass and runs the calls back to back.)
    hip = ctypes.CDLL("libamdhip64.so.7")
    nper = len(calls[0])
    tcalls = []
    for step_layers, cl in zip(rot, calls):
        tl = []
        for (K, N, M, q), (a, _, _, _) in zip(step_layers, cl):
            if ", xgather," in kernel_name(M, K, N):
                tl.append(a)
                continue
            key = ("xp", M, K, N)
            if key not in xs:
                xs[key] = xs[(M, K)][:, q["perm"].long()].contiguous()
            tl.append((ctypes.c_void_p(xs[key].data_ptr()),) + a[1:4] + (ctypes.c_void_p(0),)
                      + a[5:])
        tcalls.append(tl)
    torch.cuda.synchronize()
    nev = args.steps * nper
    ev = (ctypes.c_void_p * (2 * nev))()
    for k in range(2 * nev):
        if hip.hipEventCreate(ctypes.byref(ev, k * ctypes.sizeof(ctypes.c_void_p))) != 0:
            raise RuntimeError("hipEventCreate failed")
    torch.cuda.synchronize()
    for i in range(args.steps):
        for j, a in enumerate(tcalls[i % R]):
            k = i * nper + j
            L.w4a16_set_timing_events(ctypes.c_void_p(ev[2 * k]), ctypes.c_void_p(ev[2 * k + 1]))
            if L.w4a16_gemm(*a) != 0:
                raise RuntimeError("w4a16_gemm failed")
            if hip.hipStreamSynchronize(sptr) != 0:
                raise RuntimeError("hipStreamSynchronize failed")
    torch.cuda.synchronize()
    ms = ctypes.c_float(0.0)
    dur = np.zeros((args.steps, nper))
    for i in range(args.steps):
        for j in range(nper):
            k = i * nper + j
            if hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(ev[2 * k]),
                                       ctypes.c_void_p(ev[2 * k + 1])) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            dur[i, j] = ms.value * 1e-3
    for k in range(2 * nev):
        hip.hipEventDestroy(ctypes.c_void_p(ev[k]))

    step_wbytes = sum(c[3] for c in calls[0])
    step_flops = sum(c[2] for c in calls[0])
    step_bytes = sum(c[1] for c in calls[0])
    # the dominant kernel: the instantiation with the most time per step
    groups = {}
    for j, (K, N, M, _) in enumerate(rot[0]):
        groups.setdefault(kernel_name(M, K, N), []).append(j)
    dom = max(groups, key=lambda g: dur[:, groups[g]].sum())
    dj = groups[dom]
    avg_launch_s = float(dur[:, dj].mean())
    dom_bytes = float(np.mean([calls[0][j][1] for j in dj]))
    achieved = dom_bytes / avg_launch_s / 1e9
    per_point = []
    for j, (K, N, M, _) in enumerate(rot[0]):
        d = float(dur[:, j].mean())
        per_point.append({"M": M, "K": K, "N": N, "kernel": kernel_name(M, K, N),
                          "us": round(d * 1e6, 2),
                          "weight_GBps": round(weight_bytes(K, N) / d / 1e9, 1),
                          "pct_hbm": round(100 * call_bytes(M, K, N) / d / 1e9 / HBM_PEAK_GBS, 1)})

    props = torch.cuda.get_device_properties(dev)
    result = {
        "metric": "W4A16 GEMM TFLOP/s + weight GB/s (% of HBM/MFMA peak), M=1..16 and M=2048",
        "value": round(step_wbytes / step_s / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,0.02) weights RTN-quantized on device, N(0,1) activations)",
        "config": {
            "workload": "Llama-2-7B-shaped decode GEMMs, GPTQ act-order int4 G=128: "
                        "(K,N) in {(4096,4096),(4096,11008),(11008,4096)} x M in {1,4,16}",
            "gemm_calls_per_step": nper,
            "step_timing": "HIP graph replay per step (the GEMM kernels, plus the act-order "
                           "permutation pass where the kernel does not gather itself)",
            "weight_rotation_copies": R,
            "tflops": round(step_flops / step_s / 1e12, 3),
            "pct_hbm_step": round(100 * step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 1),
            "gpu": props.name,
            "cus": props.multi_processor_count,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "launches_per_step": len(dj),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(dom),
            "avg_launch_us": round(avg_launch_s * 1e6, 3),
            "timing": "hipExtLaunchKernel start/stop events on every launch of this kernel "
                      "in K eager steps, on the stream it runs on, the stream drained "
                      "between calls",
            "algorithmic_bytes_per_launch": round(dom_bytes),
        },
        "points": per_point,
    }
    timer = KernelTimer(L, hip)
    del rot, calls, graphs, base
    torch.cuda.empty_cache()
    if not args.no_prefill:
        result["prefill"] = bench_prefill(L, timer, sptr)
        result["prefill_m8192"] = bench_prefill(L, timer, sptr, M=8192)
    if not args.no_qwen:
        result["qwen_decode"] = bench_qwen_decode()
    if not args.no_nf4:
        result["nf4"] = bench_nf4(L, timer, sptr)
    if not args.no_variants:
        result["variants"] = bench_variants()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(xs, outs)
    print(json.dumps(result), flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "int4_decode_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "bit_weight_only_gemm_amd", "csrc", f)
                  for f in ("gemm.hip", "decode.h", "common.h", "prefill.h", "prefill.hip")]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size), or None
    when there is none or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("kernels", {}).get(kernel, {}).get("hbm_bytes_per_launch")


def pmc_probe(L, dev):
    """Each GEMM call of the workload once (act-order, one weight copy),
    then a 256 MiB device-to-device copy whose byte count calibrates the
    counters."""
    import torch
    import bit_weight_only_gemm_amd as w4
    from bit_weight_only_gemm_amd import synth
    for K, N in SHAPES:
        W = torch.from_numpy(synth.weights("C2/W/%dx%d" % (K, N), N, K)).to(dev)
        gi = torch.from_numpy(synth.act_order_gidx("C2/gidx/%dx%d" % (K, N), K, G)).to(dev)
        qw, sc, qz = w4.w4a16_quantize_rtn(W, G, g_idx=gi)
        p = w4.w4a16_repack(qw, sc, qz, gi)
        del W, qw, sc, qz
        for M in MS:
            xb = synth.to_f16_bits(synth.activations("C2/x/%dx%d" % (M, K), M, K))
            x = torch.from_numpy(xb.view(np.int16)).view(torch.float16).to(dev)
            w4.w4a16_gemm(x, p)
            torch.cuda.synchronize()
            print("call M=%d K=%d N=%d kernel=%s algorithmic_bytes=%d"
                  % (M, K, N, kernel_name(M, K, N), call_bytes(M, K, N)), flush=True)
    src = torch.ones(64 * 2**20, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print("copy bytes_read=%d bytes_written=%d" % (src.numel() * 4, dst.numel() * 4), flush=True)


class KernelTimer:
    """Durations of the library's main kernel launch, from hipExtLaunchKernel
    start/stop events (w4a16_set_timing_events) on the stream it runs on."""

    def __init__(self, L, hip):
        self.L, self.hip = L, hip
        self.ev = (ctypes.c_void_p * 2)()
        for k in range(2):
            if hip.hipEventCreate(ctypes.byref(self.ev, k * ctypes.sizeof(ctypes.c_void_p))):
                raise RuntimeError("hipEventCreate failed")

    def time(self, call, reps, warm=3):
        import torch
        ts = []
        ms = ctypes.c_float(0.0)
        for r in range(warm + reps):
            self.L.w4a16_set_timing_events(ctypes.c_void_p(self.ev[0]), ctypes.c_void_p(self.ev[1]))
            if call() != 0:
                raise RuntimeError("library call failed")
            torch.cuda.synchronize()
            self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.ev[0]),
                                         ctypes.c_void_p(self.ev[1]))
            if r >= warm:
                ts.append(ms.value * 1e-3)
        return float(np.median(ts))


PREFILL_SHAPES = [(5120, 7168), (5120, 5120), (5120, 55296), (27648, 5120)]   # (K, N)


def bench_prefill(L, timer, sptr, M=2048):
    """Qwen2.5-32B-shaped prefill layers at M tokens, bf16 activations
    ~N(0,1) with 1 % of the input channels x20, RTN int4 G=128 weights:
    median kernel time of the fused kernel, and dense bf16 torch.matmul of
    the dequantized weights (the practical matrix-core ceiling) beside it."""
    import torch
    import bit_weight_only_gemm_amd as w4
    from bit_weight_only_gemm_amd import synth
    dev = torch.device("cuda:0")
    pts = []
    for K, N in PREFILL_SHAPES:
        W = torch.from_numpy(synth.weights("C4/W/%dx%d" % (K, N), N, K)).to(dev)
        qw, sc, qz = w4.w4a16_quantize_rtn(W, G)
        p = w4.w4a16_repack(qw, sc, qz, None)
        del W, qw, sc, qz
        x32 = synth.activations("C4/x/%dx%d" % (M, K), M, K)
        x32 = synth.with_outliers(x32, synth.outlier_channels("C4/outl/%d" % K, K))
        x = torch.from_numpy(synth.to_bf16_bits(x32).view(np.int16)).view(torch.bfloat16).to(dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        wsb = w4.w4a16_workspace_bytes(M, N, K)
        ws = w4.workspace(wsb, dev)
        a = (ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(p["codes"].data_ptr()),
             ctypes.c_void_p(p["scales"].data_ptr()), ctypes.c_void_p(p["zeros"].data_ptr()),
             None, G, ctypes.c_void_p(y.data_ptr()), M, N, K, w4.BF16,
             ctypes.c_void_p(ws.data_ptr() if ws is not None else 0), wsb, sptr)
        for _ in range(20):          # clocks up before the first timed shape
            L.w4a16_gemm(*a)
        t = timer.time(lambda: L.w4a16_gemm(*a), 10)
        wd = w4.w4a16_dequant(p, torch.bfloat16)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            torch.matmul(x, wd.t())
        e0.record()
        for _ in range(10):
            torch.matmul(x, wd.t())
        e1.record()
        torch.cuda.synchronize()
        td = e0.elapsed_time(e1) * 1e-3 / 10
        fl = 2.0 * M * N * K
        pts.append({"M": M, "K": K, "N": N, "us": round(t * 1e6, 1),
                    "tflops": round(fl / t / 1e12, 1),
                    "pct_mfma": round(100 * fl / t / 1e12 / MFMA_F16_PEAK_TFLOPS, 1),
                    "dense_bf16_matmul_tflops": round(fl / td / 1e12, 1)})
        del p, x, y, wd, ws
        torch.cuda.empty_cache()
    best = max(pts, key=lambda q: q["tflops"])
    tot_fl = sum(2.0 * q["M"] * q["N"] * q["K"] for q in pts)
    tot_t = sum(q["us"] for q in pts) * 1e-6
    return {"workload": "Qwen2.5-32B-shaped prefill, int4 G=128, bf16 x with 1% outlier "
                        "channels x20, M=" + str(M),
            "kernel": "wq_prefill_kernel<bf16, INT 4-bit>",
            "tflops_all_shapes": round(tot_fl / tot_t / 1e12, 1),
            "roofline": {"bound": "mfma", "achieved": best["tflops"],
                         "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(best["tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
                         "shape": [best["M"], best["K"], best["N"]]},
            "points": pts}


def graph_call_time(call, ps, stream, n=10, reps=5):
    """Seconds per call of `call(p)` over the weight copies ps, from HIP-graph
    replays of n calls (the whole call: any preparation pass and reduction)."""
    import torch
    for r in range(3):
        call(ps[r % len(ps)])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for r in range(n):
            call(ps[r % len(ps)])
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e-3 / (reps * n)


def bench_qwen_decode(Ms=(1, 16, 64)):
    """The Qwen2.5-32B-shaped layers in AWQ layout (s ~ U[0.5, 2] folded into W,
    x divided by s before the call), int4 G=128, fp16 activations, at M in
    {1, 16, 64}: whole calls by HIP-graph replay over rotating weight copies
    (>= 512 MB), weight-stream GB/s per layer and over the four layers."""
    import torch
    import bit_weight_only_gemm_amd as w4
    from bit_weight_only_gemm_amd import synth
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    pts = []
    tot = {M: [0.0, 0] for M in Ms}
    for K, N in PREFILL_SHAPES:
        W = torch.from_numpy(synth.weights("C3/W/%dx%d" % (K, N), N, K)).to(dev)
        s = torch.from_numpy(synth.awq_scales("C3/s/%d" % K, K)).to(dev)
        qw, sc, qz = w4.w4a16_quantize_rtn(W * s[None, :], G)
        p0 = w4.w4a16_repack(qw, sc, qz)
        del W, qw, sc, qz
        wb = weight_bytes(K, N, perm=False)
        R = max(2, int(np.ceil(512e6 / wb)))
        ps = [p0] + [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in p0.items()}
                     for _ in range(R - 1)]
        for M in Ms:
            x = (torch.from_numpy(synth.activations("C3/x/%dx%d" % (M, K), M, K)).to(dev)
                 / s[None, :]).half()
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            ws = w4.workspace(w4.w4a16_workspace_bytes(M, N, K), dev)
            t = graph_call_time(lambda p: w4.w4a16_gemm(x, p, out=y, workspace=ws), ps, stream)
            byt = wb + 2 * M * K + 2 * M * N
            pts.append({"M": M, "K": K, "N": N, "us": round(t * 1e6, 2),
                        "weight_GBps": round(wb / t / 1e9, 1),
                        "pct_hbm": round(100 * byt / t / 1e9 / HBM_PEAK_GBS, 1)})
            tot[M][0] += t
            tot[M][1] += wb
            del x, y, ws
        del ps, p0, s
        torch.cuda.empty_cache()
    return {"workload": "Qwen2.5-32B-shaped layers (5120x7168, 5120x5120, 5120x55296, "
                        "27648x5120), AWQ layout, int4 G=128, fp16, whole calls",
            "weight_GBps_all_layers": {str(M): round(tot[M][1] / tot[M][0] / 1e9, 1) for M in Ms},
            "points": pts}


VARIANTS = [  # (label, bits, group size (-1: per-channel), symmetric, AWQ input scales)
    ("int4 G=128 asym", 4, 128, False, False),
    ("int4 G=64 sym", 4, 64, True, False),
    ("int4 G=32 asym", 4, 32, False, False),
    ("int4 per-channel sym", 4, -1, True, False),
    ("int4 G=128 asym + AWQ input scales", 4, 128, False, True),
    ("int3 G=128 asym", 3, 128, False, False),
    ("int8 G=128 asym", 8, 128, False, False),
]


def variant_weight_bytes(K, N, bits, G, sym):
    """Algorithmic bytes of a weight: codes + fp16 scales + zero fields per
    group (per 128-input tile for G >= 128: the repacked meta repeats per tile)."""
    g = min(K if G == -1 else G, 128)
    zbits = 8 if bits == 8 else 4
    return K * N * bits // 8 + 2 * N * K // g + (0 if sym else N * K // g * zbits // 8)


def bench_variants(K=5120, N=55296, Ms=(1, 2048)):
    """The format variants on the 5120 x 55296 layer (bf16 activations): group
    sizes, symmetric codes, 3- and 8-bit codes and AWQ input scales.  Whole
    calls (any preparation pass included) timed by HIP-graph replay of 10
    calls over rotating weight copies (>= 512 MB)."""
    import torch
    import bit_weight_only_gemm_amd as w4
    from bit_weight_only_gemm_amd import synth
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    W = torch.from_numpy(synth.weights("C6/W/%dx%d" % (K, N), N, K)).to(dev)
    s_awq = torch.from_numpy(synth.to_bf16_bits(synth.awq_scales("C6/s/%d" % K, K)[None, :])[0]
                             .view(np.int16)).view(torch.bfloat16).to(dev)
    pts = []
    for label, bits, G, sym, xs in VARIANTS:
        qw, sc, qz = w4.w4a16_quantize_rtn(W, G, sym=sym, bits=bits)
        p0 = w4.w4a16_repack(qw, sc, qz, None, G, bits=bits)
        del qw, sc, qz
        wb = variant_weight_bytes(K, N, bits, G, sym)
        R = max(2, int(np.ceil(512e6 / wb)))
        ps = [p0] + [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in p0.items()}
                     for _ in range(R - 1)]
        for M in Ms:
            x32 = synth.activations("C6/x/%d" % M, M, K)
            x = torch.from_numpy(synth.to_bf16_bits(x32).view(np.int16)).view(torch.bfloat16).to(dev)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ws = w4.workspace(w4.w4a16_workspace_bytes(M, N, K, G), dev)

            def call(p):
                if xs:
                    w4.w4a16_gemm_xscale(x, s_awq, p, out=y, workspace=ws)
                else:
                    w4.w4a16_gemm(x, p, out=y, workspace=ws)
            for r in range(3):
                call(ps[r % R])
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for r in range(10):
                    call(ps[r % R])
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / 50
            pt = {"variant": label, "bits": bits, "group_size": G, "symmetric": sym,
                  "awq_input_scales": xs, "M": M, "us": round(t * 1e6, 2)}
            if M >= 1024:
                fl = 2.0 * M * N * K
                pt.update(tflops=round(fl / t / 1e12, 1),
                          pct_mfma=round(100 * fl / t / 1e12 / MFMA_F16_PEAK_TFLOPS, 1))
            else:
                byt = wb + 2 * M * K + 2 * M * N
                pt.update(weight_bytes=wb, GBps=round(byt / t / 1e9, 1),
                          pct_hbm=round(100 * byt / t / 1e9 / HBM_PEAK_GBS, 1))
            pts.append(pt)
            del x, y, ws, g
        del ps, p0
        torch.cuda.empty_cache()
    return {"workload": "5120 x 55296 layer, bf16 activations ~N(0,1), RTN weights of each "
                        "format; whole calls by HIP-graph replay",
            "points": pts}


def bench_nf4(L, timer, sptr, K=8192, N=28672):
    """The NF4 projection: W [28672, 8192] ~N(0, 0.02), blocksize 64, double
    quant over 256 blocks, bf16 x ~N(0,1) at M in {1, 32}; 4 rotating weight
    copies so the weights stream from HBM."""
    import torch
    import bit_weight_only_gemm_amd as w4
    from bit_weight_only_gemm_amd import synth
    dev = torch.device("cuda:0")
    W = torch.from_numpy(synth.weights("C5/W/%dx%d" % (K, N), N, K)).to(dev)
    p0 = w4.nf4_quantize(W)
    del W
    ps = [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in p0.items()}
          for _ in range(4)]
    wb = K * N // 2 + N * K // 64 + 4 * ((N * K // 64 + 255) // 256)
    pts = []
    for M in (1, 32):
        xb = synth.to_bf16_bits(synth.activations("C5/x/%d" % M, M, K))
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        wsb = w4.nf4_workspace_bytes(M, N, K)
        ws = w4.workspace(wsb, dev)
        wsp = ctypes.c_void_p(ws.data_ptr() if ws is not None else 0)
        k = [0]

        def call():
            p = ps[k[0] % 4]
            k[0] += 1
            return L.nf4_gemm(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(p["qweight"].data_ptr()),
                              ctypes.c_void_p(p["absmax_q"].data_ptr()),
                              ctypes.c_void_p(p["absmax_scale"].data_ptr()), 64,
                              ctypes.c_void_p(y.data_ptr()), M, N, K, w4.BF16, wsp, wsb, sptr)
        t = timer.time(call, 20)
        byt = wb + 2 * M * K + 2 * M * N
        pts.append({"M": M, "K": K, "N": N, "us": round(t * 1e6, 2),
                    "weight_GBps": round(wb / t / 1e9, 1),
                    "pct_hbm": round(100 * byt / t / 1e9 / HBM_PEAK_GBS, 1)})
    return {"workload": "NF4 28672x8192, blocksize 64, double quant 256, bf16",
            "kernel": "nf4_decode_kernel<bf16> (M=1), wq_prefill_kernel<bf16, NF4> (M=32)",
            "points": pts}


def cpu_baseline(xs, outs):
    """The oracle, as it stands, on whole steps (all 9 calls) of the same
    workload: unpack + dequant + fp64 product per call, on this host."""
    import torch
    from bit_weight_only_gemm_amd import synth
    from oracle import int4, gemm, fp
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    packed = {}
    for K, N in SHAPES:           # oracle inputs from the oracle's own quantizer (untimed)
        W = synth.weights("C2/W/%dx%d" % (K, N), N, K)
        gi = synth.act_order_gidx("C2/gidx/%dx%d" % (K, N), K, G)
        q, s, z = int4.quantize_rtn_int4(W, G, gi)
        packed[(K, N)] = (int4.pack_qweight(q), s, int4.pack_qzeros(z), gi)
    calls = [(K, N, M) for K, N in SHAPES for M in MS]
    wbytes = sum(weight_bytes(K, N) for K, N, _ in calls)

    def step(check):
        worst, t_total = 0.0, 0.0
        for K, N, M in calls:
            qw, s, qz, gi = packed[(K, N)]
            xb = xs[(M, K)].view(torch.int16).cpu().numpy().view(np.uint16)
            t0 = time.perf_counter()
            wd = int4.dequant_int4(qw, s, qz, gi, G, "f16")
            y_ref = gemm.gemm_ref_bits(xb, wd, "f16")
            t_total += time.perf_counter() - t0
            if check:
                y = fp.bits_to_f64(outs[(M, N, K)].view(torch.int16).cpu().numpy()
                                   .view(np.uint16), "f16")
                worst = max(worst, gemm.rel_err(y, y_ref))
        return t_total, worst

    # whole steps until at least 10 s of oracle time (at most 3)
    t_total, worst = step(True)
    nsteps = 1
    while t_total < 10.0 and nsteps < 3:
        t_total += step(False)[0]
        nsteps += 1
    single = None
    try:                          # the same step with the BLAS pool held to one thread
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1, _ = step(False)
        single = {"value": round(wbytes / t1 / 1e9, 4), "cores": 1, "seconds": round(t1, 2)}
    except Exception:
        pass
    return {"value": round(nsteps * wbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": blas_threads,
            "kind": "oracle",
            "sample": "%d whole step(s) (9 calls each: 3 shapes x M in {1,4,16}), at least 10 s "
                      "of oracle time; numpy dequant is single-threaded, the fp64 matmul uses "
                      "the BLAS threads counted in cores; single_core: one step" % nsteps,
            "seconds": round(t_total, 2),
            "single_core": single,
            "host_cpus": os.cpu_count(),
            "max_rel_err_gpu_vs_oracle": worst}


if __name__ == "__main__":
    main()
