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
every GEMM launch in the timed region), per-call figures against the plain
streaming-read ceiling of the same bytes, the unfused comparator (dequantize
to 16 bits, then multiply), prefill / Qwen-shaped / NF4 / format-variant
figures, and the CPU oracle timed on a bounded sample on this host.  Kernel
names come from the library's own plan query (w4a16_gemm_plan), the names
the profiler reports.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import ctypes
import glob
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16/bf16 MFMA
SHAPES = [(4096, 4096), (4096, 11008), (11008, 4096)]   # (K, N)
MS = [1, 4, 16]
G = 128
PREFILL_SHAPES = [(5120, 7168), (5120, 5120), (5120, 55296), (27648, 5120)]   # (K, N)


def weight_bytes(K, N, perm=True):
    return K * N // 2 + 2 * N * K // G + N * K // (2 * G) + (4 * K if perm else 0)


def call_bytes(M, K, N):
    """Algorithmic bytes of the GEMM kernel itself: codes + scales + zeros, the
    (permuted) activations and the output.  The permutation vector is read by
    the gather (in the kernel, or the separate preparation pass)."""
    return weight_bytes(K, N, perm=False) + 2 * M * K + 2 * M * N


def plan(w4, M, N, K, dtype, perm=False, xs=False, ws=True):
    import torch
    return w4.w4a16_gemm_plan(M, N, K, G, 4, torch.float16 if dtype == "f16" else torch.bfloat16,
                              perm=perm, x_scale=xs, workspace=ws)


def main_kernel(kernels):
    """The call's GEMM kernel: the first launch that is not the preparation
    pass (the one the timing events attach to)."""
    return [k for k in kernels if not k.startswith("w4a16::prep_")][0]


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
    ap.add_argument("--no-unfused", action="store_true")
    ap.add_argument("--prefill-only", type=str, default=None,
                    help="run only the prefill of one layer, 'K,N,M' (for a per-shape profile)")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run each decode call of the workload once, then a 256 MiB device copy "
                         "(for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE), and exit")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write %s from the counter CSVs of two --pmc-probe runs under "
                         "rocprofv3 (--pmc FETCH_SIZE, then --pmc WRITE_SIZE), and exit"
                         % os.path.join("profiles", "int4_decode_traffic.json"))
    ap.add_argument("--min-rotation-mb", type=float, default=512.0)
    return ap.parse_args()


def host_info(torch, dev):
    """Provenance of the measurement: GPU, CUs, current and top sclk (sysfs),
    ROCm version, host CPU model and count.  Reads files only."""
    props = torch.cuda.get_device_properties(dev)
    info = {"gpu": props.name, "cus": props.multi_processor_count}
    try:
        arch = getattr(props, "gcnArchName", None)
        if arch:
            info["arch"] = arch
    except Exception:
        pass
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            lines = [l.strip() for l in open(path) if l.strip()]
        except OSError:
            continue
        mhz = [int(l.split(":")[1].strip().split("Mhz")[0].split("MHz")[0]) for l in lines
               if ":" in l and "hz" in l.lower()]
        cur = [l for l in lines if l.endswith("*")]
        if mhz:
            info["sclk_mhz_max"] = max(mhz)
            if cur:
                info["sclk_mhz_now"] = int(cur[0].split(":")[1].strip().split("M")[0])
            break
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            info["rocm"] = open(path).read().strip()
            break
        except OSError:
            pass
    try:
        for l in open("/proc/cpuinfo"):
            if l.startswith("model name"):
                info["host_cpu"] = l.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    info["host_cpus"] = os.cpu_count()
    info["torch"] = torch.__version__
    return info


class KernelTimer:
    """Durations of the library's main kernel launch, from hipExtLaunchKernel
    start/stop events (w4a16_set_timing_events) on the stream it runs on."""

    def __init__(self, L, hip):
        self.L, self.hip = L, hip
        self.ev = (ctypes.c_void_p * 2)()
        for k in range(2):
            if hip.hipEventCreate(ctypes.byref(self.ev, k * ctypes.sizeof(ctypes.c_void_p))):
                raise RuntimeError("hipEventCreate failed")

    def time(self, call, reps, warm=3, stat="median"):
        import torch
        ts = []
        ms = ctypes.c_float(0.0)
        for r in range(warm + reps):
            self.L.w4a16_set_timing_events(ctypes.c_void_p(self.ev[0]),
                                           ctypes.c_void_p(self.ev[1]))
            if call() != 0:
                raise RuntimeError("library call failed")
            torch.cuda.synchronize()
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.ev[0]),
                                            ctypes.c_void_p(self.ev[1])) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            if r >= warm:
                ts.append(ms.value * 1e-3)
        return float(np.median(ts) if stat == "median" else np.mean(ts))


def graph_time(fns, stream, reps=5):
    """Seconds per replay of a HIP graph that runs fns in order."""
    import torch
    for f in fns:
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for f in fns:
            f()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e-3 / reps


class StreamCeiling:
    """The plain streaming read of the library (w4a16_stream_read) over a given
    number of bytes, from rotating buffers past the caches: per-call kernel
    time (HIP events) and whole-call time (HIP-graph replays of 10 calls), the
    best of 256 / 512 / 1024 workgroups."""

    def __init__(self, L, timer, stream):
        self.L, self.timer, self.stream = L, timer, stream
        self.cache = {}

    def __call__(self, nbytes):
        import torch
        nb = (nbytes + 15) // 16 * 16
        if nb in self.cache:
            return self.cache[nb]
        R = max(2, int(np.ceil(600e6 / nb)))
        bufs = [torch.ones(nb // 4, dtype=torch.int32, device="cuda") for _ in range(R)]
        best = None
        sp = ctypes.c_void_p(self.stream.cuda_stream)
        for wg in (256, 512, 1024):
            out = torch.empty(wg * 256, dtype=torch.int32, device="cuda")
            k = [0]

            def one(b=None):
                b = bufs[k[0] % R] if b is None else b
                k[0] += 1
                return self.L.w4a16_stream_read(ctypes.c_void_p(b.data_ptr()), nb, wg,
                                                ctypes.c_void_p(out.data_ptr()), sp)
            kt = self.timer.time(one, 20)
            gt = graph_time([lambda b=bufs[i % R]: one(b) for i in range(10)], self.stream) / 10
            if best is None or kt < best["kernel_us"] * 1e-6:
                best = {"bytes": nb, "workgroups": wg, "kernel_us": round(kt * 1e6, 2),
                        "call_us": round(gt * 1e6, 2)}
            del out
        best["pct_hbm_kernel"] = round(100 * nb / (best["kernel_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)
        del bufs
        torch.cuda.empty_cache()
        self.cache[nb] = best
        return best


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_weight_only_gemm_amd as w4
    from bit_weight_only_gemm_amd import synth, _lib

    if args.traffic_summary:
        traffic_summary(w4, *args.traffic_summary)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = _lib.load()
    if args.pmc_probe:
        pmc_probe(L, dev)
        return
    stream = torch.cuda.Stream()          # graphs are captured on a non-default stream
    torch.cuda.set_stream(stream)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    hip = ctypes.CDLL("libamdhip64.so.7")
    timer = KernelTimer(L, hip)
    if args.prefill_only:
        K, N, M = (int(v) for v in args.prefill_only.split(","))
        print(json.dumps(bench_prefill(L, timer, sptr, M=M, shapes=[(K, N)])), flush=True)
        return

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

    # ---- HIP graphs.  One graph holds R consecutive steps, one over each
    # rotating weight copy (9 R GEMM calls with their act-order permutation
    # passes), the way a serving engine captures a whole model's decode step
    # (hundreds of GEMMs) in one graph: each graph launch costs a fixed gap on
    # this stack (about 20 us), which a real step amortizes over all its
    # layers.  K steps are K // R replays of it plus one replay of a graph of
    # the first K % R steps.  For reference, one-step graphs are timed too.
    def capture(nsteps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(nsteps):
                run_step(r)
        return g
    g_all = capture(R)
    g_rest = capture(args.steps % R) if args.steps % R else None
    g_one = [None] * R
    for r in range(R):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            run_step(r)
        g_one[r] = g
    torch.cuda.synchronize()
    for i in range(max(1, args.warmup // R)):
        g_all.replay()
    torch.cuda.synchronize()

    # ---- timed region, part 1: exactly K steps (graph replays), synchronized
    # both sides
    t0 = time.perf_counter()
    for i in range(args.steps // R):
        g_all.replay()
    if g_rest is not None:
        g_rest.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    # (context: the same steps with one graph per step)
    for i in range(R):
        g_one[i].replay()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(args.steps):
        g_one[i % R].replay()
    torch.cuda.synchronize()
    step1_s = (time.perf_counter() - t2) / args.steps
    graphs = [g_all, g_rest] + g_one

    # ---- timed region, part 2: the same K steps launched eagerly with HIP
    # timing events attached to every GEMM kernel's own dispatch
    # (hipExtLaunchKernel start/stop), on the stream the kernels run on.  A
    # dispatch's start event is taken when it is queued, so a kernel queued
    # behind another one would be charged that kernel's tail: a call with a
    # preparation pass drains the stream after the pass before it launches the
    # timed kernel (the library does so while timing events are pending), and
    # the stream is drained after every call, before the next one is queued.
    # (The step time above includes the pass and runs the calls back to back.)
    nper = len(calls[0])
    kern = {}
    tcalls = []
    for step_layers, cl in zip(rot, calls):
        tl = []
        for (K, N, M, q), (a, _, _, _) in zip(step_layers, cl):
            kern[(M, K, N)] = plan(w4, M, N, K, "f16", perm=True)
            tl.append(a)
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
        groups.setdefault(main_kernel(kern[(M, K, N)]), []).append(j)
    dom = max(groups, key=lambda g: dur[:, groups[g]].sum())
    dj = groups[dom]
    avg_launch_s = float(dur[:, dj].mean())
    dom_bytes = float(np.mean([calls[0][j][1] for j in dj]))
    achieved = dom_bytes / avg_launch_s / 1e9

    # ---- context: the streaming-read ceiling of each call's weight bytes
    ceil = StreamCeiling(L, timer, stream)
    per_point = []
    for j, (K, N, M, _) in enumerate(rot[0]):
        d = float(dur[:, j].mean())
        c = ceil(call_bytes(M, K, N))
        per_point.append({"M": M, "K": K, "N": N, "kernels": kern[(M, K, N)],
                          "us": round(d * 1e6, 2),
                          "weight_GBps": round(weight_bytes(K, N) / d / 1e9, 1),
                          "pct_hbm": round(100 * call_bytes(M, K, N) / d / 1e9 / HBM_PEAK_GBS, 1),
                          "stream_read_us": c["kernel_us"],
                          "x_stream_read": round(d * 1e6 / c["kernel_us"], 2)})

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
        "config": dict({
            "workload": "Llama-2-7B-shaped decode GEMMs, GPTQ act-order int4 G=128: "
                        "(K,N) in {(4096,4096),(4096,11008),(11008,4096)} x M in {1,4,16}",
            "gemm_calls_per_step": nper,
            "step_timing": "HIP graphs of R consecutive steps (one per rotating weight copy; "
                           "the GEMM kernels, plus the act-order permutation pass where the "
                           "kernel does not gather itself)",
            "weight_rotation_copies": R,
            "ms_per_step_one_step_graphs": round(step1_s * 1e3, 4),
            "tflops": round(step_flops / step_s / 1e12, 3),
            "pct_hbm_step": round(100 * step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 1),
        }, **host_info(torch, dev)),
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
    if not args.no_unfused:
        result["unfused"] = bench_unfused(w4, rot, xs, stream, step_s)
    del rot, calls, graphs, base
    torch.cuda.empty_cache()
    if not args.no_prefill:
        result["prefill"] = bench_prefill(L, timer, sptr)
        result["prefill_m8192"] = bench_prefill(L, timer, sptr, M=8192)
    if not args.no_qwen:
        result["qwen_decode"] = bench_qwen_decode(w4, ceil)
    if not args.no_nf4:
        result["nf4"] = bench_nf4(L, w4, timer, sptr, ceil)
    if not args.no_variants:
        result["variants"] = bench_variants()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(xs, outs)
    result["child_processes_at_exit"] = child_processes()
    print(json.dumps(result), flush=True)


def child_processes():
    """Processes this bench left running (it starts none itself)."""
    try:
        import psutil
        return [" ".join(p.cmdline()[:3]) for p in psutil.Process().children(recursive=True)]
    except Exception as e:
        return "unknown (%s)" % type(e).__name__


def bench_unfused(w4, rot, xs, stream, fused_step_s):
    """The pages' "default kernel": the weights dequantized to 16 bits on every
    forward, then a dense multiply -- here the library's dequant export
    (w4a16_dequant, W [N, K] fp16 in permuted column order) followed by
    torch's x[:, perm] and F.linear (hipBLASLt), for each call of the decode
    step, over the same rotating weight sets; one HIP graph per step."""
    import torch
    import torch.nn.functional as F
    R = len(rot)
    wbuf = {}
    for K, N, M, q in rot[0]:
        wbuf.setdefault((K, N), torch.empty((N, K), dtype=torch.float16, device="cuda"))

    perm64 = {id(q): q["perm"].long() for r in range(min(R, 3)) for _, _, _, q in rot[r]}

    def step_fns(r):
        fns = []
        for K, N, M, q in rot[r]:
            def f(K=K, N=N, M=M, q=q):
                wd = w4.w4a16_dequant(q, torch.float16, out=wbuf[(K, N)])
                F.linear(xs[(M, K)].index_select(1, perm64[id(q)]), wd)
            fns.append(f)
        return fns
    times = [graph_time(step_fns(r), stream) for r in range(min(R, 3))]
    t = float(np.median(times))
    return {"what": "w4a16_dequant (fp16 W written to HBM) + x[:, perm] + F.linear per call, "
                    "the 9 calls of the step in one HIP graph",
            "ms_per_step": round(t * 1e3, 4),
            "fused_speedup": round(t / fused_step_s, 2)}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "int4_decode_traffic.json")
# the translation unit of the decode kernels and what it includes
KERNEL_SOURCES = [os.path.join(ROOT, "bit_weight_only_gemm_amd", "csrc", f)
                  for f in ("gemm.hip", "decode.h", "common.h", "kernels.h", "launch.h")]


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
    print("source_hash %s" % kernel_source_hash(), flush=True)
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
            print("call M=%d K=%d N=%d kernels=%s algorithmic_bytes=%d"
                  % (M, K, N, " + ".join(plan(w4, M, N, K, "f16", perm=True)),
                     call_bytes(M, K, N)), flush=True)
    src = torch.ones(64 * 2**20, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print("copy bytes_read=%d bytes_written=%d" % (src.numel() * 4, dst.numel() * 4), flush=True)


def _counter_rows(d, counter):
    """(kernel name without 'void ' and the argument list, value) per
    dispatch, in dispatch order, from rocprofv3's counter CSV under d."""
    import csv
    path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
    rows = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            name = name[5:] if name.startswith("void ") else name
            depth, cut = 0, len(name)
            for i, ch in enumerate(name):      # the argument list: the first '(' outside <>
                depth += ch == "<"
                depth -= ch == ">"
                if ch == "(" and depth == 0:
                    cut = i
                    break
            did = int(r["Dispatch_Id"])
            rows[did] = (name[:cut], rows.get(did, (None, 0.0))[1] + float(r["Counter_Value"]))
    return [rows[k] for k in sorted(rows)]


def traffic_summary(w4, fetch_dir, write_dir):
    """HBM bytes per launch of each main kernel of the workload's decode calls
    (the --pmc-probe sequence: SHAPES x MS once each, then a 256 MiB copy):
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what they read for
    the copy (its last dispatch), against the calls' algorithmic bytes."""
    fetch, write = _counter_rows(fetch_dir, "FETCH_SIZE"), _counter_rows(write_dir, "WRITE_SIZE")
    copy_bytes = 64 * 2**20 * 4
    fscale = copy_bytes / (fetch[-1][1] * 1024)
    wscale = copy_bytes / (write[-1][1] * 1024)
    kernels, fi, wi = {}, 0, 0
    for K, N in SHAPES:
        for M in MS:
            main = main_kernel(plan(w4, M, N, K, "f16", perm=True))
            while fetch[fi][0] != main:
                fi += 1
            while write[wi][0] != main:
                wi += 1
            hbm = fetch[fi][1] * 1024 * fscale + write[wi][1] * 1024 * wscale
            k = kernels.setdefault(main, {"hbm": [], "alg": []})
            k["hbm"].append(hbm)
            k["alg"].append(call_bytes(M, K, N))
            fi += 1
            wi += 1
    out = {"source_hash": kernel_source_hash(),
           "kernels": {n: {"hbm_bytes_per_launch": round(float(np.mean(v["hbm"]))),
                           "algorithmic_bytes_per_launch": round(float(np.mean(v["alg"]))),
                           "launches": len(v["hbm"])} for n, v in kernels.items()},
           "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
           "calibration": "256 MiB device copy: FETCH_SIZE %d KiB, WRITE_SIZE %d KiB"
                          % (fetch[-1][1], write[-1][1]),
           "command": "cd /tmp && export TMPDIR=/tmp; rocprofv3 --pmc FETCH_SIZE "
                      "--output-format csv -d $REPO/gpurun_out/pmc_fetch -o run -- python3 "
                      "$REPO/bench.py --pmc-probe; rocprofv3 --pmc WRITE_SIZE --output-format "
                      "csv -d $REPO/gpurun_out/pmc_write -o run -- python3 $REPO/bench.py "
                      "--pmc-probe; python3 $REPO/bench.py --traffic-summary "
                      "$REPO/gpurun_out/pmc_fetch $REPO/gpurun_out/pmc_write"}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out, indent=1))


def bench_prefill(L, timer, sptr, M=2048, shapes=PREFILL_SHAPES):
    """Qwen2.5-32B-shaped prefill layers at M tokens, bf16 activations
    ~N(0,1) with 1 % of the input channels x20, RTN int4 G=128 weights:
    median kernel time of the fused kernel (all its launches: the main
    kernel's events cover the first, the whole call is timed too), and dense
    bf16 torch.matmul of the dequantized weights (the practical matrix-core
    ceiling) beside it.  The roofline fraction is over all the shapes
    together (total flops / total time); the best shape is reported too."""
    import torch
    import bit_weight_only_gemm_amd as w4
    from bit_weight_only_gemm_amd import synth
    dev = torch.device("cuda:0")
    pts = []
    for K, N in shapes:
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
        kernels = plan(w4, M, N, K, "bf16")
        t_main = timer.time(lambda: L.w4a16_gemm(*a), 10)
        # the whole call (every launch of it), event-timed around 10 calls
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            L.w4a16_gemm(*a)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / 10
        wd = w4.w4a16_dequant(p, torch.bfloat16)
        for _ in range(3):
            torch.matmul(x, wd.t())
        e0.record()
        for _ in range(10):
            torch.matmul(x, wd.t())
        e1.record()
        torch.cuda.synchronize()
        td = e0.elapsed_time(e1) * 1e-3 / 10
        fl = 2.0 * M * N * K
        pts.append({"M": M, "K": K, "N": N, "kernels": kernels, "us": round(t * 1e6, 1),
                    "main_kernel_us": round(t_main * 1e6, 1),
                    "tflops": round(fl / t / 1e12, 1),
                    "pct_mfma": round(100 * fl / t / 1e12 / MFMA_F16_PEAK_TFLOPS, 1),
                    "dense_bf16_matmul_tflops": round(fl / td / 1e12, 1)})
        del p, x, y, wd, ws
        torch.cuda.empty_cache()
    best = max(pts, key=lambda q: q["tflops"])
    tot_fl = sum(2.0 * q["M"] * q["N"] * q["K"] for q in pts)
    tot_t = sum(q["us"] for q in pts) * 1e-6
    allt = tot_fl / tot_t / 1e12
    return {"workload": "Qwen2.5-32B-shaped prefill, int4 G=128, bf16 x with 1% outlier "
                        "channels x20, M=" + str(M),
            "tflops_all_shapes": round(allt, 1),
            "roofline": {"bound": "mfma", "achieved": round(allt, 1),
                         "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(allt / MFMA_F16_PEAK_TFLOPS, 4),
                         "over": "all shapes (total flops / total whole-call time)",
                         "best_shape": [best["M"], best["K"], best["N"]],
                         "best_shape_frac": round(best["tflops"] / MFMA_F16_PEAK_TFLOPS, 4)},
            "points": pts}


def bench_qwen_decode(w4, ceil, Ms=(1, 16, 64)):
    """The Qwen2.5-32B-shaped layers in AWQ layout (s ~ U[0.5, 2] folded into W,
    x divided by s before the call), int4 G=128, fp16 activations, at M in
    {1, 16, 64}: whole calls by HIP-graph replay over rotating weight copies
    (>= 512 MB), weight-stream GB/s per layer and over the four layers, with
    the streaming-read ceiling of the same bytes (whole calls too)."""
    import torch
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
            t = graph_time([lambda p=ps[i % R]: w4.w4a16_gemm(x, p, out=y, workspace=ws)
                            for i in range(10)], stream) / 10
            byt = wb + 2 * M * K + 2 * M * N
            c = ceil(byt)
            pts.append({"M": M, "K": K, "N": N, "kernels": plan(w4, M, N, K, "f16"),
                        "us": round(t * 1e6, 2),
                        "weight_GBps": round(wb / t / 1e9, 1),
                        "pct_hbm": round(100 * byt / t / 1e9 / HBM_PEAK_GBS, 1),
                        "stream_read_call_us": c["call_us"],
                        "x_stream_read": round(t * 1e6 / c["call_us"], 2)})
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
    for label, bits, G_, sym, xsc in VARIANTS:
        qw, sc, qz = w4.w4a16_quantize_rtn(W, G_, sym=sym, bits=bits)
        p0 = w4.w4a16_repack(qw, sc, qz, None, G_, bits=bits)
        del qw, sc, qz
        wb = variant_weight_bytes(K, N, bits, G_, sym)
        R = max(2, int(np.ceil(512e6 / wb)))
        ps = [p0] + [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in p0.items()}
                     for _ in range(R - 1)]
        for M in Ms:
            x32 = synth.activations("C6/x/%d" % M, M, K)
            x = torch.from_numpy(synth.to_bf16_bits(x32).view(np.int16)).view(torch.bfloat16).to(dev)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            ws = w4.workspace(w4.w4a16_workspace_bytes(M, N, K, G_), dev)

            def call(p):
                if xsc:
                    w4.w4a16_gemm_xscale(x, s_awq, p, out=y, workspace=ws)
                else:
                    w4.w4a16_gemm(x, p, out=y, workspace=ws)
            t = graph_time([lambda p=ps[i % R]: call(p) for i in range(10)], stream) / 10
            pt = {"variant": label, "bits": bits, "group_size": G_, "symmetric": sym,
                  "awq_input_scales": xsc, "M": M, "us": round(t * 1e6, 2),
                  "kernels": w4.w4a16_gemm_plan(M, N, K, G_, bits, torch.bfloat16,
                                                x_scale=xsc)}
            if M >= 1024:
                fl = 2.0 * M * N * K
                pt.update(tflops=round(fl / t / 1e12, 1),
                          pct_mfma=round(100 * fl / t / 1e12 / MFMA_F16_PEAK_TFLOPS, 1))
            else:
                byt = wb + 2 * M * K + 2 * M * N
                pt.update(weight_bytes=wb, GBps=round(byt / t / 1e9, 1),
                          pct_hbm=round(100 * byt / t / 1e9 / HBM_PEAK_GBS, 1))
            pts.append(pt)
            del x, y, ws
        del ps, p0
        torch.cuda.empty_cache()
    return {"workload": "5120 x 55296 layer, bf16 activations ~N(0,1), RTN weights of each "
                        "format; whole calls by HIP-graph replay",
            "points": pts}


def bench_nf4(L, w4, timer, sptr, ceil, K=8192, N=28672):
    """The NF4 projection: W [28672, 8192] ~N(0, 0.02), blocksize 64, double
    quant over 256 blocks, bf16 x ~N(0,1) at M in {1, 32}; 4 rotating weight
    copies so the weights stream from HBM; main-kernel time (HIP events) and
    the streaming-read ceiling of the same bytes.  The codes are repacked once
    (nf4_repack) and nf4_gemm_repacked is the timed call; nf4_gemm on the
    canonical codes is timed beside it."""
    import torch
    from bit_weight_only_gemm_amd import synth
    dev = torch.device("cuda:0")
    W = torch.from_numpy(synth.weights("C5/W/%dx%d" % (K, N), N, K)).to(dev)
    p0 = w4.nf4_quantize(W)
    del W
    ps = [w4.nf4_repack({k: (v.clone() if isinstance(v, torch.Tensor) else v)
                         for k, v in p0.items()}) for _ in range(4)]
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

        def caller(fn, key):
            def call():
                p = ps[k[0] % 4]
                k[0] += 1
                return fn(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(p[key].data_ptr()),
                          ctypes.c_void_p(p["absmax_q"].data_ptr()),
                          ctypes.c_void_p(p["absmax_scale"].data_ptr()), 64,
                          ctypes.c_void_p(y.data_ptr()), M, N, K, w4.BF16, wsp, wsb, sptr)
            return call
        t = timer.time(caller(L.nf4_gemm_repacked, "qweight_r"), 20)
        tc = timer.time(caller(L.nf4_gemm, "qweight"), 20)
        byt = wb + 2 * M * K + 2 * M * N
        c = ceil(byt)
        pts.append({"M": M, "K": K, "N": N, "kernels": w4.nf4_gemm_repacked_plan(M, N, K),
                    "us": round(t * 1e6, 2),
                    "weight_GBps": round(wb / t / 1e9, 1),
                    "pct_hbm": round(100 * byt / t / 1e9 / HBM_PEAK_GBS, 1),
                    "stream_read_us": c["kernel_us"],
                    "x_stream_read": round(t * 1e6 / c["kernel_us"], 2),
                    "canonical_layout": {"kernels": w4.nf4_gemm_plan(M, N, K),
                                         "us": round(tc * 1e6, 2),
                                         "pct_hbm": round(100 * byt / tc / 1e9 / HBM_PEAK_GBS, 1)}})
    return {"workload": "NF4 28672x8192, blocksize 64, double quant 256, bf16; codes repacked "
                        "once into 1 KB tiles (nf4_repack), the canonical layout beside",
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
