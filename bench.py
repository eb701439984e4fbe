"""Benchmark of the W4A16 hot path on one MI355X.

Headline (the JSON `value`): decode GEMV M=1 over the gate_up layer shape, K=2048,
N=13312, group size 128, bf16, in algorithmic GB/s. A step is one w4a16_gemm call
(dispatch, split-K GEMV, in-kernel reduction and epilogue) on one activation
batch; the weights were repacked once before timing. Secondary entries in the same
JSON line measure the other rows of the path on their own workloads: the LM-head
repack from AWQ and from GPTQ-standard tensors (GB/s), the MFMA GEMM at M=512
(TFLOP/s), the GEMV on the other shapes and the tied-embedding gather of 512 tokens
from the packed LM head (GB/s). As context, not as the metric, it also times the same
products with dense bf16 weights through torch.matmul (the vendor GEMM library).

Timing: warm-up calls, then K calls captured in one HIP graph and replayed once
between two events on the launch stream, with a device synchronisation on both
sides. Each call reads a different copy of the packed weights, rotating through
at least 1 GiB of copies (at least 8 for the LM head), so the 256 MiB Infinity Cache
cannot serve repeats: the bytes come from HBM. (A rotation of only 4 x 139 MB ran
the LM-head GEMV about 8% slower than 8 copies; more copies only remove reuse.)

Algorithmic bytes of a GEMM (AWQ-sized): K*N/2 codes + (K/G)*N/2 zeros
+ (K/G)*N*2 scales + M*K*2 activations + M*N*2 outputs; flops 2*M*N*K.
Repack bytes: each AWQ byte read once and written once, 2*(K*N/2 + (K/G)*N/2 + (K/G)*N*2).
Gather bytes, per token: K/2 codes + (K/G)*2.5 zero and scale bytes + 4 (id) + 2K outputs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]
       python bench.py --pmc-probe     (launches for hardware-counter runs, no timing)

--pmc-probe runs, without graphs or timing, a 256 MiB device copy (the calibration
kernel for the byte counters: it reads and writes exactly 256 MiB) three times, then
the headline GEMV ten times on rotating weight copies and the LM-head M=512 GEMM three
times, so that counter runs see one dispatch per launch.
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMM GB/s (M=1) & TFLOP/s (M=512) vs roofline; repack GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published
ROTATE_BYTES = 1 << 30
MAX_COPIES = 128


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemm_bytes(M, K, N, G):
    KG = K // G
    return K * N // 2 + KG * N // 2 + KG * N * 2 + M * K * 2 + M * N * 2


def repack_bytes(K, N, G):
    KG = K // G
    return 2 * (K * N // 2 + KG * N // 2 + KG * N * 2)


def to_dev_bits(bits, dtype, dev):
    import numpy as np
    import torch
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(td).to(dev)


def time_graph(fn_list, warmup):
    """Runs warm-up calls eagerly, captures the timed calls in a graph and replays it
    once between events. Returns (elapsed_ms, launches)."""
    import torch
    for i in range(warmup):
        fn_list[i % len(fn_list)]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fn_list:
            fn()
    torch.cuda.synchronize()
    g.replay()                       # one untimed replay: graph upload, first-use costs
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end), len(fn_list)


def time_graphs_alternating(fn_lists, warmup, rounds=3):
    """Captures one graph per call list, replays each once untimed, then times
    `rounds` replays of each in alternation (a, b, a, b, ...) so that the entries
    compared see the same clock and power state. Returns the median ms of each."""
    import statistics
    import torch
    graphs = []
    for fns in fn_lists:
        for i in range(warmup):
            fns[i % len(fns)]()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for fn in fns:
                fn()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        graphs.append(g)
    stream = torch.cuda.current_stream()
    times = [[] for _ in graphs]
    for _ in range(rounds):
        for j, g in enumerate(graphs):
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record(stream)
            g.replay()
            end.record(stream)
            torch.cuda.synchronize()
            times[j].append(start.elapsed_time(end))
    return [statistics.median(t) for t in times]


def measure_gemm(w, workload, M, steps, warmup, dev, path="auto"):
    import torch
    import synth
    ws = synth.make(workload, Ms=(M,))
    K, N, G = ws.K, ws.N, ws.group_size
    qw = torch.from_numpy(ws.qweight).to(dev)
    qz = torch.from_numpy(ws.qzeros).to(dev)
    sc = to_dev_bits(ws.scale_bits, ws.dtype, dev)
    packed0 = w.w4a16_repack(qw, qz, sc, G)
    del qw, qz, sc
    pbytes = packed0.numel()
    copies = max(1, min(MAX_COPIES, math.ceil(ROTATE_BYTES / pbytes)))
    packs = [packed0] + [packed0.clone() for _ in range(copies - 1)]
    x = to_dev_bits(ws.x_bits[M], ws.dtype, dev)
    y = torch.empty((M, N), dtype=x.dtype, device=dev)
    calls = [(lambda p=packs[i % copies]: w.w4a16_gemm_ex(x, p, N, G, y=y, path=path)) for i in range(steps)]
    ms, n = time_graph(calls, warmup)
    per_launch_s = ms / 1e3 / n
    nbytes = gemm_bytes(M, K, N, G)
    flops = 2 * M * N * K
    del packs, packed0
    torch.cuda.empty_cache()
    return dict(workload=workload, M=M, K=K, N=N, group_size=G, dtype=ws.dtype, path=path,
                kernel="w4a16_gemv" if (path == "gemv" or (path == "auto" and M <= 8)) else "w4a16_gemm_mfma",
                weight_copies=copies, launches=n, us_per_launch=per_launch_s * 1e6,
                algorithmic_bytes=nbytes, flops=flops,
                GBps=nbytes / per_launch_s / 1e9, TFLOPs=flops / per_launch_s / 1e12)


def measure_w4a8(w, workload, M, steps, warmup, dev):
    """W4A8 on a 16-bit workload: the product alone from quantised activations (the
    kernel the roofline is for), and the whole step, quantisation included."""
    import torch
    import synth
    ws = synth.make(workload, Ms=(M,))
    K, N, G = ws.K, ws.N, ws.group_size
    qw = torch.from_numpy(ws.qweight).to(dev)
    qz = torch.from_numpy(ws.qzeros).to(dev)
    sc = to_dev_bits(ws.scale_bits, ws.dtype, dev)
    packed0 = w.w4a16_repack(qw, qz, sc, G)
    del qw, qz, sc
    copies = max(1, min(MAX_COPIES, math.ceil(ROTATE_BYTES / packed0.numel())))
    packs = [packed0] + [packed0.clone() for _ in range(copies - 1)]
    x = to_dev_bits(ws.x_bits[M], ws.dtype, dev)
    act = w.w4a8_quantize(x)
    y = torch.empty((M, N), dtype=x.dtype, device=dev)
    gemm_calls = [(lambda p=packs[i % copies]: w.w4a8_gemm(act, p, M, K, N, G, x.dtype, y=y)) for i in range(steps)]
    step_calls = [(lambda p=packs[i % copies]: w.w4a8_linear(x, p, N, G, y=y, act=act)) for i in range(steps)]
    gemm_ms, step_ms = time_graphs_alternating([gemm_calls, step_calls], warmup)
    n = steps
    gemm_s = gemm_ms / 1e3 / n
    step_s = step_ms / 1e3 / n
    flops = 2 * M * N * K
    del packs, packed0
    torch.cuda.empty_cache()
    return dict(workload=workload, M=M, K=K, N=N, group_size=G, dtype=ws.dtype, activations="fp8 e4m3",
                kernel="w4a8_gemm_mfma", weight_copies=copies, launches=n, us_per_launch=gemm_s * 1e6,
                us_per_step_with_quantize=step_s * 1e6, flops=flops, TFLOPs=flops / gemm_s / 1e12,
                TFLOPs_step=flops / step_s / 1e12)


def measure_repack(w, workload, steps, warmup, dev, fmt="awq"):
    """fmt "awq": w4a16_repack from AWQ tensors; "gptq": w4a16_repack_gptq from
    GPTQ-standard tensors of the same shape (same recipe, same byte count)."""
    import torch
    import synth
    if fmt == "awq":
        ws = synth.make(workload, Ms=())
        fn = w.w4a16_repack
    else:
        wl = synth.WORKLOADS[workload]
        ws = synth.draw_gptq_weights(wl.seed, wl.K, wl.N, wl.dtype, wl.group_size)
        fn = w.w4a16_repack_gptq
    K, N, G = ws.K, ws.N, ws.group_size
    qw = torch.from_numpy(ws.qweight).to(dev)
    qz = torch.from_numpy(ws.qzeros).to(dev)
    sc = to_dev_bits(ws.scale_bits, ws.dtype, dev)
    pbytes = w.w4a16_packed_bytes(K, N, G)
    in_bytes = qw.numel() * 4 + qz.numel() * 4 + sc.numel() * 2
    copies = max(1, min(16, math.ceil(ROTATE_BYTES / (in_bytes + pbytes))))
    ins = [(qw, qz, sc)] + [(qw.clone(), qz.clone(), sc.clone()) for _ in range(copies - 1)]
    outs = [torch.empty(pbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
    calls = [(lambda a=ins[i % copies], o=outs[i % copies]: fn(a[0], a[1], a[2], G, packed=o))
             for i in range(steps)]
    ms, n = time_graph(calls, warmup)
    per_launch_s = ms / 1e3 / n
    nbytes = repack_bytes(K, N, G)
    del ins, outs
    torch.cuda.empty_cache()
    return dict(workload=workload + (" repack" if fmt == "awq" else " repack from GPTQ"), K=K, N=N, group_size=G,
                dtype=ws.dtype, kernel="w4a16_repack" if fmt == "awq" else "w4a16_repack_gptq",
                copies=copies, launches=n, us_per_launch=per_launch_s * 1e6, algorithmic_bytes=nbytes,
                GBps=nbytes / per_launch_s / 1e9)


def embedding_bytes(T, K, G):
    """Algorithmic bytes of a T-token gather: per token its K codes (K/2 bytes), its
    K/G zeros and scales (2.5 bytes each), the id (4 bytes) and the K outputs (2K)."""
    return T * (K // 2 + (K // G) * 5 // 2 + 4 + 2 * K)


def measure_embedding(w, workload, T, steps, warmup, dev):
    import numpy as np
    import torch
    import synth
    ws = synth.make(workload, Ms=())
    K, N, G = ws.K, ws.N, ws.group_size
    qw = torch.from_numpy(ws.qweight).to(dev)
    qz = torch.from_numpy(ws.qzeros).to(dev)
    sc = to_dev_bits(ws.scale_bits, ws.dtype, dev)
    packed0 = w.w4a16_repack(qw, qz, sc, G)
    del qw, qz, sc
    copies = max(1, min(MAX_COPIES, math.ceil(ROTATE_BYTES / packed0.numel())))
    packs = [packed0] + [packed0.clone() for _ in range(copies - 1)]
    # a different set of prompt tokens per call, so repeated calls do not re-read the
    # same columns from the caches
    ids = [torch.from_numpy(synth.draw_token_ids(7000 + i, T, N)).to(dev) for i in range(steps)]
    out = torch.empty((T, K), dtype=torch.bfloat16 if ws.dtype == "bf16" else torch.float16, device=dev)
    calls = [(lambda p=packs[i % copies], t=ids[i]: w.w4a16_embedding(t, p, K, N, G, out.dtype, out=out))
             for i in range(steps)]
    ms, n = time_graph(calls, warmup)
    per_launch_s = ms / 1e3 / n
    nbytes = embedding_bytes(T, K, G)
    del packs, packed0, ids
    torch.cuda.empty_cache()
    return dict(workload=workload + " tied-embedding gather", T=T, K=K, N=N, group_size=G, dtype=ws.dtype,
                kernel="w4a16_embedding", weight_copies=copies, launches=n, us_per_launch=per_launch_s * 1e6,
                algorithmic_bytes=nbytes, GBps=nbytes / per_launch_s / 1e9)


def measure_dense_reference(workload, M, steps, warmup, dev):
    """Context, not the metric: the same product with dense bf16 weights through
    torch.matmul (the vendor GEMM library), weights rotated through >= 1 GiB of copies
    and timed like the W4A16 entries. Algorithmic bytes: K*N*2 weights + M*K*2 + M*N*2."""
    import torch
    import synth
    shape = synth.WORKLOADS[workload]
    K, N = shape.K, shape.N
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    w0 = (torch.randn((K, N), device=dev, generator=g) * 0.05).to(torch.bfloat16)
    copies = max(1, min(MAX_COPIES, math.ceil(ROTATE_BYTES / (K * N * 2))))
    ws = [w0] + [w0.clone() for _ in range(copies - 1)]
    x = torch.randn((M, K), device=dev, generator=g).to(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    calls = [(lambda wt=ws[i % copies]: torch.matmul(x, wt, out=y)) for i in range(steps)]
    try:
        ms, n = time_graph(calls, warmup)
        how = "HIP graph of K calls, events"
    except Exception as exc:  # a library call that cannot be captured: time it eagerly
        torch.cuda.synchronize()
        log(f"dense reference not capturable ({type(exc).__name__}); timed eagerly")
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for fn in calls:
            fn()
        end.record()
        torch.cuda.synchronize()
        ms, n = start.elapsed_time(end), len(calls)
        how = "eager launches, events"
    per_launch_s = ms / 1e3 / n
    nbytes = K * N * 2 + M * K * 2 + M * N * 2
    flops = 2 * M * N * K
    del ws, w0
    torch.cuda.empty_cache()
    return dict(workload=workload, M=M, K=K, N=N, dtype="bf16", kind="dense bf16 weights, torch.matmul",
                weight_copies=copies, launches=n, timing=how, us_per_launch=per_launch_s * 1e6,
                algorithmic_bytes=nbytes, flops=flops, GBps=nbytes / per_launch_s / 1e9,
                TFLOPs=flops / per_launch_s / 1e12)


def roofline_hbm(entry, traffic=None):
    return {"bound": "hbm", "achieved": round(entry["GBps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(entry["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic}


def roofline_mfma(entry, peak=None):
    peak = MFMA_BF16_PEAK_TFLOPS if peak is None else peak
    return {"bound": "mfma", "achieved": round(entry["TFLOPs"], 1), "peak": peak,
            "unit": "TFLOP/s", "frac": round(entry["TFLOPs"] / peak, 4), "traffic": None}


CALIBRATION_COPY_BYTES = 256 << 20
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "gemv_gate_up_decode_M1_counters.md")
GEMV_SOURCES = ("w4a16_int4_weight_amd/csrc/gemv.hip", "w4a16_int4_weight_amd/csrc/device_common.h")


def gemv_source_hash():
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic():
    """HBM bytes per headline launch from the committed byte-counter summary, or None
    when there is none or the GEMV source changed since the counters were taken."""
    try:
        with open(COUNTER_SUMMARY) as f:
            text = f.read()
    except OSError:
        return None
    vals = dict(re.findall(r"^(traffic_bytes_per_launch|kernel_source_sha256_16): (\S+)$", text, re.M))
    if vals.get("kernel_source_sha256_16") != gemv_source_hash() or "traffic_bytes_per_launch" not in vals:
        return None
    return int(vals["traffic_bytes_per_launch"])


def pmc_probe(dev):
    import torch
    import synth
    import w4a16_int4_weight_amd as w
    src = torch.empty(CALIBRATION_COPY_BYTES, dtype=torch.uint8, device=dev).fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    ws = synth.make("gate_up_decode", Ms=(1,))
    qw = torch.from_numpy(ws.qweight).to(dev)
    qz = torch.from_numpy(ws.qzeros).to(dev)
    sc = to_dev_bits(ws.scale_bits, ws.dtype, dev)
    packed0 = w.w4a16_repack(qw, qz, sc, ws.group_size)
    packs = [packed0] + [packed0.clone() for _ in range(9)]
    x = to_dev_bits(ws.x_bits[1], ws.dtype, dev)
    y = torch.empty((1, ws.N), dtype=x.dtype, device=dev)
    torch.cuda.synchronize()
    for i in range(10):
        w.w4a16_gemm(x, packs[i], ws.N, ws.group_size, y=y)
    torch.cuda.synchronize()
    del packs, packed0
    # the MFMA GEMM on the LM-head prefill (M=512), three launches on one weight copy
    ws = synth.make("lm_head", Ms=(512,))
    qw = torch.from_numpy(ws.qweight).to(dev)
    qz = torch.from_numpy(ws.qzeros).to(dev)
    sc = to_dev_bits(ws.scale_bits, ws.dtype, dev)
    packed = w.w4a16_repack(qw, qz, sc, ws.group_size)
    del qw, qz, sc
    x = to_dev_bits(ws.x_bits[512], ws.dtype, dev)
    y = torch.empty((512, ws.N), dtype=x.dtype, device=dev)
    torch.cuda.synchronize()
    for _ in range(3):
        w.w4a16_gemm(x, packed, ws.N, ws.group_size, y=y)
    torch.cuda.synchronize()
    # the W4A8 GEMM on the same weights, three launches from one quantised activation buffer
    act = w.w4a8_quantize(x)
    for _ in range(3):
        w.w4a8_gemm(act, packed, 512, ws.K, ws.N, ws.group_size, x.dtype, y=y)
    torch.cuda.synchronize()
    log("pmc probe done: 3 x 256 MiB copy, 10 x gate_up_decode GEMV, 3 x lm_head M=512 GEMM, "
        "3 x lm_head M=512 W4A8 GEMM")


def cpu_baseline(workload, M, budget_s=15.0):
    """The oracle as it stands (unpack, float64 dequant, float64 matmul), BLAS held
    to one thread, timed on whole steps of the same workload until ~budget_s."""
    import numpy as np
    import synth
    from oracle import gemm as ogemm
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    ws = synth.make(workload, Ms=(M,))
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        n = 0
        while True:
            ogemm.w4a16_reference(ws.x_bits[M], ws.qweight, ws.qzeros, ws.scale_bits, ws.dtype, ws.group_size)
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = (time.perf_counter() - t0) / n
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    nbytes = gemm_bytes(M, ws.K, ws.N, ws.group_size)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} whole steps of {workload} M={M} ({dt:.2f} s each): AWQ unpack, float64 dequant, "
                      f"float64 matmul, BLAS limited to 1 thread, elementwise NumPy single-threaded"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline only, no secondary entries")
    ap.add_argument("--pmc-probe", action="store_true", help="launches for counter runs, no timing")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path, so --gpus {args.gpus} "
              "is not supported (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import torch
    import w4a16_int4_weight_amd as w
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"device {torch.cuda.get_device_name(0)}")
    if args.pmc_probe:
        pmc_probe(dev)
        return

    head = measure_gemm(w, "gate_up_decode", 1, args.steps, args.warmup, dev)
    log(f"headline gate_up_decode M=1: {head['us_per_launch']:.2f} us, {head['GBps']:.0f} GB/s")
    secondary = []
    if not args.quick:
        for wl, M in [("lm_head", 1), ("down_proj", 1), ("down_proj", 8), ("down_proj", 16),
                      ("qkv_prefill", 512), ("gate_up_prefill", 512), ("lm_head", 512)]:
            steps = args.steps if M <= 16 else max(20, args.steps // 4)
            e = measure_gemm(w, wl, M, steps, min(args.warmup, 10), dev)
            e["roofline"] = roofline_hbm(e) if M <= 16 else roofline_mfma(e)
            log(f"{wl} M={M}: {e['us_per_launch']:.2f} us, {e['GBps']:.0f} GB/s, {e['TFLOPs']:.1f} TFLOP/s")
            secondary.append(e)
        r = measure_repack(w, "lm_head", max(10, args.steps // 10), 3, dev)
        r["roofline"] = roofline_hbm(r)
        log(f"lm_head repack: {r['us_per_launch']:.1f} us, {r['GBps']:.0f} GB/s")
        secondary.append(r)
        r = measure_repack(w, "lm_head", max(10, args.steps // 10), 3, dev, fmt="gptq")
        r["roofline"] = roofline_hbm(r)
        log(f"lm_head repack from GPTQ: {r['us_per_launch']:.1f} us, {r['GBps']:.0f} GB/s")
        secondary.append(r)
        for wl in ("qkv_prefill", "gate_up_prefill", "lm_head"):
            e = measure_w4a8(w, wl, 512, max(20, args.steps // 4), min(args.warmup, 10), dev)
            e["roofline"] = roofline_mfma(e, MFMA_FP8_PEAK_TFLOPS)
            log(f"{wl} W4A8 M=512: {e['us_per_launch']:.2f} us, {e['TFLOPs']:.1f} TFLOP/s (with quantisation "
                f"{e['us_per_step_with_quantize']:.2f} us)")
            secondary.append(e)
        e = measure_embedding(w, "lm_head", 512, args.steps, min(args.warmup, 10), dev)
        e["roofline"] = roofline_hbm(e)
        log(f"lm_head tied-embedding gather T=512: {e['us_per_launch']:.2f} us, {e['GBps']:.0f} GB/s")
        secondary.append(e)

    dense = []
    if not args.quick:
        # context: the same products with dense bf16 weights (4x the weight bytes)
        w4 = {(head["workload"], 1): head}
        w4.update({(e["workload"], e["M"]): e for e in secondary if "M" in e and "activations" not in e})
        for wl, M in [("gate_up_decode", 1), ("down_proj", 1), ("lm_head", 1), ("qkv_prefill", 512),
                      ("gate_up_prefill", 512), ("lm_head", 512)]:
            steps = args.steps if M <= 16 else max(20, args.steps // 4)
            d = measure_dense_reference(wl, M, steps, min(args.warmup, 10), dev)
            if (wl, M) in w4:
                d["w4a16_speedup"] = round(d["us_per_launch"] / w4[(wl, M)]["us_per_launch"], 3)
            log(f"dense bf16 reference {wl} M={M}: {d['us_per_launch']:.2f} us, {d['GBps']:.0f} GB/s, "
                f"{d['TFLOPs']:.1f} TFLOP/s")
            dense.append(d)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline("gate_up_decode", 1)
        log(f"cpu baseline: {cpu['value']} GB/s")

    line = {
        "metric": METRIC,
        "value": round(head["GBps"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_launch"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gate_up_decode: W4A16 GEMV M=1 K=2048 N=13312 group_size=128 bf16",
                   "M": 1, "K": 2048, "N": 13312, "group_size": 128,
                   "weight_copies_rotated": head["weight_copies"], "timing": "HIP graph of K calls, events"},
        "roofline": roofline_hbm(head, counter_traffic()),
        "cpu_baseline": cpu,
        "secondary": secondary,
        "dense_bf16_reference": dense,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
