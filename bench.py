"""Benchmark of the W4A16 hot path on one MI355X.

Headline (the JSON `value`): decode GEMV M=1 over the gate_up layer shape, K=2048,
N=13312, group size 128, bf16, in algorithmic GB/s. A step is one w4a16_gemm call
(dispatch, split-K GEMV, in-kernel reduction and epilogue) on one activation
batch; the weights were repacked once before timing. Secondary entries in the same
JSON line measure the other rows of the path on their own workloads: the GEMV on the
down-projection and LM-head shapes, the MFMA GEMM at M=512 (TFLOP/s), the W4A8 GEMM,
the LM-head repack from AWQ and from GPTQ-standard tensors (GB/s) and the
tied-embedding gather of 512 tokens from the packed LM head (GB/s).

Timing of every entry:
  * the weights (or repack inputs) exist in `copies` copies spanning >= 1 GiB, call i
    reading copy i mod copies, so a copy is never read twice within 1 GiB of traffic;
  * W warm-up calls run eagerly, then exactly K calls (--steps) are captured in one HIP
    graph and replayed once untimed; every entry after the headline (and its streaming
    reference) then replays the graph untimed, after scrubs, until SETTLE_CALLS calls
    have run over its just-written weight copies;
  * REPLAYS timed replays follow, each preceded by a 512 MiB streaming read of another
    buffer (the MALL scrub: the 256 MiB Infinity Cache then holds none of the copies),
    with a synchronisation before the scrub and after the replay;
  * the interval is read from the GPU's wall clock (w4a16_clock_stamp, 100 MHz),
    stamped by a one-lane kernel captured as the graph's first node and again as its
    last: it holds the GPU's execution of the K calls plus one stamp kernel (3.7 us per
    replay when no call sits between the stamps), and not the host's graph-launch
    latency. HIP events cannot be recorded inside a graph with this PyTorch build, and
    events recorded around the replay add ~9-11 us per replay (graphs of 0 to 200 calls:
    15.0 us against 3.7 us with nothing between, 5.70 against 5.15 us per call at K = 20,
    5.08 against 5.02 at K = 200); the event figure is reported beside the stamped one
    (`us_per_launch_events`);
  * per-launch time = stamped interval / K; the entry reports the median over replays
    (the value used everywhere), p10 and p90, the copies one replay touches and their
    bytes.
So with the default K every call reads its weights from HBM, and with any K the first
read of every copy in a replay does.

Achievable references beside each entry, timed the same way (context, not targets):
  * HBM-bound entries: w4a16_stream_read over the entry's algorithmic byte count (a
    plain 16-byte streaming read; for the repack, w4a16_stream_copy of half the bytes,
    reading one half and writing the other), reported as `achievable` and
    `frac_of_achievable` in the entry's roofline object;
  * MFMA-bound entries: the same product with dense bf16 weights through torch.matmul
    (the vendor GEMM library), reported in `dense_bf16_reference`.

The LM-head GEMV, a 140 MB stream, runs faster for its first ~80 back-to-back
launches than after (the chip's response to a sustained ~6 TB/s stream): its entry
carries a `fresh` state (replays of 20 calls after the scrub) and a `sustained` state
(the third of three back-to-back replays of 128 calls).

Algorithmic bytes of a GEMM (AWQ-sized): K*N/2 codes + (K/G)*N/2 zeros
+ (K/G)*N*2 scales + M*K*2 activations + M*N*2 outputs; flops 2*M*N*K.
Repack bytes: each AWQ byte read once and written once, 2*(K*N/2 + (K/G)*N/2 + (K/G)*N*2).
Gather bytes, per token: K/2 codes + (K/G)*2.5 zero and scale bytes + 4 (id) + 2K outputs.

cpu_baseline: the oracle as it stands (AWQ unpack, float64 dequant, float64 matmul) on
whole steps of the headline workload, on the host's cores: once on a pool of one
thread per allotted core (each thread the oracle on its own range of output columns,
BLAS held to one thread each), once on one thread.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]
       python bench.py --pmc-probe     (launches for hardware-counter runs, no timing)

--pmc-probe runs, without graphs or timing, a 256 MiB device copy (the calibration
kernel for the byte counters: it reads and writes exactly 256 MiB) three times, then
the headline GEMV ten times on rotating weight copies, the down-projection GEMV at M=1
and M=8 ten times each, the LM-head repack 1 + 3 times and the LM-head M=512 GEMM and
W4A8 GEMM three times each, so that counter runs see one dispatch per launch.
"""

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 GEMM GB/s (M=1) & TFLOP/s (M=512) vs roofline; repack GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published
ROTATE_BYTES = 1 << 30          # weight copies per entry span at least this
SCRUB_BYTES = 512 << 20         # streaming read between timed replays (2x the Infinity Cache)
MAX_COPIES = 128
REPLAYS = 7
LM_HEAD_FRESH_CALLS = 20
# Untimed launches each entry other than the headline (and its streaming reference)
# runs over its weight copies before timing, in replays after scrubs like the timed
# ones: over copies just allocated and written, the LM-head GEMV's first few hundred
# launches measured up to 30% slower (29 -> 22.8 us per launch in 20-call replays after
# scrubs) than every later one. The headline keeps exactly its W warm-up calls.
SETTLE_CALLS = 400
SUSTAINED_CALLS = 128
CPU_THREADS_CAP = 16            # the host cores allotted to one GPU


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gemm_bytes(M, K, N, G):
    KG = K // G
    return K * N // 2 + KG * N // 2 + KG * N * 2 + M * K * 2 + M * N * 2


def repack_bytes(K, N, G):
    KG = K // G
    return 2 * (K * N // 2 + KG * N // 2 + KG * N * 2)


def embedding_bytes(T, K, G):
    """Algorithmic bytes of a T-token gather: per token its K codes (K/2 bytes), its
    K/G zeros and scales (2.5 bytes each), the id (4 bytes) and the K outputs (2K)."""
    return T * (K // 2 + (K // G) * 5 // 2 + 4 + 2 * K)


def to_dev_bits(bits, dtype, dev):
    import numpy as np
    import torch
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(td).to(dev)


def copies_for(nbytes, cap=MAX_COPIES):
    return max(1, min(cap, math.ceil(ROTATE_BYTES / max(nbytes, 1))))


def pct(vals, q):
    """q-th percentile (0..100) of a small sample, linear interpolation."""
    s = sorted(vals)
    if len(s) == 1:
        return s[0]
    pos = (len(s) - 1) * q / 100.0
    lo = int(math.floor(pos))
    hi = min(lo + 1, len(s) - 1)
    return s[lo] + (s[hi] - s[lo]) * (pos - lo)


class Timer:
    """Graph capture, MALL scrub and GPU-clock timing shared by every entry."""

    def __init__(self, w, dev, steps, warmup, replays=REPLAYS):
        import torch
        self.w, self.dev, self.steps, self.warmup, self.replays = w, dev, steps, warmup, replays
        self.settle = False          # switched on after the headline (see SETTLE_CALLS)
        self.scrub_buf = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        self.scrub_sink = torch.empty(w.w4a16_stream_sink_bytes(SCRUB_BYTES), dtype=torch.uint8, device=dev)
        self.stamps = torch.zeros(2, dtype=torch.int64, device=dev)
        self.clock_hz = w.w4a16_wall_clock_hz()

    def scrub(self):
        self.w.w4a16_stream_read(self.scrub_buf, sink=self.scrub_sink)

    def capture(self, fns):
        """A graph of the calls between two wall-clock stamps (first and last node)."""
        import torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.w.w4a16_clock_stamp(self.stamps, 0)
            for fn in fns:
                fn()
            self.w.w4a16_clock_stamp(self.stamps, 1)
        torch.cuda.synchronize()
        g.replay()                   # untimed: graph upload, first-use costs
        torch.cuda.synchronize()
        return g

    def stamped_ms(self):
        """The interval between the last replay's two stamps, in ms (after a sync)."""
        a, b = self.stamps.cpu().tolist()
        return (b - a) * 1e3 / self.clock_hz

    def replay_ms(self, g):
        """One timed replay after a scrub: (stamped interval, interval between events
        recorded around the replay), in ms."""
        import torch
        stream = torch.cuda.current_stream()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        self.scrub()
        start.record(stream)
        g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        return self.stamped_ms(), start.elapsed_time(end)

    def time(self, rotation, copies, bytes_per_copy, calls=None, settle=None):
        """rotation[i] is a call reading copy i mod copies. Runs the warm-up, captures
        `calls` (default K) calls, times self.replays replays after scrubs. Returns the
        per-launch statistics in microseconds. settle: first replay the graph untimed,
        each replay after a scrub, until SETTLE_CALLS calls have run (the entry's weight
        copies were just allocated and written; see SETTLE_CALLS)."""
        import torch
        n = self.steps if calls is None else calls
        for i in range(self.warmup):
            rotation[(n + i) % len(rotation)]()
        torch.cuda.synchronize()
        g = self.capture([rotation[i % len(rotation)] for i in range(n)])
        settle = self.settle if settle is None else settle
        if settle:
            for _ in range(max(1, math.ceil(SETTLE_CALLS / n))):
                self.replay_ms(g)
        both = [self.replay_ms(g) for _ in range(self.replays)]
        per = [s * 1e3 / n for s, _ in both]
        per_events = [e * 1e3 / n for _, e in both]
        del g
        touched = min(n, copies)
        return {"us_per_launch": statistics.median(per), "us_p10": pct(per, 10), "us_p90": pct(per, 90),
                "us_per_launch_events": statistics.median(per_events),
                "replays": self.replays, "calls_per_replay": n, "copies": copies, "copies_touched_per_replay": touched,
                "footprint_bytes_per_replay": touched * bytes_per_copy, "mall_scrub_bytes": SCRUB_BYTES,
                "settle_calls": (max(1, math.ceil(SETTLE_CALLS / n)) * n) if settle else 0}

    def time_sustained(self, rotation, calls=SUSTAINED_CALLS):
        """Three back-to-back replays of `calls` launches (no scrub, no host
        synchronisation between them); the third, read from its stamps, is timed.
        Returns microseconds per launch."""
        import torch
        g = self.capture([rotation[i % len(rotation)] for i in range(calls)])
        torch.cuda.synchronize()
        g.replay()
        g.replay()
        g.replay()
        torch.cuda.synchronize()
        us = self.stamped_ms() * 1e3 / calls
        del g
        return us

    def stream_floor(self, nbytes, copy=False):
        """The streaming reference over `nbytes` algorithmic bytes: a read of nbytes, or
        (copy=True) a copy of nbytes / 2 (reading one half, writing the other)."""
        import torch
        w = self.w
        part = (nbytes // 2 if copy else nbytes) // 16 * 16
        per_copy = 2 * part if copy else part
        copies = copies_for(per_copy)
        srcs = [torch.empty(part, dtype=torch.uint8, device=self.dev).fill_(3) for _ in range(copies)]
        if copy:
            dsts = [torch.empty(part, dtype=torch.uint8, device=self.dev) for _ in range(copies)]
            rotation = [(lambda s=srcs[i], d=dsts[i]: w.w4a16_stream_copy(s, d)) for i in range(copies)]
        else:
            sink = torch.empty(w.w4a16_stream_sink_bytes(part), dtype=torch.uint8, device=self.dev)
            rotation = [(lambda s=srcs[i]: w.w4a16_stream_read(s, sink=sink)) for i in range(copies)]
        t = self.time(rotation, copies, per_copy)
        del srcs, rotation
        if copy:
            del dsts
        torch.cuda.empty_cache()
        return {"kernel": "w4a16_stream_copy" if copy else "w4a16_stream_read", "bytes": 2 * part if copy else part,
                "us_per_launch": round(t["us_per_launch"], 3), "us_p10": round(t["us_p10"], 3),
                "us_p90": round(t["us_p90"], 3), "GBps": round(nbytes / t["us_per_launch"] / 1e3, 1)}


_WEIGHT_SETS = {}


def weight_set(workload):
    """synth.make(workload) with every M of the workload, drawn once per process."""
    import synth
    if workload not in _WEIGHT_SETS:
        _WEIGHT_SETS[workload] = synth.make(workload)
    return _WEIGHT_SETS[workload]


def packed_copies(w, ws, dev):
    import torch
    qw = torch.from_numpy(ws.qweight).to(dev)
    qz = torch.from_numpy(ws.qzeros).to(dev)
    sc = to_dev_bits(ws.scale_bits, ws.dtype, dev)
    packed0 = w.w4a16_repack(qw, qz, sc, ws.group_size)
    del qw, qz, sc
    copies = copies_for(packed0.numel())
    return [packed0] + [packed0.clone() for _ in range(copies - 1)]


def round_entry(e):
    for k in ("us_per_launch", "us_p10", "us_p90", "us_per_launch_events"):
        if k in e:
            e[k] = round(e[k], 3)
    return e


def measure_gemm(T, w, workload, M, dev, path="auto", sustained=False):
    import torch
    ws = weight_set(workload)
    K, N, G = ws.K, ws.N, ws.group_size
    packs = packed_copies(w, ws, dev)
    copies = len(packs)
    x = to_dev_bits(ws.x_bits[M], ws.dtype, dev)
    y = torch.empty((M, N), dtype=x.dtype, device=dev)
    rotation = [(lambda p=packs[i]: w.w4a16_gemm_ex(x, p, N, G, y=y, path=path)) for i in range(copies)]
    nbytes = gemm_bytes(M, K, N, G)
    flops = 2 * M * N * K
    e = dict(workload=workload, M=M, K=K, N=N, group_size=G, dtype=ws.dtype, path=path,
             algorithmic_bytes=nbytes, flops=flops)
    if sustained:
        # fresh: replays of a few calls after the scrub; sustained: back-to-back launches
        e.update(T.time(rotation, copies, packs[0].numel(), calls=LM_HEAD_FRESH_CALLS))
        e["state"] = f"fresh: {LM_HEAD_FRESH_CALLS} calls per replay after the scrub"
        us_s = T.time_sustained(rotation)
        e["sustained"] = {"us_per_launch": round(us_s, 3), "GBps": round(nbytes / us_s / 1e3, 1),
                          "calls": SUSTAINED_CALLS,
                          "timing": f"third of three back-to-back replays of {SUSTAINED_CALLS} calls, "
                                    "read from its stamps"}
    else:
        e.update(T.time(rotation, copies, packs[0].numel()))
    del packs, rotation
    torch.cuda.empty_cache()
    us = e["us_per_launch"]
    e["GBps"] = nbytes / us / 1e3
    e["TFLOPs"] = flops / us / 1e6
    return round_entry(e)


def measure_w4a8(T, w, workload, M, dev):
    """W4A8 on a 16-bit workload: the product alone from quantised activations (the
    kernel the roofline is for), and the whole step with the activation quantisation."""
    import torch
    ws = weight_set(workload)
    K, N, G = ws.K, ws.N, ws.group_size
    packs = packed_copies(w, ws, dev)
    copies = len(packs)
    x = to_dev_bits(ws.x_bits[M], ws.dtype, dev)
    act = w.w4a8_quantize(x)
    y = torch.empty((M, N), dtype=x.dtype, device=dev)
    gemm_rot = [(lambda p=packs[i]: w.w4a8_gemm(act, p, M, K, N, G, x.dtype, y=y)) for i in range(copies)]
    step_rot = [(lambda p=packs[i]: w.w4a8_linear(x, p, N, G, y=y, act=act)) for i in range(copies)]
    flops = 2 * M * N * K
    e = dict(workload=workload, M=M, K=K, N=N, group_size=G, dtype=ws.dtype, activations="fp8 e4m3",
             kernel="w4a8_gemm_mfma", flops=flops)
    e.update(T.time(gemm_rot, copies, packs[0].numel()))
    step = T.time(step_rot, copies, packs[0].numel())
    e["us_per_step_with_quantize"] = round(step["us_per_launch"], 3)
    e["TFLOPs"] = flops / e["us_per_launch"] / 1e6
    e["TFLOPs_step"] = flops / step["us_per_launch"] / 1e6
    del packs, gemm_rot, step_rot
    torch.cuda.empty_cache()
    return round_entry(e)


def measure_repack(T, w, workload, dev, fmt="awq"):
    """fmt "awq": w4a16_repack from AWQ tensors; "gptq": w4a16_repack_gptq from
    GPTQ-standard tensors of the same shape (same recipe, same byte count)."""
    import torch
    import synth
    if fmt == "awq":
        ws = weight_set(workload)
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
    copies = copies_for(in_bytes + pbytes, cap=16)
    ins = [(qw, qz, sc)] + [(qw.clone(), qz.clone(), sc.clone()) for _ in range(copies - 1)]
    outs = [torch.empty(pbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
    rotation = [(lambda a=ins[i], o=outs[i]: fn(a[0], a[1], a[2], G, packed=o)) for i in range(copies)]
    nbytes = repack_bytes(K, N, G)
    e = dict(workload=workload + (" repack" if fmt == "awq" else " repack from GPTQ"), K=K, N=N, group_size=G,
             dtype=ws.dtype, kernel="w4a16_repack" if fmt == "awq" else "w4a16_repack_gptq",
             algorithmic_bytes=nbytes)
    e.update(T.time(rotation, copies, in_bytes + pbytes))
    del ins, outs, rotation
    torch.cuda.empty_cache()
    e["GBps"] = nbytes / e["us_per_launch"] / 1e3
    return round_entry(e)


def measure_embedding(T, w, workload, tokens, dev):
    import torch
    import synth
    ws = weight_set(workload)
    K, N, G = ws.K, ws.N, ws.group_size
    packs = packed_copies(w, ws, dev)
    copies = len(packs)
    # a different set of prompt tokens per copy, so repeated calls do not re-read the
    # same columns from the caches
    ids = [torch.from_numpy(synth.draw_token_ids(7000 + i, tokens, N)).to(dev) for i in range(copies)]
    out = torch.empty((tokens, K), dtype=torch.bfloat16 if ws.dtype == "bf16" else torch.float16, device=dev)
    rotation = [(lambda p=packs[i], t=ids[i]: w.w4a16_embedding(t, p, K, N, G, out.dtype, out=out))
                for i in range(copies)]
    nbytes = embedding_bytes(tokens, K, G)
    e = dict(workload=workload + " tied-embedding gather", T=tokens, K=K, N=N, group_size=G, dtype=ws.dtype,
             kernel="w4a16_embedding", algorithmic_bytes=nbytes)
    e.update(T.time(rotation, copies, packs[0].numel()))
    del packs, ids, rotation
    torch.cuda.empty_cache()
    e["GBps"] = nbytes / e["us_per_launch"] / 1e3
    return round_entry(e)


def measure_dense_reference(T, workload, M, dev):
    """Context, not the metric: the same product with dense bf16 weights through
    torch.matmul (the vendor GEMM library), weights rotated and timed like the W4A16
    entries. Algorithmic bytes: K*N*2 weights + M*K*2 + M*N*2."""
    import torch
    import synth
    shape = synth.WORKLOADS[workload]
    K, N = shape.K, shape.N
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    w0 = (torch.randn((K, N), device=dev, generator=g) * 0.05).to(torch.bfloat16)
    copies = copies_for(K * N * 2)
    wts = [w0] + [w0.clone() for _ in range(copies - 1)]
    x = torch.randn((M, K), device=dev, generator=g).to(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    rotation = [(lambda wt=wts[i]: torch.matmul(x, wt, out=y)) for i in range(copies)]
    nbytes = K * N * 2 + M * K * 2 + M * N * 2
    flops = 2 * M * N * K
    e = dict(workload=workload, M=M, K=K, N=N, dtype="bf16", kind="dense bf16 weights, torch.matmul",
             algorithmic_bytes=nbytes, flops=flops)
    e.update(T.time(rotation, copies, K * N * 2))
    del wts, w0, rotation
    torch.cuda.empty_cache()
    e["GBps"] = nbytes / e["us_per_launch"] / 1e3
    e["TFLOPs"] = flops / e["us_per_launch"] / 1e6
    return round_entry(e)


def roofline_hbm(entry, floor=None, traffic=None):
    r = {"bound": "hbm", "achieved": round(entry["GBps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(entry["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic}
    if floor is not None:
        r["achievable"] = floor["GBps"]
        r["frac_of_achievable"] = round(entry["GBps"] / floor["GBps"], 4)
        r["achievable_reference"] = floor
    return r


def roofline_mfma(entry, peak=None, dense=None):
    peak = MFMA_BF16_PEAK_TFLOPS if peak is None else peak
    r = {"bound": "mfma", "achieved": round(entry["TFLOPs"], 1), "peak": peak,
         "unit": "TFLOP/s", "frac": round(entry["TFLOPs"] / peak, 4), "traffic": None}
    if dense is not None:
        r["dense_bf16_TFLOPs"] = round(dense["TFLOPs"], 1)
        r["speedup_vs_dense_bf16"] = round(dense["us_per_launch"] / entry["us_per_launch"], 3)
    return r


CALIBRATION_COPY_BYTES = 256 << 20
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "gemv_gate_up_decode_M1_counters.md")
# the headline launch runs the balanced M = 1 GEMV (gemv_strip.hip), dispatched from gemv.hip
GEMV_SOURCES = ("w4a16_int4_weight_amd/csrc/gemv_strip.hip", "w4a16_int4_weight_amd/csrc/gemv.hip",
                "w4a16_int4_weight_amd/csrc/device_common.h")


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
    for workload, M in (("gate_up_decode", 1), ("down_proj", 1), ("down_proj", 8)):
        ws = synth.make(workload, Ms=(M,))
        packs = packed_copies(w, ws, dev)[:10]
        x = to_dev_bits(ws.x_bits[M], ws.dtype, dev)
        y = torch.empty((M, ws.N), dtype=x.dtype, device=dev)
        torch.cuda.synchronize()
        for i in range(10):
            w.w4a16_gemm(x, packs[i % len(packs)], ws.N, ws.group_size, y=y)
        torch.cuda.synchronize()
        del packs
    # the LM-head repack three times, then the MFMA GEMM on the LM-head prefill (M=512),
    # three launches on one weight copy
    ws = synth.make("lm_head", Ms=(512,))
    qw = torch.from_numpy(ws.qweight).to(dev)
    qz = torch.from_numpy(ws.qzeros).to(dev)
    sc = to_dev_bits(ws.scale_bits, ws.dtype, dev)
    packed = w.w4a16_repack(qw, qz, sc, ws.group_size)
    torch.cuda.synchronize()
    for _ in range(3):
        w.w4a16_repack(qw, qz, sc, ws.group_size, packed=packed)
    torch.cuda.synchronize()
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
    log("pmc probe done: 3 x 256 MiB copy, 10 x gate_up_decode GEMV, 10 x down_proj GEMV M=1 and M=8, "
        "1 + 3 x lm_head repack, 3 x lm_head M=512 GEMM, 3 x lm_head M=512 W4A8 GEMM")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(workload, M, budget_s=16.0):
    """The oracle as it stands (unpack, float64 dequant, float64 matmul) on whole steps
    of the workload: first on a pool of one thread per allotted core, each thread the
    oracle on its own range of output columns (whole AWQ words), then on one thread;
    BLAS held to one thread per caller throughout. About budget_s in all."""
    from concurrent.futures import ThreadPoolExecutor
    import synth
    from oracle import gemm as ogemm
    from threadpoolctl import threadpool_limits
    ws = synth.make(workload, Ms=(M,))
    J = ws.qweight.shape[1]
    threads = max(1, min(len(os.sched_getaffinity(0)), CPU_THREADS_CAP))

    def run(nthreads, seconds):
        edges = [J * i // nthreads for i in range(nthreads + 1)]

        def part(i):
            j0, j1 = edges[i], edges[i + 1]
            return ogemm.w4a16_reference(ws.x_bits[M], ws.qweight[:, j0:j1], ws.qzeros[:, j0:j1],
                                         ws.scale_bits[:, 8 * j0:8 * j1], ws.dtype, ws.group_size)

        with ThreadPoolExecutor(max_workers=nthreads) as pool:
            list(pool.map(part, range(nthreads)))          # one untimed step
            t0 = time.perf_counter()
            n = 0
            while True:
                list(pool.map(part, range(nthreads)))
                n += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            return (time.perf_counter() - t0) / n, n

    nbytes = gemm_bytes(M, ws.K, ws.N, ws.group_size)
    with threadpool_limits(limits=1):
        dt_all, n_all = run(threads, budget_s / 2)
        dt_one, n_one = run(1, budget_s / 2)
    return {"value": round(nbytes / dt_all / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_all} whole steps of {workload} M={M} ({dt_all:.3f} s each) on {threads} threads, each the "
                      f"oracle (AWQ unpack, float64 dequant, float64 matmul, BLAS 1 thread) on 1/{threads} of the "
                      f"output columns",
            "value_1_thread": round(nbytes / dt_one / 1e9, 4),
            "sample_1_thread": f"{n_one} whole steps on 1 thread ({dt_one:.3f} s each)",
            "cpu_model": cpu_model(), "host_cpus_visible": os.cpu_count()}


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

    t_start = time.perf_counter()
    T = Timer(w, dev, args.steps, args.warmup)
    head = measure_gemm(T, w, "gate_up_decode", 1, dev)
    head["kernel"] = "w4a16_gemv"
    head_floor = T.stream_floor(head["algorithmic_bytes"])
    log(f"headline gate_up_decode M=1: {head['us_per_launch']:.2f} us (p10 {head['us_p10']:.2f}, "
        f"p90 {head['us_p90']:.2f}), {head['GBps']:.0f} GB/s; same-byte stream read "
        f"{head_floor['us_per_launch']:.2f} us")
    T.settle = True
    secondary = []
    dense = []
    if not args.quick:
        for wl, M in [("lm_head", 1), ("down_proj", 1), ("down_proj", 8), ("down_proj", 16)]:
            e = measure_gemm(T, w, wl, M, dev, sustained=(wl == "lm_head"))
            e["kernel"] = "w4a16_gemv" if M <= 8 else "w4a16_gemm_mfma"
            floor = T.stream_floor(e["algorithmic_bytes"])
            e["roofline"] = roofline_hbm(e, floor)
            log(f"{wl} M={M}: {e['us_per_launch']:.2f} us, {e['GBps']:.0f} GB/s (stream read "
                f"{floor['us_per_launch']:.2f} us)" + (f"; sustained {e['sustained']['us_per_launch']:.2f} us"
                                                        if "sustained" in e else ""))
            secondary.append(e)
        for wl in ("qkv_prefill", "gate_up_prefill", "lm_head"):
            e = measure_gemm(T, w, wl, 512, dev)
            e["kernel"] = "w4a16_gemm_mfma"
            d = measure_dense_reference(T, wl, 512, dev)
            e["roofline"] = roofline_mfma(e, dense=d)
            log(f"{wl} M=512: {e['us_per_launch']:.2f} us, {e['TFLOPs']:.1f} TFLOP/s (dense bf16 "
                f"{d['us_per_launch']:.2f} us)")
            secondary.append(e)
            dense.append(d)
        for wl in ("qkv_prefill", "gate_up_prefill", "lm_head"):
            e = measure_w4a8(T, w, wl, 512, dev)
            e["roofline"] = roofline_mfma(e, MFMA_FP8_PEAK_TFLOPS)
            log(f"{wl} W4A8 M=512: {e['us_per_launch']:.2f} us, {e['TFLOPs']:.1f} TFLOP/s (with quantisation "
                f"{e['us_per_step_with_quantize']:.2f} us)")
            secondary.append(e)
        for fmt in ("awq", "gptq"):
            r = measure_repack(T, w, "lm_head", dev, fmt=fmt)
            floor = T.stream_floor(r["algorithmic_bytes"], copy=True)
            r["roofline"] = roofline_hbm(r, floor)
            log(f"lm_head repack ({fmt}): {r['us_per_launch']:.1f} us, {r['GBps']:.0f} GB/s (stream copy "
                f"{floor['us_per_launch']:.1f} us)")
            secondary.append(r)
        e = measure_embedding(T, w, "lm_head", 512, dev)
        floor = T.stream_floor(e["algorithmic_bytes"])
        e["roofline"] = roofline_hbm(e, floor)
        log(f"lm_head tied-embedding gather T=512: {e['us_per_launch']:.2f} us, {e['GBps']:.0f} GB/s")
        secondary.append(e)
        for wl, M in [("gate_up_decode", 1), ("down_proj", 1), ("lm_head", 1)]:
            d = measure_dense_reference(T, wl, M, dev)
            log(f"dense bf16 reference {wl} M={M}: {d['us_per_launch']:.2f} us, {d['GBps']:.0f} GB/s")
            dense.append(d)
    gpu_s = time.perf_counter() - t_start
    del T
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline("gate_up_decode", 1)
        log(f"cpu baseline: {cpu['value']} GB/s on {cpu['cores']} threads, {cpu['value_1_thread']} GB/s on 1")

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
                   "weight_copies": head["copies"], "copies_touched_per_replay": head["copies_touched_per_replay"],
                   "footprint_bytes_per_replay": head["footprint_bytes_per_replay"],
                   "mall_scrub_bytes": SCRUB_BYTES, "replays": head["replays"],
                   "us_per_launch_p10": head["us_p10"], "us_per_launch_p90": head["us_p90"],
                   "us_per_launch_events": head["us_per_launch_events"],
                   "timing": "HIP graph of K calls between two GPU wall-clock stamps (first and last graph "
                             "node); median over timed replays, each after a 512 MiB streaming read, "
                             "synchronised before the scrub and after the replay; us_per_launch_events: "
                             "events recorded around the replay, which add the host's graph-launch latency"},
        "roofline": roofline_hbm(head, head_floor, counter_traffic()),
        "cpu_baseline": cpu,
        "secondary": secondary,
        "dense_bf16_reference": dense,
        "measure_wall_s": round(gpu_s, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
