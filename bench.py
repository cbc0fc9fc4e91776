"""Throughput of the weight-only-quantized MoE forward on one MI355X.

A step is one whole forward (route, permute, fc1+SwiGLU, fc2, combine) over one batch of
synthetic tokens: one call of the library's qmoe_forward C entry point, which launches the
kernels (routing and grouping as one kernel at small batches) directly on one stream. The
same forwards are run again with their fc1 and fc2 kernels recording their own start and
end on HIP events (qmoe_time_next_gemm), for the kernel times and the roofline of the fc1
kernel; replayed from HIP graphs (one per weight copy, captured once), timed as
``hip_graph_ms_per_step`` (``--no-graph`` skips them); and as the stages' separate C entry
points (``staged_ms_per_step``). The default decode run adds a ``prefill`` object: the
prefill-shaped layer at T=4096 measured the same way in the same run. Inputs are resident in HBM
before the timed region. Several device copies of the expert stacks are rotated
from step to step so that the 256 MB Infinity Cache cannot serve a step's weights from
the previous step.

Default workload: the decode-shaped int4 layer (T=64, H=I=2880, E=32, k=4, 4-bit,
block 32, bf16 scales, interleaved SwiGLU with alpha 1.702, beta 1, limit 7, bf16 biases).

Prints one JSON line. ``roofline.traffic`` is the dominant kernel's HBM bytes per launch
from rocprofv3 FETCH_SIZE / WRITE_SIZE counter passes, each divided by what the same
counter reads per byte of a plain device copy (``--calibrate-copy``); it is read from the
counter summary committed under profiles/ and reported only while the kernel sources
still hash to the value recorded there, else null.

``--calibrate-copy MB`` instead runs a plain device-to-device copy of MB megabytes a few
times (the known-size kernel the counters are calibrated on) and prints its size.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import hashlib  # noqa: E402

import numpy as np  # noqa: E402

METRIC = "tokens/s per QMoE layer + weight-stream HBM GB/s (decode T<=64; prefill T=4096)"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
CPU_SECONDS = 10.0     # minimum oracle time of the cpu_baseline sample
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "weight_only_quantized_softmax_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2",
                    choices=["c1", "c2", "c3", "c4", "c5", "c2-mx", "c5-mx", "lin-decode",
                             "lin-prefill"],
                    help="c1-c5: the MoE layer workloads; c2-mx, c5-mx: the same shapes with "
                         "MX FP4 weights; lin-*: the single-expert linear layer "
                         "(qmoe_linear_woq) at two layer shapes")
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--bits", type=int, default=4)
    ap.add_argument("--block", type=int, default=32)
    ap.add_argument("--copies", type=int, default=0, help="weight copies rotated (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--int8", action="store_true",
                    help="the int8 activation tier: x and h rounded to per-block int8")
    ap.add_argument("--cpu-tokens", type=int, default=16, help="tokens per oracle call")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB")
    ap.add_argument("--tile-m", type=int, default=0,
                    help="rows per expert tile (0 = the library's choice for the shapes)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the second timing of the forward replayed from HIP graphs")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill line (T=4096 on the prefill-shaped layer) that the "
                         "default decode run adds")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--layout", default="tiles", choices=["tiles", "rows"],
                    help="weight layout handed to the GEMMs: tiled (packed once, before any "
                         "timing) or the pages' rows layout")
    return ap.parse_args()


def kernel_sources_sha(files):
    """Hash of the kernel sources' code: comments and blank space are dropped first, so that
    an edit of a comment does not retire a counter summary taken on the same code."""
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


# dominant kernel of each path: the fc1 launch, by the file that holds it
KERNEL_FILES = {"decode": ("gemm_bf16.hip", "gemm_bf16_tiled.hip", "gemm_bf16_kernel.h", "gemm_gemv_kernel.h",
                           "gemm_common.h", "common.h", "launch.h"),
                "prefill": ("gemm_prefill.hip", "gemm_prefill_rows.hip", "gemm_prefill_blk.hip", "gemm_prefill_blk_tiled.hip",
                            "gemm_prefill_blk_kernel.h", "gemm_prefill_sw.hip", "gemm_prefill_sw8.hip", "gemm_prefill_sw_kernel.h",
                            "gemm_prefill_i8.hip", "gemm_prefill_i8_kernel.h", "gemm_prefill_h16.hip",
                            "gemm_prefill_h16_kernel.h", "f16prep.hip", "gemm_common.h", "common.h", "launch.h"),
                "f32": ("gemm_f32.hip", "common.h", "launch.h")}


def committed_traffic(kind, workload):
    """HBM bytes per launch from the committed counter summary of this kernel and workload,
    or None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, f"traffic_fc1_{kind}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256") != kernel_sources_sha(KERNEL_FILES[kind]):
        return None
    try:
        return int(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy(mb, steps):
    import torch
    torch.cuda.set_device(0)
    n = mb << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps(dict(calibrate_copy_bytes=n, launches=steps)), flush=True)


class TimingEvents:
    """HIP events for kernel timing, created with hipEventDisableSystemFence: recording one
    then skips the system-scope cache writeback a default event performs, which would
    otherwise be timed as part of the kernel (a few microseconds at decode sizes). Called
    through the HIP runtime that torch has already loaded."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes
        path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line)
        self.hip = ctypes.CDLL(path)
        self.ct = ctypes
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            self._ok(self.hip.hipEventCreateWithFlags(ctypes.byref(e),
                                                      ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)))
            self.ev.append(e.value)

    def _ok(self, rc):
        if rc != 0:
            raise RuntimeError(f"HIP event call failed with error {rc}")

    def ms(self, i, j):
        out = self.ct.c_float()
        self._ok(self.hip.hipEventElapsedTime(self.ct.byref(out), self.ct.c_void_p(self.ev[i]),
                                              self.ct.c_void_p(self.ev[j])))
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(self.ct.c_void_p(e))
        self.ev = []


def workload(args):
    from synth import configs
    if args.workload in configs.LINEAR:
        cfg = configs.LINEAR[args.workload]
        return cfg, args.T if args.T is not None else max(cfg.T_points)
    if args.workload in configs.MX:
        cfg = configs.MX[args.workload]
        return cfg, args.T if args.T is not None else (64 if args.workload == "c2-mx" else 4096)
    cfg = configs.ALL[args.workload]
    if args.workload == "c5":
        cfg = configs.c5_point(args.bits, args.block)
    T = args.T if args.T is not None else (64 if args.workload == "c2" else max(cfg.T_points))
    return cfg, T


def stack_bytes(cfg, N, K, bias):
    w = N * K * cfg.bits // 8
    sb = {"bf16": 2, "f32": 4, "e8m0": 1}[cfg.scale_dtype]
    ab = 2 if cfg.act_dtype == "bf16" else 4
    s = N * (cfg.nblocks(K) if cfg.block_size else 1) * sb
    return w + s + (N * ab if bias else 0)


def algorithmic(cfg, T, counts):
    """Minimum bytes each launch must move, and the forward's flops (real rows only)."""
    ab = 2 if cfg.act_dtype == "bf16" else 4
    A = T * cfg.k
    touched = int(np.count_nonzero(counts))
    fc1_e = stack_bytes(cfg, cfg.n1, cfg.H, cfg.fc1_bias)
    if cfg.has_fc3:
        fc1_e += stack_bytes(cfg, cfg.I, cfg.H, cfg.fc1_bias)
    fc2_e = stack_bytes(cfg, cfg.H, cfg.I, cfg.fc2_bias)
    fc1 = touched * fc1_e + T * cfg.H * ab + A * cfg.I * ab
    fc2 = touched * fc2_e + A * cfg.I * ab + A * cfg.H * 4
    weights = touched * (fc1_e + fc2_e)
    flops = 2 * A * (cfg.n1 * cfg.H + (cfg.I * cfg.H if cfg.has_fc3 else 0) + cfg.I * cfg.H)
    return dict(touched=touched, fc1_bytes=fc1, fc2_bytes=fc2, weight_bytes=weights, flops=flops,
                fc1_flops=2 * A * (cfg.n1 + (cfg.I if cfg.has_fc3 else 0)) * cfg.H)


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), for the cpu_baseline record."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measure_moe(args, cfg, T, steps, warmup, cpu_leg, graph):
    """One MoE workload: the whole forward timed (one qmoe_forward per step, launched
    directly, and with graph also replayed from HIP graphs), the fc1/fc2 kernels' own
    durations from a staged pass, the
    roofline of the fc1 kernel and, with cpu_leg, the oracle on a bounded sample."""
    import torch

    import weight_only_quantized_softmax_amd as qm
    from synth import gen
    from synth.device import DeviceInputs, params_for

    print(f"[bench] {cfg.name} T={T}: generating inputs", file=sys.stderr, flush=True)
    inp = gen.make_inputs(cfg, T)
    d = DeviceInputs(inp)
    layout = args.layout if cfg.act_dtype == "bf16" else "rows"  # tiles serve bf16 activations
    p = params_for(cfg, T, tile_m=args.tile_m, layout=layout, ebias=d.ebias)
    qm.qmoe_validate(p)

    # stage buffers (the same kernels qmoe_forward launches, called one by one)
    A = T * cfg.k
    rows, tiles = qm.qmoe_max_rows(p), qm.qmoe_max_tiles(p)
    i32 = dict(dtype=torch.int32, device="cuda")
    adt = torch.bfloat16 if cfg.act_dtype == "bf16" else torch.float32
    ids = torch.empty((T, cfg.k), **i32)
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    counts = torch.empty(cfg.E, **i32)
    offs = torch.empty(cfg.E + 1, **i32)
    sa = torch.empty(rows, **i32)
    pos = torch.empty(A, **i32)
    tl = torch.empty((tiles, 2), **i32)
    nt = torch.empty(1, **i32)
    scratch = torch.empty(max(qm.qmoe_permute_scratch_size(p), 256), dtype=torch.uint8, device="cuda")
    h = torch.empty((rows, cfg.I), dtype=adt, device="cuda")
    xq = torch.empty((T, cfg.H), dtype=adt, device="cuda") if cfg.int8 else None
    y = torch.empty((rows, cfg.H), dtype=torch.float32, device="cuda")
    out = torch.empty((T, cfg.H), dtype=adt, device="cuda")
    stream = torch.cuda.current_stream()

    # the routing of this batch fixes which experts are touched; rotate enough copies of the
    # stacks that the touched bytes of the other copies exceed twice the 256 MB Infinity Cache
    qm.qmoe_route(p, d.logits, ids, w, stream)
    qm.qmoe_permute(p, ids, counts, offs, sa, pos, tl, nt, scratch, stream)
    alg = algorithmic(cfg, T, counts.cpu().numpy())
    copies = args.copies or max(2, math.ceil(2 * MALL_BYTES / max(alg["weight_bytes"], 1)) + 1)
    copies = min(copies, 64)
    if layout == "tiles":
        d = d.tiled(p)  # the one-time packing of the weights, outside every timed region
    stacks = [(d.fc1, d.fc2, d.fc3)]
    for _ in range(copies - 1):
        stacks.append(tuple(None if st is None else tuple(None if t is None else t.clone() for t in st)
                            for st in (d.fc1, d.fc2, d.fc3)))
    per_copy = sum(t.numel() * t.element_size() for st in (d.fc1, d.fc2, d.fc3) if st
                   for t in st if t is not None)

    # pre-marshalled C ABI calls, so that the host keeps ahead of the GPU at decode sizes
    lib = qm._lib.load()
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    sid = stream.cuda_stream
    st_args = [tuple(qm._stack(st, n) for st, n in zip(c, ("fc1", "fc2", "fc3"))) for c in stacks]
    ws = qm.alloc_workspace(p)
    wsn = ws.numel()
    route = (p, ptr(d.logits), ptr(ids), ptr(w), sid)
    perm = (p, ptr(ids), ptr(counts), ptr(offs), ptr(sa), ptr(pos), ptr(tl), ptr(nt),
            ptr(scratch), scratch.numel(), sid)
    comb = (p, ptr(y), ptr(pos), ptr(w), None, ptr(out), sid)

    def run(status):
        if status != 0:
            qm.check(status)

    def step(i):
        s1, s2, s3 = st_args[i % copies]
        run(lib.qmoe_route(*route))
        run(lib.qmoe_permute(*perm))
        x = d.x
        if cfg.int8:
            run(lib.qmoe_quantize_act(p, ptr(d.x), T, cfg.H, ptr(xq), sid))
            x = xq
        run(lib.qmoe_grouped_gemm_fc1_swiglu(p, ptr(x), ptr(sa), ptr(tl), ptr(nt), ptr(w), s1,
                                             s3, ptr(h), sid))
        if cfg.int8:
            run(lib.qmoe_quantize_act(p, ptr(h), rows, cfg.I, ptr(h), sid))
        run(lib.qmoe_grouped_gemm_fc2(p, ptr(h), ptr(tl), ptr(nt), s2, ptr(y), sid))
        run(lib.qmoe_combine(*comb))

    print(f"[bench] {copies} weight copies of {per_copy / 1e6:.1f} MB "
          f"({alg['weight_bytes'] / 1e6:.1f} MB touched); warmup {warmup}",
          file=sys.stderr, flush=True)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    staged_ms = (t1 - t0) * 1e3 / steps

    # the timed step: the whole-forward entry point (one C call per step, the same kernels
    # with routing and grouping in one launch at small batches); with graph, each weight
    # copy's forward is also captured once into a HIP graph and timed as graph replays
    xp, lp, op = ptr(d.x), ptr(d.logits), ptr(out)

    def fwd(i, s):
        s1, s2, s3 = st_args[i % copies]
        run(lib.qmoe_forward(p, xp, lp, s1, s2, s3, None, op, ptr(ws), wsn, s))

    def timed(launch):
        for i in range(warmup):
            launch(i)
        torch.cuda.synchronize()
        f0 = time.perf_counter()
        for i in range(steps):
            launch(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - f0) * 1e3 / steps

    ms_per_step = timed(lambda i: fwd(i, sid))

    # the kernels' own durations: the same forwards, the fc1 and fc2 launches each recording
    # their start and end on HIP events (qmoe_time_next_gemm armed twice per forward:
    # hipExtLaunchKernel events)
    tev = TimingEvents(4 * steps)
    for i in range(steps):
        run(lib.qmoe_time_next_gemm(tev.ev[4 * i], tev.ev[4 * i + 1]))
        run(lib.qmoe_time_next_gemm(tev.ev[4 * i + 2], tev.ev[4 * i + 3]))
        fwd(i, sid)
    torch.cuda.synchronize()
    fc1_ms = float(np.mean([tev.ms(4 * i, 4 * i + 1) for i in range(steps)]))
    fc2_ms = float(np.mean([tev.ms(4 * i + 2, 4 * i + 3) for i in range(steps)]))
    tev.close()
    graph_ms = None
    if graph:
        cap = torch.cuda.Stream()
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                fwd(c, torch.cuda.current_stream().cuda_stream)
            graphs.append(g)
        torch.cuda.synchronize()
        graph_ms = timed(lambda i: graphs[i % copies].replay())

    fc1_gbps = alg["fc1_bytes"] / (fc1_ms * 1e-3) / 1e9
    stream_gbps = alg["weight_bytes"] / ((fc1_ms + fc2_ms) * 1e-3) / 1e9
    kind = "f32" if cfg.act_dtype == "f32" else ("prefill" if qm.qmoe_tile_m(p) == 128 else "decode")
    traffic = committed_traffic(kind, f"{cfg.name}_T{T}")
    if T <= 64 or alg["flops"] / alg["weight_bytes"] < 300:
        roof = dict(bound="hbm", achieved=round(fc1_gbps, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(fc1_gbps / HBM_PEAK_GBPS, 4), traffic=traffic)
    else:
        tf = alg["fc1_flops"] / (fc1_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(tf, 2), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(tf / BF16_PEAK_TFLOPS, 4), traffic=traffic)
    fc2_flops = alg["flops"] - alg["fc1_flops"]
    kernels = dict(fc1_ms=round(fc1_ms, 5), fc2_ms=round(fc2_ms, 5),
                   fc1_hbm_frac=round(fc1_gbps / HBM_PEAK_GBPS, 4),
                   fc2_hbm_frac=round(alg["fc2_bytes"] / (fc2_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                   fc1_mfma_frac=round(alg["fc1_flops"] / (fc1_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                   fc2_mfma_frac=round(fc2_flops / (fc2_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4))

    cpu = None
    if cpu_leg:
        import oracle
        threads = min(16, os.cpu_count() or 1)
        chunk = min(T, args.cpu_tokens)
        print(f"[bench] cpu oracle, {chunk}-token calls, {threads} threads, >= {CPU_SECONDS:.0f} s",
              file=sys.stderr, flush=True)
        done, calls, start = 0, 0, 0
        c0 = time.perf_counter()
        while time.perf_counter() - c0 < CPU_SECONDS:
            sel = (start + np.arange(chunk)) % T
            oracle.forward(cfg, inp, sel=sel, nthreads=threads)
            done += chunk
            calls += 1
            start = (start + chunk) % T
        csec = time.perf_counter() - c0
        cpu = dict(value=round(done / csec, 3), unit="tokens/s", cores=threads, kind="oracle",
                   cpu_model=cpu_model(),
                   sample=f"{calls} fp64 oracle forwards of {chunk} consecutive tokens of the same "
                          f"T={T} workload (cycling through its tokens), {done} tokens in {csec:.1f} s "
                          f"on {threads} threads of the host CPU ({cpu_model()})")
    return dict(cfg=cfg, T=T, p=p, layout=layout, copies=copies, alg=alg, ms_per_step=ms_per_step,
                staged_ms=staged_ms, fc1_ms=fc1_ms, fc2_ms=fc2_ms, roof=roof, cpu=cpu,
                stream_gbps=stream_gbps, kernels=kernels, graph_ms=graph_ms)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the forward runs on a single MI355X, and no "
              "multi-GPU (sharded) run is launched by this script.",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, max(args.steps, 1))
        return

    import torch

    import weight_only_quantized_softmax_amd as qm
    from synth import configs

    cfg, T = workload(args)
    torch.cuda.set_device(0)
    if cfg.E == 1 and cfg.k == 1:
        if args.int8:
            sys.exit("--int8 applies to the MoE forward")
        return main_linear(args, cfg, T)
    if args.int8:
        cfg = cfg.with_(int8=True, name=f"{cfg.name}-a8")
    graph = not args.no_graph
    r = measure_moe(args, cfg, T, args.steps, args.warmup, not args.no_cpu_baseline, graph)
    alg = r["alg"]
    value = T / (r["ms_per_step"] * 1e-3)
    line = dict(
        metric=METRIC, value=round(value, 1), unit="tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(r["ms_per_step"], 5), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="bf16" if cfg.act_dtype == "bf16" else "f32",
        data="synthetic",
        config=dict(workload=f"{cfg.name} T={T}", T=T, H=cfg.H, I=cfg.I, E=cfg.E, k=cfg.k,
                    bits=cfg.bits, block_size=cfg.block_size, swiglu_fusion=cfg.fusion,
                    weight_layout=r["layout"], tile_m=qm.qmoe_tile_m(r["p"]),
                    weight_copies=r["copies"], touched_experts=alg["touched"],
                    activations="int8 blocks" if cfg.int8 else cfg.act_dtype),
        roofline=r["roof"],
        cpu_baseline=r["cpu"],
        weight_stream_GBps=round(r["stream_gbps"], 1),
        kernel_ms=dict(fc1=round(r["fc1_ms"], 5), fc2=round(r["fc2_ms"], 5)),
        kernels=r["kernels"],
        staged_ms_per_step=round(r["staged_ms"], 5),
        hip_graph_ms_per_step=None if r["graph_ms"] is None else round(r["graph_ms"], 5),
        algorithmic=dict(fc1_bytes=alg["fc1_bytes"], fc2_bytes=alg["fc2_bytes"],
                         weight_bytes=alg["weight_bytes"], flops=alg["flops"]),
    )
    # the prefill half of the metric (T = 4096 on the prefill-shaped layer), in the same run
    if args.workload == "c2" and not args.no_prefill:
        q = measure_moe(args, configs.C3, 4096, args.prefill_steps, 3, False, False)
        line["prefill"] = dict(
            workload=f"{configs.C3.name} T=4096", tokens_per_s=round(4096 / (q["ms_per_step"] * 1e-3), 1),
            ms_per_step=round(q["ms_per_step"], 5), steps=args.prefill_steps, warmup=3,
            kernel_ms=dict(fc1=round(q["fc1_ms"], 5), fc2=round(q["fc2_ms"], 5)),
            roofline=q["roof"], kernels=q["kernels"],
            tile_m=qm.qmoe_tile_m(q["p"]), weight_copies=q["copies"])
    print(json.dumps(line), flush=True)


def main_linear(args, cfg, T):
    """The single-expert linear layer: one qmoe_linear_woq call per step."""
    import torch

    import weight_only_quantized_softmax_amd as qm
    from synth import gen
    from synth.device import dev

    print(f"[bench] {cfg.name} T={T}: generating inputs", file=sys.stderr, flush=True)
    inp = gen.make_linear_inputs(cfg, T)
    layout = args.layout if cfg.act_dtype == "bf16" else "rows"
    p = qm.linear_params(T, cfg.H, cfg.I, expert_weight_bits=cfg.bits, block_size=cfg.block_size,
                         activation=cfg.activation, act_dtype=cfg.act_dtype,
                         scale_dtype=cfg.scale_dtype, tile_m=args.tile_m, weight_layout=layout)
    qm.qmoe_validate(p)
    x = dev(inp.x, cfg.act_dtype)
    w = dev(inp.w1)
    if layout == "tiles":
        w = qm.pack_stack(p, "fc1", w)  # the one-time packing, outside every timed region
    st = (w, dev(inp.s1, cfg.scale_dtype), dev(inp.b1, cfg.act_dtype) if inp.b1 is not None else None)
    wbytes = stack_bytes(cfg, cfg.I, cfg.H, cfg.fc1_bias)
    copies = args.copies or max(2, math.ceil(2 * MALL_BYTES / wbytes) + 1)
    copies = min(copies, 64)
    stacks = [st] + [tuple(None if t is None else t.clone() for t in st) for _ in range(copies - 1)]
    y = torch.empty((T, cfg.I), dtype=x.dtype, device="cuda")
    stream = torch.cuda.Stream()
    lib = qm._lib.load()
    sargs = [qm._stack(c, "weight") for c in stacks]
    sid = stream.cuda_stream
    xp, yp = x.data_ptr(), y.data_ptr()
    torch.cuda.synchronize()

    def run(status):
        if status != 0:
            qm.check(status)

    tev = TimingEvents(2 * args.steps)
    print(f"[bench] {copies} weight copies of {wbytes / 1e6:.1f} MB; warmup {args.warmup}",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        run(lib.qmoe_linear_woq(p, xp, sargs[i % copies], yp, sid))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(lib.qmoe_linear_woq(p, xp, sargs[i % copies], yp, sid))
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # the kernel's own duration: the same launches, each recording its start and end
    for i in range(args.steps):
        run(lib.qmoe_time_next_gemm(tev.ev[2 * i], tev.ev[2 * i + 1]))
        run(lib.qmoe_linear_woq(p, xp, sargs[i % copies], yp, sid))
    torch.cuda.synchronize()
    k_ms = float(np.mean([tev.ms(2 * i, 2 * i + 1) for i in range(args.steps)]))
    tev.close()

    ab = 2 if cfg.act_dtype == "bf16" else 4
    bytes_ = wbytes + T * cfg.H * ab + T * cfg.I * ab
    flops = 2 * T * cfg.I * cfg.H
    if flops / wbytes < 300:
        gbps = bytes_ / (k_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(gbps, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(gbps / HBM_PEAK_GBPS, 4), traffic=None)
    else:
        tf = flops / (k_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(tf, 2), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(tf / BF16_PEAK_TFLOPS, 4), traffic=None)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        threads = min(16, os.cpu_count() or 1)
        chunk = min(T, args.cpu_tokens)
        done, calls, start = 0, 0, 0
        c0 = time.perf_counter()
        while time.perf_counter() - c0 < CPU_SECONDS:
            oracle.linear(cfg, inp, rows=(start + np.arange(chunk)) % T, nthreads=threads)
            done += chunk
            calls += 1
            start = (start + chunk) % T
        csec = time.perf_counter() - c0
        cpu = dict(value=round(done / csec, 3), unit="tokens/s", cores=threads, kind="oracle",
                   sample=f"{calls} fp64 oracle evaluations of {chunk} rows of the same T={T} "
                          f"layer, {done} rows in {csec:.1f} s")
    line = dict(
        metric="tokens/s per QLinearWoQ layer + weight-stream HBM GB/s", value=round(T / (ms_per_step * 1e-3), 1),
        unit="tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms_per_step, 5), higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16" if cfg.act_dtype == "bf16" else "f32", data="synthetic",
        config=dict(workload=f"{cfg.name} T={T}", T=T, in_features=cfg.H, out_features=cfg.I,
                    bits=cfg.bits, block_size=cfg.block_size, activation=cfg.activation,
                    weight_layout=layout, tile_m=qm.qmoe_tile_m(p), weight_copies=copies),
        roofline=roof, cpu_baseline=cpu, kernel_ms=dict(linear=round(k_ms, 5)),
        algorithmic=dict(bytes=bytes_, weight_bytes=wbytes, flops=flops),
    )
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
