#!/usr/bin/env python3
"""Benchmark of the MoE expert-parallel dispatch/combine path on one MI355X.

One step = layout -> notify -> dispatch -> combine over one batch, on the
workload the headline metric is quoted on: bs = 4096 tokens, hidden = 7168,
top-8 of 256 experts over 16 logical ranks, bf16 rows, dynamic int8 dispatch,
bf16 combine output (a DeepSeek-V3-style MoE layer, synthetic seeded data).

Timing: W untimed warm-up steps, then K timed steps.  Before each step and
between dispatch and combine a read-only pass over a 1 GiB buffer evicts the
L2s and the 256 MB Infinity Cache, so x is read from HBM by dispatch and the
receive buffer from HBM by combine (between the two, a real MoE layer runs its
expert GEMMs).  HIP events recorded on the stream the kernels run on (created without the
system-scope fence, which only serves host visibility) time each stage;
flushes are outside the timed intervals.  ``ms_per_step`` is the mean
of layout+notify+dispatch+combine over the K steps and ``value`` is bs divided
by it (tokens/s, whole pipeline).  Reported beside it, labelled:
``steady_state``, the back-to-back step replayed from one captured HIP graph
with nothing flushed (every write's cost inside the timed region, with the
caches as a running pipeline leaves them); ``write_back_inclusive``, dispatch
plus the flush after it minus the same flush on clean caches (dispatch's rows
partly stay in the 256 MB Infinity Cache when the kernel ends and are written
back during the next flush); per-stage GB/s beside a plain device copy;
the dispatch and combine kernels timed on their own
(``dispatch_combine_kernels_alone``: without the layout work the fused launch
carries); and the CPU oracle.

``--stage epilogue`` times the expert-side epilogue kernel (dequantise the
first expert GEMM's int32 output, SwiGLU, requantise to int8 rows) alone, on
every receive row of the large shape with an FFN width of 2048, and prints
its own JSON line (rows/s).  ``--stage gemm`` times the first expert matmul
(int8 receive rows x int8 expert weights -> int32, grouped by expert) on one
GPU's share of the large shape on a 16-rank expert-parallel group (32768
rows, 16 experts, k = 7168, 2 x 2048 output columns) and prints its own line
(rows/s, with int8 TOP/s against the MFMA peak).  ``--stage gemm_swiglu``
times the same matmul with its epilogue fused (int8 rows in, int8 rows of
width 2048 out), beside the two separate calls in the same run.

Output: one JSON line on stdout.  ``--gpus N`` with N > 1 exits: the bench
measures one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, 8 TB/s
GRAPH_STEPS = 10  # steps captured into one HIP graph for the graph-replay figure
METRIC = "dispatch+combine tokens/s and HBM GB/s (% of peak) at bs=4096 h=7168 top-8"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "combine_moe_layout_03_amd", "csrc")
# A kernel's source: its own file and the headers every kernel file includes.
KERNEL_HEADERS = [os.path.join(CSRC, f) for f in ("device_util.h", "launch.h", "quant.h", "select.h")]
KERNEL_SOURCES = {
    "dispatch": [os.path.join(CSRC, "dispatch.hip")] + KERNEL_HEADERS,
    "combine": [os.path.join(CSRC, "combine.hip")] + KERNEL_HEADERS,
    "fused": [os.path.join(CSRC, "fused.hip")] + KERNEL_HEADERS,
    "epilogue": [os.path.join(CSRC, "epilogue.hip"), os.path.join(CSRC, "swiglu.h")] + KERNEL_HEADERS,
    "gemm": [os.path.join(CSRC, "gemm.hip"), os.path.join(CSRC, "gemm.h"), os.path.join(CSRC, "swiglu.h")]
    + KERNEL_HEADERS,
}
KERNEL_SOURCES["gemm_swiglu"] = KERNEL_SOURCES["gemm"]
EPILOGUE_METRIC = "expert epilogue (dequant + SwiGLU + int8 requant) rows/s and HBM GB/s (% of peak)"
GEMM_METRIC = "first expert matmul (int8 x int8 -> int32, grouped by expert) rows/s and TOP/s (% of peak)"
GEMM_SWIGLU_METRIC = ("first expert matmul with its dequant + SwiGLU + int8 requant epilogue fused, rows/s and "
                      "TOP/s (% of peak)")
MFMA_I8_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA, 5.0 POP/s


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """Raw HIP events (ctypes on the HIP runtime torch already loaded),
    recorded on the stream the library's kernels run on.  By default they are
    created with hipEventDisableSystemFence: the system-scope fence only
    matters for host visibility of memory and adds dispatch latency to every
    timed interval."""

    FLAGS = {"nofence": 0x20000000, "default": 0x0}

    def __init__(self, flags: str = "nofence"):
        import ctypes

        self.ct = ctypes
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.flags = self.FLAGS[flags]
        self.events = []

    def new(self):
        ev = self.ct.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(self.ct.byref(ev), self.flags)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        self.events.append(ev)
        return ev

    def record(self, ev, stream) -> None:
        rc = self.lib.hipEventRecord(ev, self.ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def ms(self, a, b) -> float:
        out = self.ct.c_float(0.0)
        rc = self.lib.hipEventElapsedTime(self.ct.byref(out), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return out.value

    def close(self) -> None:
        for ev in self.events:
            self.lib.hipEventDestroy(ev)
        self.events = []


def algorithmic_bytes(bs: int, h: int, k: int, quant: bool, out_bytes: int = 2):
    """Bytes each stage must move (indices int32, weights fp32):
    dispatch reads x and (topkIdx, sendTokenIdx) and writes k rows per token;
    combine reads k rows plus (topkIdx, sendTokenIdx, weight) and writes out."""
    row = (h + 4) if quant else 2 * h  # int8 codes + one fp32 inverse scale, or the row
    dispatch = bs * 2 * h + bs * k * row + bs * k * 8
    combine = bs * k * row + bs * k * 12 + bs * h * out_bytes
    layout = bs * k * 8
    return dispatch, combine, layout


def epilogue_bytes(rows: int, n: int) -> int:
    """Bytes the epilogue must move: each row reads 2n int32 accumulators and
    its float token scale and writes n int8 codes and a float inverse scale;
    the 2n float weight scales are read once per launch."""
    return rows * (8 * n + 4 + n + 4) + 8 * n


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pct(values, q):
    v = sorted(values)
    if not v:
        return None
    i = min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))
    return v[i]


def load_traffic(kernel: str, workload: str, mode: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}_{mode}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return t.get("traffic_bytes_per_launch")


def gemm_ops(rows: int, n: int, k: int) -> int:
    """Multiplies and adds of the first expert matmul over `rows` owned rows."""
    return 2 * rows * n * k


def gemm_bytes(rows: int, n: int, k: int, groups: int) -> int:
    """Bytes the first expert matmul must move at least once: the k codes of
    every row, every expert's weights, the int32 output and the counts."""
    return rows * k + groups * n * k + rows * n * 4 + groups * 4


def host_cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), else what platform reports."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, quant: bool, budget_s: float):
    """The oracle as it stands, single-threaded on a host core, over the full
    workload, repeated until about ``budget_s`` seconds have passed."""
    import oracle

    oracle.default()
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.pipeline(w.x, w.x_dtype, w.topk_idx, w.topk_w, w.expert_num_per_rank, w.rank_size,
                        quant, w.x_dtype)
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s or passes >= 50:
            break
    return dict(value=w.bs * passes / el, unit="tokens/s", cores=1, kind="oracle",
                sample=f"full {w.name} workload ({w.bs} tokens, all four stages), {passes} pass(es) "
                       f"in {el:.1f} s on one host thread",
                host_cpu=host_cpu_model(), host_nproc=os.cpu_count())


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large", choices=["tiny", "small", "mid", "large", "stress"])
    ap.add_argument("--mode", default="int8", choices=["int8", "pass"])
    ap.add_argument("--x-dtype", default="bf16", choices=["bf16", "fp16"],
                    help="element type of x (and of the combine output)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work (0: skip)")
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--event-flags", default="nofence", choices=["nofence", "default"],
                    help="HIP event creation flags for the stage timers")
    ap.add_argument("--path", default="fused", choices=["separate", "fused"],
                    help="layout, notify and dispatch as three launches, or one fused launch")
    ap.add_argument("--sources", type=int, default=1,
                    help="split the workload's tokens into this many source ranks sharing one receive "
                         "buffer (multi-source notify, per-source dispatch and combine)")
    ap.add_argument("--skip-kernels-only", action="store_true",
                    help="with the fused path, do not also time the dispatch and combine kernels alone")
    ap.add_argument("--stage", default="pipeline", choices=["pipeline", "epilogue", "gemm", "gemm_swiglu"],
                    help="pipeline: layout + notify + dispatch + combine (the headline); epilogue: the "
                         "expert-side dequant + SwiGLU + int8 requant kernel on its own; gemm: the first "
                         "expert matmul on its own; gemm_swiglu: the matmul with that epilogue fused")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, then WRITE_SIZE) of a bench "
                         "run into profiles/traffic_*.json and exit")
    ap.add_argument("--counters", choices=["flushed", "unflushed"],
                    help="a short run for rocprofv3 --pmc: W + K steps of the fused path, then K steps of the "
                         "separate stages, flushed before each stage or back to back, then the 1 GiB copy "
                         "kernel the counters are calibrated on; prints what it ran and exits")
    ap.add_argument("--ingest-dram", nargs=2, metavar=("FLUSHED_CSV", "UNFLUSHED_CSV"),
                    help="turn the DRAM request counters of two --counters runs (flushed, unflushed) into "
                         "profiles/dram_requests_<workload>_<mode>.json and exit")
    args = ap.parse_args(argv)

    if args.ingest_pmc:
        return ingest_pmc(args, *args.ingest_pmc)
    if args.ingest_dram:
        return ingest_dram(args, *args.ingest_dram)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the expert-parallel ranks are logical partitions of one "
              "device's receive buffer; this bench does not launch multi-GPU runs.", file=sys.stderr)
        return 2

    import torch
    import workloads as W
    import combine_moe_layout_03_amd as M

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.stage == "epilogue":
        return bench_epilogue(args, M, torch, W, dev)
    if args.stage == "gemm":
        return bench_gemm(args, M, torch, W, dev)
    if args.stage == "gemm_swiglu":
        return bench_gemm_swiglu(args, M, torch, W, dev)
    quant = args.mode == "int8"

    log(f"generating workload {args.workload}")
    w = W.make_workload(args.workload, args.x_dtype)
    xt = torch.float16 if args.x_dtype == "fp16" else torch.bfloat16
    x = torch.from_numpy(w.x.view("int16")).to(dev).view(xt)
    idx = torch.from_numpy(w.topk_idx).to(dev)
    wts = torch.from_numpy(w.topk_w).to(dev)
    buf = M.EpBuffers(w.bs, w.hidden, w.topk, w.expert_num_per_rank, w.rank_size,
                      x_dtype=xt, quant_int8=quant, out_dtype=xt)
    flush = torch.ones(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    flush_out = torch.zeros((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def do_flush():
        torch.sum(flush, dim=0, out=flush_out)

    if args.sources > 1:
        del buf
        return bench_sources(args, M, torch, w, x, idx, wts, quant, do_flush, stream)
    if args.counters:
        return counter_run(args, torch, w, buf, x, idx, wts, flush, do_flush)

    fused = args.path == "fused"
    if fused and not M.moe_fused_supported(w.bs, w.hidden, w.topk, w.expert_num_per_rank, w.rank_size,
                                           xt, quant):
        log("the fused kernel does not apply to this shape; the fused entry point runs the three stages")

    def first_stages():
        if fused:
            buf.layout_notify_dispatch(x, idx)
        else:
            buf.layout(idx)
            buf.notify()
            buf.dispatch(x, idx)

    # warm-up (also the first touch of every buffer)
    log(f"warm-up x{args.warmup}")
    for _ in range(args.warmup):
        do_flush()
        buf.run(x, idx, wts, fused=fused)
    torch.cuda.synchronize()

    # timed steps
    log(f"timed x{args.steps}")
    hev = HipEvents(args.event_flags)
    ev = [[hev.new() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for i in range(args.steps):
        e = ev[i]
        do_flush()
        if fused:
            # one launch for layout + notify + dispatch: timed as one interval
            # (e[0] unused: two events with nothing between them still read
            # a few microseconds apart)
            hev.record(e[1], stream)
            first_stages()
            hev.record(e[2], stream)
        else:
            hev.record(e[0], stream)
            buf.layout(idx)
            buf.notify()
            hev.record(e[1], stream)
            buf.dispatch(x, idx)
            hev.record(e[2], stream)
        do_flush()
        hev.record(e[3], stream)
        buf.combine(idx, wts)
        hev.record(e[4], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    lay_ms = [0.0 if fused else hev.ms(e[0], e[1]) for e in ev]
    dis_ms = [hev.ms(e[1], e[2]) for e in ev]
    com_ms = [hev.ms(e[3], e[4]) for e in ev]
    # the dispatch launch plus the flush after it: the flush also writes back
    # whatever dispatch left dirty in the caches
    dis_flush_ms = [hev.ms(e[1], e[3]) for e in ev]
    step_ms = [a + b + c for a, b, c in zip(lay_ms, dis_ms, com_ms)]
    ms_per_step = sum(step_ms) / len(step_ms)

    # the same flush on caches holding only clean lines (a flush after a
    # flush): subtracted from the above, it leaves dispatch with its
    # write-back
    log(f"flush on clean caches x{args.steps}")
    fev = [(hev.new(), hev.new()) for _ in range(args.steps)]
    for f0, f1 in fev:
        do_flush()
        hev.record(f0, stream)
        do_flush()
        hev.record(f1, stream)
    torch.cuda.synchronize()
    flush_clean_ms = [hev.ms(f0, f1) for f0, f1 in fev]

    # un-flushed back-to-back pipeline (labelled; combine may hit the Infinity Cache)
    log("un-flushed back-to-back")
    e0, e1 = hev.new(), hev.new()
    hev.record(e0, stream)
    for _ in range(args.steps):
        buf.run(x, idx, wts, fused=fused)
    hev.record(e1, stream)
    torch.cuda.synchronize()
    unflushed_ms = hev.ms(e0, e1) / args.steps

    # the same back-to-back steps replayed from one captured HIP graph of
    # GRAPH_STEPS steps (the library only enqueues kernels, so steps
    # capture); this removes the host launch overhead that dominates the
    # small workloads (one graph launch itself costs tens of microseconds
    # here, hence several steps per graph)
    log("graph replay, un-flushed back-to-back")
    graph_ms = None
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(GRAPH_STEPS):
                buf.run(x, idx, wts, fused=fused)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // GRAPH_STEPS)
        g0, g1 = hev.new(), hev.new()
        hev.record(g0, stream)
        for _ in range(reps):
            graph.replay()
        hev.record(g1, stream)
        torch.cuda.synchronize()
        graph_ms = hev.ms(g0, g1) / (reps * GRAPH_STEPS)
        del graph
    except RuntimeError as exc:  # an auxiliary figure: report it as missing, say why
        log(f"graph capture failed, graph_unflushed_ms_per_step is null: {exc}")

    # with the fused path, the dispatch and combine kernels on their own as
    # well (the layout and notify outputs are in place from the steps
    # above), each after a flush: dispatch + combine without the layout work
    # that the fused launch carries
    kernels_only = None
    if fused and not args.skip_kernels_only:
        log(f"dispatch and combine kernels alone x{args.steps}")
        for _ in range(max(1, args.warmup)):  # the first launch of a kernel also loads it
            do_flush()
            buf.dispatch(x, idx)
            buf.combine(idx, wts)
        torch.cuda.synchronize()
        kev = [[hev.new() for _ in range(4)] for _ in range(args.steps)]
        for e in kev:
            do_flush()
            hev.record(e[0], stream)
            buf.dispatch(x, idx)
            hev.record(e[1], stream)
            do_flush()
            hev.record(e[2], stream)
            buf.combine(idx, wts)
            hev.record(e[3], stream)
        torch.cuda.synchronize()
        kd = statistics.mean(hev.ms(e[0], e[1]) for e in kev) * 1e3
        kc = statistics.mean(hev.ms(e[2], e[3]) for e in kev) * 1e3
        bd, bc, _ = algorithmic_bytes(w.bs, w.hidden, w.topk, quant)
        gbps = (bd + bc) / ((kd + kc) * 1e-6) / 1e9
        kernels_only = {"dispatch_us": kd, "combine_us": kc, "tokens_per_s": w.bs / ((kd + kc) * 1e-6),
                        "hbm_gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS}

    # plain device copy of 1 GiB (read + write) as the practical ceiling
    log("copy ceiling")
    src = flush
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)
    c0, c1 = hev.new(), hev.new()
    reps = 10
    hev.record(c0, stream)
    for _ in range(reps):
        torch.neg(src, out=dst)
    hev.record(c1, stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 4 * reps / (hev.ms(c0, c1) * 1e-3) / 1e9
    del dst
    hev.close()

    b_dis, b_com, b_lay = algorithmic_bytes(w.bs, w.hidden, w.topk, quant)
    dis_mean = statistics.mean(dis_ms)
    com_mean = statistics.mean(com_ms)
    # the launch that carries the dispatch: the dispatch kernel, or the fused
    # kernel, which reads the ids once from HBM (dispatch's own index read;
    # its other workgroups' reads of them hit L2) and writes the slots (in
    # place of dispatch's slot read), so its bytes are dispatch's
    first = "fused" if fused else "dispatch"
    b_first = b_dis
    dom = first if dis_mean >= com_mean else "combine"
    dom_ms = dis_mean if dom == first else com_mean
    dom_bytes = b_first if dom == first else b_com
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    mode_tag = "int8" if quant else "pass"
    traffic = load_traffic(dom, args.workload, mode_tag)
    dc_gbps = (b_dis + b_com) / ((dis_mean + com_mean) * 1e-3) / 1e9
    if fused:
        stages = (("layout+notify+dispatch", dis_ms), ("combine", com_ms))
    else:
        stages = (("layout+notify", lay_ms), ("dispatch", dis_ms), ("combine", com_ms))

    # write-back-inclusive dispatch, and the steady state (graph replay of
    # back-to-back steps, nothing flushed): the whole step with every write's
    # cost paid inside the timed region
    dis_wb_mean = statistics.mean(dis_flush_ms) - statistics.mean(flush_clean_ms)
    gb = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    write_back = {
        "dispatch_us": dis_wb_mean * 1e3,
        "dispatch_plus_flush_us": statistics.mean(dis_flush_ms) * 1e3,
        "flush_on_clean_caches_us": statistics.mean(flush_clean_ms) * 1e3,
        "dispatch_combine_us": (dis_wb_mean + com_mean) * 1e3,
        "dispatch_combine_tokens_per_s": w.bs / ((dis_wb_mean + com_mean) * 1e-3),
        "dispatch_combine_hbm_frac": gb(b_dis + b_com, dis_wb_mean + com_mean) / HBM_PEAK_GBPS,
        "how": "dispatch launch + the 1 GiB read-flush after it, minus the same flush on clean caches",
    }
    steady = None
    if graph_ms is not None:
        steady = {
            "ms_per_step": graph_ms,
            "tokens_per_s": w.bs / (graph_ms * 1e-3),
            "hbm_gbps": gb(b_dis + b_com, graph_ms),
            "hbm_frac": gb(b_dis + b_com, graph_ms) / HBM_PEAK_GBPS,
            "eager_ms_per_step": unflushed_ms,
            "how": f"{GRAPH_STEPS} back-to-back steps (layout + notify + dispatch + combine) captured in one "
                   "HIP graph and replayed, nothing flushed; bytes are the step's algorithmic bytes",
        }
    stage_gbps = {
        "dispatch_flushed": gb(b_first, dis_mean),
        "dispatch_write_back_inclusive": gb(b_first, dis_wb_mean),
        "combine_flushed": gb(b_com, com_mean),
        "copy_ceiling": copy_gbps,
    }

    cpu = None
    if args.cpu_budget > 0:
        log(f"cpu baseline (oracle, ~{args.cpu_budget:.0f} s)")
        cpu = cpu_baseline(w, quant, args.cpu_budget)

    line = {
        "metric": METRIC,
        "value": w.bs / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "payload": (f"{args.x_dtype} rows in, int8 codes + fp32 inverse scale per row on the wire, "
                    f"{args.x_dtype} out" if quant
                    else f"{args.x_dtype} rows in and on the wire, {args.x_dtype} out"),
        "data": "synthetic",
        "config": {"workload": args.workload, "bs": w.bs, "hidden": w.hidden, "topk": w.topk,
                   "num_experts": w.num_experts, "rank_size": w.rank_size, "x_dtype": args.x_dtype,
                   "dispatch": "int8" if quant else "passthrough", "out_dtype": args.x_dtype,
                   "parallelism": "1 GPU, ranks are logical partitions of one receive buffer"},
        "step": "layout + notify + dispatch + combine, caches flushed before the step and before combine",
        "path": ("layout+notify+dispatch fused in one launch, then combine" if fused
                 else "four launches: layout, notify, dispatch, combine"),
        "timer": f"HIP events on the kernels' stream ({args.event_flags})",
        "dispatch_combine_tokens_per_s": w.bs / ((dis_mean + com_mean) * 1e-3),
        "dispatch_combine_hbm_gbps": dc_gbps,
        "dispatch_combine_hbm_frac": dc_gbps / HBM_PEAK_GBPS,
        "stages_us": {
            name: {"mean": statistics.mean(v) * 1e3, "p10": pct(v, 0.1) * 1e3,
                   "p50": pct(v, 0.5) * 1e3, "p90": pct(v, 0.9) * 1e3}
            for name, v in stages
        },
        "algorithmic_bytes": ({"fused": b_first, "combine": b_com} if fused else
                              {"dispatch": b_dis, "combine": b_com, "layout": b_lay}),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic},
        "unflushed_ms_per_step": unflushed_ms,
        "unflushed_tokens_per_s": w.bs / (unflushed_ms * 1e-3),
        "graph_unflushed_ms_per_step": graph_ms,
        "steady_state": steady,
        "write_back_inclusive": write_back,
        "stage_gbps": stage_gbps,
        "dispatch_combine_kernels_alone": kernels_only,
        "copy_ceiling_gbps": copy_gbps,
        "wall_ms_per_step_incl_flush": wall / args.steps * 1e3,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_epilogue(args, M, torch, W, dev) -> int:
    """The expert-side epilogue kernel alone on every receive row of the large
    shape (4096 tokens x top-8 = 32768 rows) with an FFN width of n = 2048:
    int32 [rows, 2n] in, int8 rows out.  The caches are flushed before each
    timed launch."""
    c = W.EPILOGUE_CONFIG
    log(f"generating epilogue inputs rows={c['rows']} n={c['n']}")
    case = W.epilogue_case(c["seed"], c["rows"], c["n"])
    acc = torch.from_numpy(case.acc).to(dev)
    ws = torch.from_numpy(case.weight_scale).to(dev)
    ts = torch.from_numpy(case.token_scale).to(dev)
    rb = M.moe_recv_row_bytes(case.n, M.MOE_INT8_ROWSCALE)
    out = torch.zeros(case.rows * rb, dtype=torch.uint8, device=dev)
    flush = torch.ones(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    flush_out = torch.zeros((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    log(f"warm-up x{args.warmup}")
    for _ in range(args.warmup):
        torch.sum(flush, dim=0, out=flush_out)
        M.moe_deq_swiglu_quant(acc, ws, ts, out)
    torch.cuda.synchronize()
    log(f"timed x{args.steps}")
    hev = HipEvents(args.event_flags)
    ev = [(hev.new(), hev.new()) for _ in range(args.steps)]
    for e0, e1 in ev:
        torch.sum(flush, dim=0, out=flush_out)
        hev.record(e0, stream)
        M.moe_deq_swiglu_quant(acc, ws, ts, out)
        hev.record(e1, stream)
    torch.cuda.synchronize()
    us = [hev.ms(e0, e1) * 1e3 for e0, e1 in ev]
    log("copy ceiling")
    dst = torch.empty_like(flush)
    for _ in range(2):
        torch.neg(flush, out=dst)
    c0, c1 = hev.new(), hev.new()
    hev.record(c0, stream)
    for _ in range(10):
        torch.neg(flush, out=dst)
    hev.record(c1, stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * flush.numel() * 4 * 10 / (hev.ms(c0, c1) * 1e-3) / 1e9
    del dst
    hev.close()
    mean_us = statistics.mean(us)
    alg = epilogue_bytes(case.rows, case.n)
    achieved = alg / (mean_us * 1e-6) / 1e9
    cpu = None
    if args.cpu_budget > 0:
        import oracle

        log(f"cpu baseline (oracle, ~{args.cpu_budget:.0f} s)")
        oracle.default()
        passes, t0 = 0, time.perf_counter()
        while True:
            oracle.swiglu_quant(case.acc, case.weight_scale, case.token_scale)
            passes += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_budget or passes >= 50:
                break
        cpu = dict(value=case.rows * passes / el, unit="rows/s", cores=1, kind="oracle",
                   sample=f"all {case.rows} rows x n={case.n}, {passes} pass(es) in {el:.1f} s on one host thread",
                   host_cpu=host_cpu_model(), host_nproc=os.cpu_count())
    line = {
        "metric": EPILOGUE_METRIC,
        "value": case.rows / (mean_us * 1e-6),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": mean_us * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "payload": "int32 GEMM accumulators in, int8 codes + fp32 inverse scale per row out",
        "data": "synthetic",
        "config": {"workload": "epilogue", "rows": case.rows, "n": case.n,
                   "rows_from": "4096 tokens x top-8 receive rows of the large shape",
                   "parallelism": "1 GPU"},
        "step": "one moe_deq_swiglu_quant launch, caches flushed before it",
        "timer": f"HIP events on the kernel's stream ({args.event_flags})",
        "stages_us": {"epilogue": {"mean": mean_us, "p10": pct(us, 0.1), "p50": pct(us, 0.5),
                                   "p90": pct(us, 0.9)}},
        "algorithmic_bytes": {"epilogue": alg},
        "roofline": {"bound": "hbm", "kernel": "deq_swiglu_quant", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": load_traffic("epilogue", "epilogue", f"n{case.n}")},
        "copy_ceiling_gbps": copy_gbps,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_gemm(args, M, torch, W, dev) -> int:
    """The first expert matmul alone on one GPU's share of the large shape on
    a 16-rank expert-parallel group: 32768 int8 rows (7296-byte receive rows)
    spread over 16 experts as uniform routing spreads them, k = 7168, n = 4096
    (gate and up columns of an FFN of width 2048).  The caches are flushed
    before each timed launch."""
    import numpy as np

    c = W.GEMM_CONFIG
    rows, k, n, groups = c["rows"], c["k"], c["n"], c["groups"]
    stride = M.moe_recv_row_bytes(k, M.MOE_INT8_ROWSCALE)
    log(f"generating gemm inputs rows={rows} k={k} n={n} groups={groups}")
    case = W.gemm_case(c["seed"], rows, k, n, groups, stride=stride)
    a = torch.from_numpy(case.a.reshape(-1).view("uint8")).to(dev)
    wt = torch.from_numpy(case.w.view("uint8")).to(dev)
    gc = torch.from_numpy(case.group_count).to(dev)
    out = torch.zeros((rows, n), dtype=torch.int32, device=dev)
    owned = int(min(max(case.group_count.astype("int64").clip(0).sum(), 0), rows))
    flush = torch.ones(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    flush_out = torch.zeros((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def launch():
        M.moe_grouped_gemm_i8(a, stride, rows, k, gc, wt, out)

    log(f"warm-up x{args.warmup}")
    for _ in range(args.warmup):
        torch.sum(flush, dim=0, out=flush_out)
        launch()
    torch.cuda.synchronize()
    log(f"timed x{args.steps}")
    hev = HipEvents(args.event_flags)
    ev = [(hev.new(), hev.new()) for _ in range(args.steps)]
    for e0, e1 in ev:
        torch.sum(flush, dim=0, out=flush_out)
        hev.record(e0, stream)
        launch()
        hev.record(e1, stream)
    torch.cuda.synchronize()
    us = [hev.ms(e0, e1) * 1e3 for e0, e1 in ev]
    log("un-flushed back-to-back")
    u0, u1 = hev.new(), hev.new()
    hev.record(u0, stream)
    for _ in range(args.steps):
        launch()
    hev.record(u1, stream)
    torch.cuda.synchronize()
    unflushed_us = hev.ms(u0, u1) * 1e3 / args.steps
    log("copy ceiling")
    dst = torch.empty_like(flush)
    for _ in range(2):
        torch.neg(flush, out=dst)
    c0, c1 = hev.new(), hev.new()
    hev.record(c0, stream)
    for _ in range(10):
        torch.neg(flush, out=dst)
    hev.record(c1, stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * flush.numel() * 4 * 10 / (hev.ms(c0, c1) * 1e-3) / 1e9
    del dst
    log("vendor library reference (torch._int_mm)")
    library = library_int8_reference(torch, hev, stream, flush, flush_out, rows, k, n, case.group_count,
                                     min(args.steps, 10))
    hev.close()
    mean_us = statistics.mean(us)
    ops = gemm_ops(owned, n, k)
    tops = ops / (mean_us * 1e-6) / 1e12
    alg = gemm_bytes(owned, n, k, groups)
    cpu = None
    if args.cpu_budget > 0:
        import oracle

        log(f"cpu baseline (oracle, ~{args.cpu_budget:.0f} s)")
        oracle.default()
        done, t0, batch = 0, time.perf_counter(), 8
        while True:
            sel = (W.u64(c["seed"], 40 + done // batch, batch) % np.uint64(rows)).astype("int64")
            oracle.grouped_gemm_i8(case.a, k, case.group_count, case.w, rows=sel)
            done += batch
            el = time.perf_counter() - t0
            if el >= args.cpu_budget or done >= 4096:
                break
        cpu = dict(value=done / el, unit="rows/s", cores=1, kind="oracle",
                   sample=f"{done} random rows of the {rows} (each: {n} x {k} products), {el:.1f} s on one "
                          "host thread",
                   host_cpu=host_cpu_model(), host_nproc=os.cpu_count())
    line = {
        "metric": GEMM_METRIC,
        "value": owned / (mean_us * 1e-6),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": mean_us * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "payload": "int8 receive rows and int8 expert weights in, int32 sums out",
        "data": "synthetic",
        "config": {"workload": "gemm", "rows": rows, "owned_rows": owned, "k": k, "n": n, "groups": groups,
                   "row_bytes": stride,
                   "rows_from": "one rank's receive rows on a 16-rank expert-parallel group at the large "
                                "shape (16 experts of 256)",
                   "parallelism": "1 GPU"},
        "step": "one moe_grouped_gemm_i8 launch, caches flushed before it",
        "timer": f"HIP events on the kernel's stream ({args.event_flags})",
        "stages_us": {"gemm": {"mean": mean_us, "p10": pct(us, 0.1), "p50": pct(us, 0.5),
                               "p90": pct(us, 0.9)}},
        "ops_per_launch": ops,
        "algorithmic_bytes": {"gemm": alg},
        "hbm_gbps_at_algorithmic_bytes": alg / (mean_us * 1e-6) / 1e9,
        "roofline": {"bound": "mfma", "kernel": "grouped_gemm_i8", "achieved": tops,
                     "peak": MFMA_I8_PEAK_TOPS, "unit": "TOP/s", "frac": tops / MFMA_I8_PEAK_TOPS,
                     "traffic": load_traffic("gemm", "gemm", f"n{n}")},
        "unflushed_us_per_launch": unflushed_us,
        "copy_ceiling_gbps": copy_gbps,
        "library_reference": library,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def gemm_swiglu_bytes(rows: int, n: int, k: int, groups: int) -> int:
    """Bytes the fused matmul and epilogue must move at least once: the k
    codes and the token scale of every row, every expert's 2n weight rows and
    2n column scales, the n int8 codes and inverse scale written per row, and
    the counts."""
    return rows * (k + 4) + groups * 2 * n * (k + 4) + rows * (n + 4) + groups * 4


def bench_gemm_swiglu(args, M, torch, W, dev) -> int:
    """The first expert matmul with its epilogue fused, on the shape of
    ``--stage gemm`` (2048 activation columns from 2 x 2048 weight rows per
    expert); caches flushed before each timed call.  The same run times the
    two separate calls (the matmul to int32, then the epilogue over every
    row) for comparison."""
    import numpy as np

    c = W.GEMM_CONFIG
    rows, k, n2, groups = c["rows"], c["k"], c["n"], c["groups"]
    n = n2 // 2
    stride = M.moe_recv_row_bytes(k, M.MOE_INT8_ROWSCALE)
    log(f"generating inputs rows={rows} k={k} n={n} groups={groups}")
    case = W.gemm_case(c["seed"], rows, k, n2, groups, stride=stride)
    ws, ts = W.gemm_swiglu_scales(c["seed"], rows, k, n, groups)
    a = torch.from_numpy(case.a.reshape(-1).view("uint8")).to(dev)
    wt = torch.from_numpy(case.w.view("uint8")).to(dev)
    gc = torch.from_numpy(case.group_count).to(dev)
    ws_d = torch.from_numpy(ws).to(dev)
    ts_d = torch.from_numpy(ts).to(dev)
    rb = M.moe_recv_row_bytes(n, M.MOE_INT8_ROWSCALE)
    out = torch.zeros(rows * rb, dtype=torch.uint8, device=dev)
    wsp = torch.empty(M.moe_gemm_swiglu_quant_workspace_bytes(rows, n), dtype=torch.uint8, device=dev)
    acc = torch.zeros((rows, n2), dtype=torch.int32, device=dev)
    out2 = torch.zeros(rows * rb, dtype=torch.uint8, device=dev)
    owned = int(min(max(case.group_count.astype("int64").clip(0).sum(), 0), rows))
    flush = torch.ones(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    flush_out = torch.zeros((), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def fused():
        M.moe_grouped_gemm_swiglu_quant_i8(a, stride, rows, k, gc, wt, ws_d, ts_d, out, wsp)

    def two_calls():
        M.moe_grouped_gemm_i8(a, stride, rows, k, gc, wt, acc)
        M.moe_deq_swiglu_quant(acc, ws_d[0], ts_d, out2)

    def timed(fn, steps):
        hev = HipEvents(args.event_flags)
        ev = [(hev.new(), hev.new()) for _ in range(steps)]
        for e0, e1 in ev:
            torch.sum(flush, dim=0, out=flush_out)
            hev.record(e0, stream)
            fn()
            hev.record(e1, stream)
        torch.cuda.synchronize()
        us = [hev.ms(e0, e1) * 1e3 for e0, e1 in ev]
        hev.close()
        return us

    log(f"warm-up x{args.warmup}")
    for _ in range(args.warmup):
        torch.sum(flush, dim=0, out=flush_out)
        fused()
        two_calls()
    torch.cuda.synchronize()
    log(f"timed x{args.steps}: fused")
    us = timed(fused, args.steps)
    log(f"timed x{args.steps}: two calls")
    us2 = timed(two_calls, args.steps)
    log("copy ceiling")
    hev = HipEvents(args.event_flags)
    dst = torch.empty_like(flush)
    for _ in range(2):
        torch.neg(flush, out=dst)
    c0, c1 = hev.new(), hev.new()
    hev.record(c0, stream)
    for _ in range(10):
        torch.neg(flush, out=dst)
    hev.record(c1, stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * flush.numel() * 4 * 10 / (hev.ms(c0, c1) * 1e-3) / 1e9
    hev.close()
    del dst
    mean_us, mean2 = statistics.mean(us), statistics.mean(us2)
    ops = gemm_ops(owned, n2, k)
    tops = ops / (mean_us * 1e-6) / 1e12
    alg = gemm_swiglu_bytes(owned, n, k, groups)
    cpu = None
    if args.cpu_budget > 0:
        import oracle

        log(f"cpu baseline (oracle, ~{args.cpu_budget:.0f} s)")
        oracle.default()
        done, t0, batch = 0, time.perf_counter(), 8
        while True:
            sel = (W.u64(c["seed"], 40 + done // batch, batch) % np.uint64(owned)).astype("int64")
            accs, grp = oracle.grouped_gemm_i8(case.a, k, case.group_count, case.w, rows=sel)
            for i, m in enumerate(sel):
                oracle.swiglu_quant_row(accs[i], ws[grp[i]], ts[m])
            done += batch
            el = time.perf_counter() - t0
            if el >= args.cpu_budget or done >= 4096:
                break
        cpu = dict(value=done / el, unit="rows/s", cores=1, kind="oracle",
                   sample=f"{done} random rows of the {rows} (each: {n2} x {k} products, then the epilogue), "
                          f"{el:.1f} s on one host thread",
                   host_cpu=host_cpu_model(), host_nproc=os.cpu_count())
    line = {
        "metric": GEMM_SWIGLU_METRIC,
        "value": owned / (mean_us * 1e-6),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": mean_us * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "payload": "int8 receive rows and int8 expert weights in, int8 rows (codes + fp32 inverse scale) out",
        "data": "synthetic",
        "config": {"workload": "gemm_swiglu", "rows": rows, "owned_rows": owned, "k": k, "n": n,
                   "weight_rows_per_expert": n2, "groups": groups, "row_bytes": stride,
                   "parallelism": "1 GPU"},
        "step": "one moe_grouped_gemm_swiglu_quant_i8 call (clear, matmul with the activation, quantisation), "
                "caches flushed before it",
        "timer": f"HIP events on the kernels' stream ({args.event_flags})",
        "stages_us": {"gemm_swiglu": {"mean": mean_us, "p10": pct(us, 0.1), "p50": pct(us, 0.5),
                                      "p90": pct(us, 0.9)},
                      "two_calls": {"mean": mean2, "p10": pct(us2, 0.1), "p50": pct(us2, 0.5),
                                    "p90": pct(us2, 0.9)}},
        "ops_per_launch": ops,
        "algorithmic_bytes": {"gemm_swiglu": alg},
        "roofline": {"bound": "mfma", "kernel": "grouped_gemm_swiglu", "achieved": tops,
                     "peak": MFMA_I8_PEAK_TOPS, "unit": "TOP/s", "frac": tops / MFMA_I8_PEAK_TOPS,
                     "traffic": load_traffic("gemm_swiglu", "gemm_swiglu", f"n{n}")},
        "copy_ceiling_gbps": copy_gbps,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def library_int8_reference(torch, hev, stream, flush, flush_out, rows, k, n, group_count, reps):
    """The vendor library's int8 x int8 -> int32 GEMM (torch._int_mm, which
    calls hipBLASLt on this stack) at the same sizes, after the same flush,
    for scale: one dense GEMM over all rows with one weight matrix (no
    grouping), and one GEMM per expert at that expert's row count (the host
    knows the counts here; the library entry point does not need them).
    Weights column-major (each output column's k contiguous, as the
    library's [groups][n][k] layout).  Inputs are random bytes; only the
    time is used.  None when the call is not available."""
    try:
        g = torch.Generator(device="cuda").manual_seed(5)
        a = torch.randint(-128, 127, (rows, k), dtype=torch.int8, device="cuda", generator=g)
        w = torch.randint(-128, 127, (n, k), dtype=torch.int8, device="cuda", generator=g).t()
        counts = [int(c) for c in group_count]

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            ev = [(hev.new(), hev.new()) for _ in range(reps)]
            for e0, e1 in ev:
                torch.sum(flush, dim=0, out=flush_out)
                hev.record(e0, stream)
                fn()
                hev.record(e1, stream)
            torch.cuda.synchronize()
            return statistics.mean(hev.ms(e0, e1) for e0, e1 in ev) * 1e3

        def per_expert():
            start = 0
            for c in counts:
                if c > 0:
                    torch._int_mm(a[start:start + c], w)
                start += max(c, 0)

        dense_us = timed(lambda: torch._int_mm(a, w))
        grouped_us = timed(per_expert)
        ops = 2 * rows * n * k
        return {"call": "torch._int_mm (hipBLASLt)", "dense_us": dense_us,
                "dense_tops": ops / (dense_us * 1e-6) / 1e12, "per_expert_calls_us": grouped_us,
                "per_expert_calls_tops": ops / (grouped_us * 1e-6) / 1e12}
    except (RuntimeError, AttributeError) as exc:
        log(f"library reference unavailable: {exc}")
        return None


def bench_sources(args, M, torch, w, x, idx, wts, quant: bool, do_flush, stream) -> int:
    """The workload's tokens split evenly into ``--sources`` source ranks
    sharing one receive buffer: a step is every source's layout, one notify
    over the [S, E] count matrix, every source's dispatch, then every
    source's combine (all on one stream; the caches are flushed before the
    step and before the combines)."""
    n_src = args.sources
    if w.bs % n_src:
        print(f"--sources must divide bs = {w.bs}", file=sys.stderr)
        return 2
    per = w.bs // n_src
    xs = [x[s * per:(s + 1) * per] for s in range(n_src)]
    idxs = [idx[s * per:(s + 1) * per] for s in range(n_src)]
    wss = [wts[s * per:(s + 1) * per] for s in range(n_src)]
    buf = M.EpMultiBuffers([per] * n_src, w.hidden, w.topk, w.expert_num_per_rank, w.rank_size,
                           x_dtype=x.dtype, quant_int8=quant, out_dtype=x.dtype)
    log(f"{n_src} sources of {per} tokens: warm-up x{args.warmup}")
    for _ in range(args.warmup):
        do_flush()
        buf.run(xs, idxs, wss)
    torch.cuda.synchronize()
    log(f"timed x{args.steps}")
    hev = HipEvents(args.event_flags)
    ev = [[hev.new() for _ in range(5)] for _ in range(args.steps)]
    for i in range(args.steps):
        e = ev[i]
        do_flush()
        hev.record(e[0], stream)
        for s in range(n_src):
            buf.layout(s, idxs[s])
        buf.notify()
        hev.record(e[1], stream)
        for s in range(n_src):
            buf.dispatch(s, xs[s], idxs[s])
        hev.record(e[2], stream)
        do_flush()
        hev.record(e[3], stream)
        for s in range(n_src):
            buf.combine(s, idxs[s], wss[s])
        hev.record(e[4], stream)
    torch.cuda.synchronize()
    lay_ms = [hev.ms(e[0], e[1]) for e in ev]
    dis_ms = [hev.ms(e[1], e[2]) for e in ev]
    com_ms = [hev.ms(e[3], e[4]) for e in ev]
    ms_per_step = statistics.mean([a + b + c for a, b, c in zip(lay_ms, dis_ms, com_ms)])
    log("un-flushed back-to-back")
    e0, e1 = hev.new(), hev.new()
    hev.record(e0, stream)
    for _ in range(args.steps):
        buf.run(xs, idxs, wss)
    hev.record(e1, stream)
    torch.cuda.synchronize()
    unflushed_ms = hev.ms(e0, e1) / args.steps
    hev.close()
    b_dis, b_com, b_lay = algorithmic_bytes(w.bs, w.hidden, w.topk, quant)
    dis_mean, com_mean = statistics.mean(dis_ms), statistics.mean(com_ms)
    dom = "dispatch" if dis_mean >= com_mean else "combine"
    dom_ms, dom_bytes = (dis_mean, b_dis) if dom == "dispatch" else (com_mean, b_com)
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    dc_gbps = (b_dis + b_com) / ((dis_mean + com_mean) * 1e-3) / 1e9
    cpu = cpu_baseline(w, quant, args.cpu_budget) if args.cpu_budget > 0 else None
    line = {
        "metric": METRIC,
        "value": w.bs / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "payload": (f"{args.x_dtype} rows in, int8 codes + fp32 inverse scale per row on the wire, "
                    f"{args.x_dtype} out" if quant
                    else f"{args.x_dtype} rows in and on the wire, {args.x_dtype} out"),
        "data": "synthetic",
        "config": {"workload": args.workload, "bs": w.bs, "hidden": w.hidden, "topk": w.topk,
                   "num_experts": w.num_experts, "rank_size": w.rank_size, "x_dtype": args.x_dtype,
                   "dispatch": "int8" if quant else "passthrough", "out_dtype": args.x_dtype,
                   "sources": n_src, "tokens_per_source": per,
                   "parallelism": "1 GPU, source and destination ranks are logical partitions"},
        "step": (f"{n_src} layouts + notify over the [{n_src}, E] counts, {n_src} dispatches, {n_src} "
                 "combines; caches flushed before the step and before the combines"),
        "path": "multi-source (one stream; each source's launches cover 1/S of the tokens)",
        "timer": f"HIP events on the kernels' stream ({args.event_flags})",
        "dispatch_combine_tokens_per_s": w.bs / ((dis_mean + com_mean) * 1e-3),
        "dispatch_combine_hbm_gbps": dc_gbps,
        "dispatch_combine_hbm_frac": dc_gbps / HBM_PEAK_GBPS,
        "stages_us": {
            name: {"mean": statistics.mean(v) * 1e3, "p10": pct(v, 0.1) * 1e3,
                   "p50": pct(v, 0.5) * 1e3, "p90": pct(v, 0.9) * 1e3}
            for name, v in (("layouts+notify", lay_ms), ("dispatches", dis_ms), ("combines", com_ms))
        },
        "algorithmic_bytes": {"dispatch": b_dis, "combine": b_com, "layout": b_lay},
        "roofline": {"bound": "hbm", "kernel": dom + " (all sources' launches)", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None},
        "unflushed_ms_per_step": unflushed_ms,
        "unflushed_tokens_per_s": w.bs / (unflushed_ms * 1e-3),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def counter_run(args, torch, w, buf, x, idx, wts, flush, do_flush) -> int:
    """Launches for a rocprofv3 --pmc run: the fused path and the separate
    stages, each K times, either flushed before every stage or back to back,
    then the copy kernel (torch.neg over the 1 GiB flush buffer: 1 GiB read,
    1 GiB written) on which the counters are calibrated."""
    flushed = args.counters == "flushed"
    maybe_flush = do_flush if flushed else (lambda: None)
    log(f"counter run ({args.counters}): warm-up x{args.warmup}")
    for _ in range(args.warmup):
        maybe_flush()
        buf.run(x, idx, wts, fused=True)
    log(f"fused path x{args.steps}")
    for _ in range(args.steps):
        maybe_flush()
        buf.layout_notify_dispatch(x, idx)
        maybe_flush()
        buf.combine(idx, wts)
    log(f"separate stages x{args.steps}")
    for _ in range(args.steps):
        maybe_flush()
        buf.layout(idx)
        buf.notify()
        buf.dispatch(x, idx)
        maybe_flush()
        buf.combine(idx, wts)
    dst = torch.empty_like(flush)
    for _ in range(3):
        torch.neg(flush, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"counter_run": args.counters, "workload": args.workload, "mode": args.mode,
                      "steps": args.steps, "warmup": args.warmup, "copy_bytes_each_way": flush.numel() * 4}),
          flush=True)
    return 0


DRAM_COUNTERS = ("TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum", "TCC_EA0_RDREQ_DRAM_sum",
                 "TCC_EA0_WRREQ_DRAM_sum")


def _read_counters(path: str):
    """{(kernel name, counter name): [value per dispatch]} from a rocprofv3
    counter_collection.csv."""
    import csv

    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("Kernel-Name") or ""
            ctr = row.get("Counter_Name") or row.get("Counter-Name") or ""
            val = row.get("Counter_Value") or row.get("Counter-Value")
            if val is None:
                continue
            out.setdefault((name, ctr), []).append(float(val))
    return out


def ingest_dram(args, flushed_csv: str, unflushed_csv: str) -> int:
    """Per-kernel DRAM-bound request counts of the fused, dispatch and
    combine kernels (median per dispatch) in both modes, in bytes: the 32-byte
    counters times 32, each scaled by what it reads for the 1 GiB copy kernel
    against the copy's bytes.  These are requests leaving L2 for the memory
    side; the 256 MB Infinity Cache sits behind them, so they bound HBM
    traffic from above rather than measure it."""
    import workloads as W

    c = W.CONFIGS[args.workload]
    quant = args.mode == "int8"
    b_dis, b_com, _ = algorithmic_bytes(c["bs"], c["hidden"], c["topk"], quant)
    copy_bytes = args.flush_mib * (1 << 20)
    kernels = (("fused", "fused_kernel", b_dis), ("dispatch", "dispatch_kernel", b_dis),
               ("combine", "combine_rows_kernel", b_com))
    rec = {"workload": args.workload, "mode": args.mode, "counters": list(DRAM_COUNTERS),
           "copy_bytes_each_way": copy_bytes, "runs": {},
           "note": "L2-to-memory-side requests destined for DRAM; the Infinity Cache is behind them"}
    for run, path in (("flushed", flushed_csv), ("unflushed", unflushed_csv)):
        t = _read_counters(path)

        def med(sym, ctr):
            vals = [v for (k, cn), vs in t.items() if sym in k and cn == ctr for v in vs]
            return statistics.median(vals) if vals else None

        rd_copy = med("neg", "TCC_EA0_RDREQ_DRAM_32B_sum")
        wr_copy = med("neg", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")
        cal = {"read_bytes_per_unit": copy_bytes / rd_copy if rd_copy else None,
               "write_bytes_per_unit": copy_bytes / wr_copy if wr_copy else None}
        out = {"copy_calibration": {"read_32B_units": rd_copy, "write_32B_units": wr_copy, **cal}}
        for name, sym, alg in kernels:
            rd, wr = med(sym, "TCC_EA0_RDREQ_DRAM_32B_sum"), med(sym, "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")
            if rd is None or wr is None:
                continue
            rb = rd * (cal["read_bytes_per_unit"] or 32.0)
            wb = wr * (cal["write_bytes_per_unit"] or 32.0)
            out[name] = {"rdreq_dram_32B": rd, "wrreq_write_dram_32B": wr,
                         "rdreq_dram": med(sym, "TCC_EA0_RDREQ_DRAM_sum"),
                         "wrreq_dram": med(sym, "TCC_EA0_WRREQ_DRAM_sum"),
                         "read_bytes": rb, "write_bytes": wb, "algorithmic_bytes": alg,
                         "over_algorithmic": (rb + wb) / alg}
        rec["runs"][run] = out
    rec["source_sha256_16"] = {k: source_hash(KERNEL_SOURCES[k]) for k in ("fused", "dispatch", "combine")}
    path = os.path.join(PROFILES, f"dram_requests_{args.workload}_{args.mode}.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(path, json.dumps(rec))
    return 0


def _read_counter_csv(path: str):
    """{kernel name: [value per dispatch]} from a rocprofv3 counter_collection.csv."""
    import csv

    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("Kernel-Name") or ""
            val = row.get("Counter_Value") or row.get("Counter-Value")
            if val is None:
                continue
            out.setdefault(name, []).append(float(val))
    return out


def ingest_pmc(args, fetch_csv: str, write_csv: str) -> int:
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the dispatch,
    combine and fused kernels (those the run launched) by what the same counters read for the bench's plain copy
    kernel (torch.neg over the 1 GiB flush buffer: 1 GiB read, 1 GiB written),
    and store bytes per launch with the kernel source hash."""
    fetch = _read_counter_csv(fetch_csv)
    write = _read_counter_csv(write_csv)
    copy_bytes = args.flush_mib * (1 << 20)

    def pick(table, key, required=True):
        cands = [(n, v) for n, v in table.items() if key in n]
        if not cands:
            if required:
                raise SystemExit(f"no kernel matching {key!r} in counters")
            return None, None
        n, v = max(cands, key=lambda nv: len(nv[1]))
        return n, statistics.median(v)

    _, f_copy = pick(fetch, "neg")
    _, w_copy = pick(write, "neg")
    f_scale = copy_bytes / (f_copy * 1024.0)
    w_scale = copy_bytes / (w_copy * 1024.0)
    quant = args.mode == "int8"
    w = None
    import workloads as W

    if args.stage == "gemm_swiglu":
        cg = W.GEMM_CONFIG
        workload, mode = "gemm_swiglu", f"n{cg['n'] // 2}"
        counts = W.gemm_case(cg["seed"], 1, 16, 1, cg["groups"], owned=cg["rows"]).group_count
        owned = int(min(counts.astype("int64").sum(), cg["rows"]))
        # the fused instance only (the run also times the plain matmul)
        kernels = (("gemm_swiglu", ("true>(moe::GemmArgs)",),
                    gemm_swiglu_bytes(owned, cg["n"] // 2, cg["k"], cg["groups"])),)
    elif args.stage == "gemm":
        cg = W.GEMM_CONFIG
        workload, mode = "gemm", f"n{cg['n']}"
        counts = W.gemm_case(cg["seed"], 1, 16, 1, cg["groups"], owned=cg["rows"]).group_count
        owned = int(min(counts.astype("int64").sum(), cg["rows"]))
        kernels = (("gemm", ("grouped_gemm_kernel",), gemm_bytes(owned, cg["n"], cg["k"], cg["groups"])),)
    elif args.stage == "epilogue":
        ce = W.EPILOGUE_CONFIG
        workload, mode = "epilogue", f"n{ce['n']}"
        kernels = (("epilogue", ("deq_swiglu_quant_kernel",), epilogue_bytes(ce["rows"], ce["n"])),)
    else:
        c = W.CONFIGS[args.workload]
        workload, mode = args.workload, args.mode
        b_dis, b_com, b_lay = algorithmic_bytes(c["bs"], c["hidden"], c["topk"], quant)
        kernels = (("dispatch", ("dispatch_kernel",), b_dis),
                   ("combine", ("combine_rows_kernel", "combine_kernel"), b_com),
                   ("fused", ("fused_kernel",), b_dis))
    for kernel, symbols, alg in kernels:
        if isinstance(symbols, str):
            symbols = (symbols,)
        kname = f = wr = None
        for symbol in symbols:  # the first symbol the run launched
            kname, f = pick(fetch, symbol, required=False)
            _, wr = pick(write, symbol, required=False)
            if f is not None and wr is not None:
                break
        if f is None or wr is None:
            continue  # not launched in this run
        traffic = f * 1024.0 * f_scale + wr * 1024.0 * w_scale
        rec = {
            "kernel": kname, "workload": workload, "mode": mode,
            "fetch_kib_per_dispatch": f, "write_kib_per_dispatch": wr,
            "copy_calibration": {"bytes_each_way": copy_bytes, "fetch_kib": f_copy, "write_kib": w_copy,
                                 "fetch_scale": f_scale, "write_scale": w_scale},
            "traffic_bytes_per_launch": traffic, "algorithmic_bytes_per_launch": alg,
            "traffic_over_algorithmic": traffic / alg,
            "source_sha256_16": source_hash(KERNEL_SOURCES[kernel]),
            "counters_from": [os.path.basename(fetch_csv), os.path.basename(write_csv)],
        }
        path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}_{mode}.json")
        with open(path, "w") as fh:
            json.dump(rec, fh, indent=1)
        print(path, json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
