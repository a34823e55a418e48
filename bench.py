"""Decode-step benchmark of the CLO hot path on one MI355X.

Default workload: the Llama3-8B decode-layer shape at batch 64 -- 32 query / 8
KV heads, d = 128, bf16, context 131072, top-k 13108 (10%), 80% of (sequence,
KV head) units with query cosine in [0.801, 0.98] (reuse hits) and 20% in
[0.2, 0.6] (misses), every KV head offloaded to pinned host memory.  One step =
the steady decode step (step 1): reuse test, scoring + top-k + zero-copy host
gather for the miss units, sparse attention for all units.

Prints one JSON line: steps/s, ms/step, the dominant kernel's roofline (host
gather against the host link; scoring against HBM is reported beside it), the
measured host-link reference, and the CPU oracle timed on a bounded sample.
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

METRIC = "sparse-attn decode steps/s (Llama3-8B shape, B=64); HBM & host-link GB/s vs peak"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
HOST_LINK_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction
HEAD_DIM = 128


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Markers:
    """roctx ranges around the benchmark's phases, so that a trace taken with
    `rocprofv3 --marker-trace` names them beside the kernels.  Each range is
    closed after its phase's closing synchronize, so the kernels that run inside
    it are that phase's.  A no-op where the roctx library is not installed."""

    def __init__(self):
        import ctypes

        self.lib = None
        for name in ("librocprofiler-sdk-roctx.so.1", "/opt/rocm/lib/librocprofiler-sdk-roctx.so.1"):
            try:
                lib = ctypes.CDLL(name)
            except OSError:
                continue
            lib.roctxRangePushA.argtypes, lib.roctxRangePushA.restype = [ctypes.c_char_p], ctypes.c_int
            lib.roctxRangePop.argtypes, lib.roctxRangePop.restype = [], ctypes.c_int
            self.lib = lib
            break

    def push(self, name: str):
        if self.lib is not None:
            self.lib.roctxRangePushA(name.encode())

    def pop(self):
        if self.lib is not None:
            self.lib.roctxRangePop()


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--data-layers", type=int, default=0,
                    help="configs 4-5: distinct K/V layer buffers, reused cyclically over the 48 layers")
    ap.add_argument("--step", type=int, default=1, choices=[0, 1], help="1 = steady step (headline), 0 = cold")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the host-link reference probes")
    ap.add_argument("--cpu-sample-seconds", type=float, default=10.0)
    ap.add_argument("--host-memory", choices=["mapped", "coherent", "noncoherent"], default="mapped",
                    help="pinned host memory kind for offloaded K/V (hipHostMalloc flags)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device-to-device copy first (reference for HBM byte counters)")
    ap.add_argument("--volatile", type=float, default=0.0, metavar="F",
                    help="head-dependent similarity: a fraction F of the (layer, KV head) slots draw the low "
                         "cosine class with probability 0.6, the others less often (20%% low overall)")
    ap.add_argument("--plan-persistent", action="store_true",
                    help="choose the persistent heads from profiling (mean reuse-test cosine per slot on "
                         "separately seeded instances, lowest first) instead of the seeded draw; same count")
    ap.add_argument("--profile-instances", type=int, default=8)
    ap.add_argument("--host-kv", choices=["native", "int8", "int4"], default="native",
                    help="format of the offloaded K/V in host memory: the step's dtype, or int8 / int4 rows with "
                         "one power-of-two scale per row (a half / a quarter of the host-link bytes of bf16; "
                         "dequantized exactly by the gather)")
    ap.add_argument("--block-size", type=int, default=0, metavar="B",
                    help="select blocks of B consecutive tokens instead of tokens (top-k a multiple of B: "
                         "k is rounded down to one)")
    ap.add_argument("--no-compare-native", action="store_true",
                    help="quantized host KV, configs 1-3: skip the output comparison against the native format")
    ap.add_argument("--layer", type=int, default=None, metavar="L",
                    help="configs 4-5: layer L alone through the single-layer fused step (clo_decode_step) "
                         "instead of the 48-layer loop: one layer's latency and phases, and a launch sequence "
                         "that rocprofv3 --pmc can run one kernel at a time (the loop's kernels wait on flags "
                         "that kernels on other streams set, which a serialized run cannot satisfy)")
    ap.add_argument("--counters", action="store_true",
                    help="for runs under rocprofv3 --pmc, which runs one kernel at a time: decode steps run in "
                         "order on one stream (CLO_STEP_IN_ORDER=1), since the overlapped step's gather and "
                         "attention wait for flags that kernels queued behind them raise; the 48-layer loop "
                         "is refused (use --layer)")
    ap.add_argument("--sync-probe", action="store_true",
                    help="measure the cross-stream hand-off instead of a decode step: HIP events, the command "
                         "processor's stream memory operations (hipStreamWaitValue32) and the library's device "
                         "flags, each between small calls on two streams")
    ap.add_argument("--select", choices=["batched", "per-layer"], default="batched",
                    help="48-layer loop: selections in multi-layer batches (clo_select_layers) or one "
                         "clo_reuse_select per layer")
    ap.add_argument("--attend", choices=["batched", "per-layer"], default="batched",
                    help="48-layer loop: attention in multi-layer batches (clo_attend_layers) or one "
                         "clo_sparse_attn per layer")
    ap.add_argument("--attend-batches", default="", metavar="N,N,...",
                    help="48-layer loop: attention batch sizes (default: workload.default_attend_batches)")
    ap.add_argument("--select-batches", default="", metavar="N,N,...",
                    help="48-layer loop: selection batch sizes (default: workload.default_select_batches)")
    ap.add_argument("--gather-blocks", type=int, default=0, metavar="G",
                    help="48-layer loop: blocks of the resident gather launch (default: clo_gather_plan's)")
    ap.add_argument("--select-streams", type=int, default=1, metavar="S",
                    help="48-layer loop: streams the layers' selections alternate between")
    ap.add_argument("--graph", action="store_true",
                    help="single-layer configs: capture one step into a HIP graph and time its replays "
                         "(launch-bound small steps)")
    ap.add_argument("--growing", type=int, default=0, metavar="T",
                    help="configs 1-3: T decode steps over a context that grows by one appended token per "
                         "step, under both reference policies (previous step's query / query at the last "
                         "miss): step time, hit rate, host bytes and drift from a fresh top-k step")
    return ap.parse_args()


def algorithmic_bytes(layers):
    """Bytes the method must move in one step over the given layers (no scores,
    histograms, q or idx), from each layer's reuse flags after the step.

    HBM: M * N * d * b (scoring) + M_p * k * 2 d b (persistent miss rows)
         + M_np * k * 2 d b (cache writes) + H * k * 2 d b (rows of reuse units)
    host: M_np * k * 2 d b_host (b_host = 1 for the int8 host format and 1/2 for
          int4, whose row exponents come from HBM: + M_np * k * 2 bytes there)
    """
    import numpy as np

    tot = dict(misses=0, misses_persistent=0, misses_host=0, hits=0, hbm_bytes=0, host_bytes=0, score_bytes=0,
               attn_bytes=0, flops=0)
    for bufs in layers:
        b = 4 if bufs.dtype == "f32" else 2
        reuse = bufs.reuse.cpu().numpy()
        miss = ~reuse.astype(bool)
        pers = np.array([bufs.is_persistent(h) for h in range(bufs.Hkv)])[None, :].repeat(bufs.B, 0)
        M = int(miss.sum())
        M_p = int((miss & pers).sum())
        M_np = M - M_p
        H = int((~miss).sum())
        g = bufs.Hq // bufs.Hkv
        row2 = bufs.k * 2 * HEAD_DIM * b
        score = M * bufs.N * HEAD_DIM * b
        tot["misses"] += M
        tot["misses_persistent"] += M_p
        tot["misses_host"] += M_np
        tot["hits"] += H
        tot["score_bytes"] += score
        fmt = getattr(bufs, "host_format", 0)
        q8 = fmt != 0  # a quantized host format
        host_row2 = bufs.k * 2 * {0: HEAD_DIM * b, 1: HEAD_DIM, 2: HEAD_DIM // 2}[fmt]
        tot["hbm_bytes"] += score + M_p * row2 + M_np * row2 + H * row2 + (M_np * bufs.k * 2 if q8 else 0)
        tot["host_bytes"] += M_np * host_row2
        tot["attn_bytes"] += bufs.B * bufs.Hkv * row2
        tot["flops"] += M * 2 * g * HEAD_DIM * bufs.N + bufs.B * bufs.Hkv * 4 * g * HEAD_DIM * bufs.k
    return tot


def profiled_traffic(kernel: str, cfg: int, layer=None):
    """HBM/host traffic of a kernel from a committed rocprofv3 counter record, or None.

    The record (profiles/<kernel>_traffic__*.json) stores the sha256 of the kernel
    source it was measured on; once the source changes the figure no longer
    applies and None is reported."""
    import glob
    import hashlib

    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic__*.json"))):
        try:
            rec = json.load(open(path))
        except (OSError, ValueError):
            continue
        if rec.get("kernel") != kernel or not rec.get("workload", "").startswith(f"config {cfg} "):
            continue
        if rec.get("layer") != layer:  # a record of one layer of a 48-layer workload names it
            continue
        src = os.path.join(ROOT, rec["source"])
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
            return None
        rec["path"] = os.path.relpath(path, ROOT)
        return rec
    return None


def score_roofline(score_gbs: float, alg: dict, args, multi: bool, hbm_probe=None) -> dict:
    """The scoring pass against HBM peak: live, as the whole clo_topk_select call
    (compaction, scoring and top-k, timed with events), and, where a committed
    kernel-trace record for this workload and source exists, the scoring kernel
    alone (rocprofv3 durations of the same launch)."""
    out = {"bound": "hbm", "kernel": "compact+score+topk", "achieved": round(score_gbs, 1), "peak": HBM_PEAK_GBS,
           "unit": "GB/s", "frac": round(score_gbs / HBM_PEAK_GBS, 4), "bytes_per_step": alg["score_bytes"]}
    rec = profiled_traffic("score_mfma_kernel", args.config, args.layer) if not multi and args.step == 1 else None
    if rec:
        gbs = rec["algorithmic_bytes_per_launch"] / (rec["mean_us"] * 1e3)
        out["kernel_only"] = {"kernel": "score_mfma_kernel", "achieved": round(gbs, 1),
                              "frac": round(gbs / HBM_PEAK_GBS, 4), "mean_us": rec["mean_us"],
                              "traffic": rec["traffic_bytes_per_launch"], "source": rec["path"]}
        if hbm_probe:
            out["kernel_only"]["frac_measured"] = round(gbs / hbm_probe["read_gbs"], 4)
    if hbm_probe:
        out["peak_measured"] = round(hbm_probe["read_gbs"], 1)
        out["frac_measured"] = round(score_gbs / hbm_probe["read_gbs"], 4)
    return out


def probe_hbm_read(torch, nbytes=4 << 30):
    """Measured HBM read ceiling: a plain streaming read (16-byte loads, nothing
    computed, almost nothing written) over a 4 GiB buffer, far larger than the
    256 MB MALL; best of a few grid sizes."""
    from top_sparse_attention_02_amd import clo

    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = (0.0, 0)
    for blocks in (512, 1024, 2048, 4096):
        times = []
        for i in range(4):
            e0.record()
            clo.clo_stream_read(buf, nbytes, blocks, sink)
            e1.record()
            e1.synchronize()
            if i:
                times.append(e0.elapsed_time(e1) / 1e3)
        gbs = nbytes / min(times) / 1e9
        if gbs > best[0]:
            best = (gbs, blocks)
    del buf, sink
    return {"read_gbs": best[0], "blocks": best[1], "bytes": nbytes}


def probe_host_link(torch, nbytes=1 << 30):
    """Measured host-link reference: SDMA memcpy of pinned memory, and the gather
    kernel streaming contiguous rows (identity index) from pinned memory."""
    from top_sparse_attention_02_amd import clo
    from top_sparse_attention_02_amd.hip_host import HostBuffer, copy_async

    res = {}
    hb = HostBuffer(nbytes)
    hb.numpy("u1")[:] = 1
    dev = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for i in range(4):
        e0.record()
        copy_async(dev.data_ptr(), hb.ptr, nbytes, s.cuda_stream)
        e1.record()
        e1.synchronize()
        if i:
            times.append(e0.elapsed_time(e1) / 1e3)
    res["memcpy_h2d_gbs"] = nbytes / min(times) / 1e9
    # zero-copy streaming read: one unit whose k = N rows are all selected in order
    rows = nbytes // (2 * HEAD_DIM * 2)  # K and V halves
    kv = HostBuffer(2 * rows * HEAD_DIM * 2)
    kv.numpy("u1")[:] = 1
    idx = torch.arange(rows, dtype=torch.int32, device="cuda").view(1, 1, rows)
    cache = torch.empty(2, rows, HEAD_DIM, dtype=torch.bfloat16, device="cuda")
    shape = clo.Shape(1, 1, 1, rows, rows, math.inf, clo.CLO_BF16)
    layer = clo.Layer(0, None, None, kv.ptr, kv.ptr + rows * HEAD_DIM * 2, None, cache[0], cache[1], idx)
    pws = torch.empty(clo.clo_workspace_size(shape), dtype=torch.uint8, device="cuda")
    times = []
    for i in range(4):
        e0.record()
        clo.clo_gather_kv(shape, layer, None, pws)
        e1.record()
        e1.synchronize()
        if i:
            times.append(e0.elapsed_time(e1) / 1e3)
    res["zero_copy_stream_gbs"] = 2 * rows * HEAD_DIM * 2 / min(times) / 1e9
    res["h_meas_gbs"] = max(res["memcpy_h2d_gbs"], res["zero_copy_stream_gbs"])
    del dev, cache, idx
    kv.close()
    hb.close()
    return res


def host_cpu_info():
    """CPUs this process may run on, and the CPU model from /proc/cpuinfo."""
    try:
        cpus = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        cpus = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cpus, model


def cpu_baseline(p, layers, budget_s, step_kind, full_step: bool, one_thread=False):
    """The CPU oracle, as it is, timed on the machine's host cores.

    Units run in parallel on a pool of worker threads (one per core of the
    process's CPU share, at most 16), each with a one-thread BLAS, so the
    oracle's matrix products and sorts of different units overlap.  Inputs are
    the generated ones only: the oracle classifies units with its own cosine
    test, and for a reused unit first makes its own previous selection from
    q_prev (untimed, before the timed region).  full_step: the whole step's
    units, timed three times, median (single-layer workloads); otherwise a
    bounded sample of miss and reuse units in the step's proportions, scaled
    to the step.  one_thread: the same with a single worker."""
    import concurrent.futures as cf

    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    cpus, model = host_cpu_info()
    workers = max(1, min(cpus, 16))
    g = p.g
    tau = p.tau if step_kind == 1 else math.inf
    miss_u, hit_u = [], []
    qs = {}
    for l in range(p.layers):
        qf, qpf = oracle.as_f64(p.q(l), p.dtype), oracle.as_f64(p.q_prev(l), p.dtype)
        query = qf if step_kind == 1 else qpf
        qs[l] = (query, qpf)
        for b in range(p.batch):
            for h in range(p.hkv):
                c = oracle.group_cosine(query[b, h * g:(h + 1) * g], qpf[b, h * g:(h + 1) * g])
                (hit_u if oracle.reuse_decision(c, tau) else miss_u).append((l, b, h))

    hit_set = set(hit_u)

    stored = {}  # persistent heads' K/V, generated again before the timed passes

    def kv_stored(l, b, h):
        bufs = layers[l]
        if bufs.is_persistent(h):
            return stored[(l, b, h)]
        return bufs.host_view("k", b, h), bufs.host_view("v", b, h)

    def groups(u):
        l, b, h = u
        query, qpf = qs[l]
        return query[b, h * g:(h + 1) * g], qpf[b, h * g:(h + 1) * g]

    def prev_selection(u):
        K, _ = kv_stored(*u)
        return oracle.select_topk(oracle.token_scores(groups(u)[1], oracle.as_f64(K, p.dtype)), p.topk)

    def unit(u, prev):
        K, V = kv_stored(*u)
        qg, qpg = groups(u)
        oracle.decode_unit(qg, qpg, oracle.as_f64(K, p.dtype), oracle.as_f64(V, p.dtype), p.topk, tau, prev)

    def run(units, prevs, nworkers):
        """Wall seconds of the oracle over `units` on nworkers threads."""
        t = time.perf_counter()
        with cf.ThreadPoolExecutor(max_workers=nworkers) as ex:
            list(ex.map(lambda u: unit(u, prevs.get(u)), units))
        return time.perf_counter() - t

    def prevs_of(units, nworkers):
        """Untimed preparation: the inputs of persistent heads (from the generator;
        non-persistent heads are read in place from pinned memory) and each reuse
        unit's previous selection."""
        for u in units:
            l, b, h = u
            if layers[l].is_persistent(h) and u not in stored:
                stored[u] = (p.kv("k", l, b, h), p.kv("v", l, b, h))
        hits = [u for u in units if u in hit_set]
        with cf.ThreadPoolExecutor(max_workers=nworkers) as ex:
            return dict(zip(hits, ex.map(prev_selection, hits)))

    def measure(nworkers, budget):
        """(seconds per step, miss units timed, reuse units timed)."""
        if full_step:
            units = miss_u + hit_u
            prevs = prevs_of(units, nworkers)
            return float(np.median([run(units, prevs, nworkers) for _ in range(3)])), len(miss_u), len(hit_u)
        # per class, a sample sized for about budget / 6 seconds per pass; its
        # median wall time over 3 passes per unit, times the class's units
        rng = np.random.default_rng(0)
        est, counts = 0.0, []
        for us in (miss_u, hit_u):
            if not us:
                counts.append(0)
                continue
            one = [us[0]]
            t1 = run(one, prevs_of(one, 1), 1)
            n = int(min(len(us), max(nworkers, budget / 6 / max(t1, 1e-4) * nworkers)))
            sample = [us[i] for i in rng.permutation(len(us))[:n]]
            prevs = prevs_of(sample, nworkers)
            wall = float(np.median([run(sample, prevs, nworkers) for _ in range(3)]))
            est += wall / n * len(us)
            counts.append(n)
        return est, counts[0], counts[1]

    def limited(fn, *a):
        if threadpool_limits is None:
            return fn(*a)
        with threadpool_limits(limits=1):
            return fn(*a)

    est, n_m, n_h = limited(measure, workers, budget_s)
    total = len(miss_u) + len(hit_u)
    what = (f"the whole step ({len(miss_u)} miss + {len(hit_u)} reuse units), median of 3" if full_step else
            f"samples of {n_m} miss and {n_h} reuse units of the {total}-unit step (median of 3 passes each), "
            f"per-unit wall times scaled to the step's {len(miss_u)} miss / {len(hit_u)} reuse units")
    out = {"value": round(1.0 / est, 6) if est > 0 else None, "unit": "steps/s", "cores": workers,
           "kind": "oracle",
           "sample": f"{what}; fp64 numpy oracle unchanged, units in parallel on {workers} worker threads with "
                     f"a one-thread BLAS each; each reuse unit's previous selection made by the oracle first, "
                     f"untimed",
           "seconds_per_step": round(est, 4), "host_cpus": cpus, "cpu_model": model, "blas_threads_per_worker": 1,
           "full_step": full_step}
    if one_thread:
        est1, _, _ = limited(measure, 1, budget_s / 2)
        out["value_1thread"] = round(1.0 / est1, 6) if est1 > 0 else None
        out["sample_1thread"] = "the same on one worker thread (one-thread BLAS)"
    return out


WORKLOADS = {
    1: "one layer, B=1, 32Q/8KV, d=128, N=4096, fp32, top-k 410, all heads persistent",
    2: "Llama3-8B layer, B=16, 32Q/8KV, d=128, N=32768, bf16, top-k 3277, 2/8 heads persistent",
    3: "Llama3-8B layer, B=64, 32Q/8KV, d=128, N=131072, bf16, top-k 13108, all heads host-resident",
    4: "Qwen2.5-14B, 48 layers, B=8, 40Q/8KV, d=128, N=262144, bf16, top-k 26215, ~47% of (layer, KV head) "
       "slots persistent",
    5: "Qwen2.5-14B, 48 layers, B=1, 40Q/8KV, d=128, N=524288, bf16, top-k 52429, ~47% of (layer, KV head) "
       "slots persistent",
}


def phase_times(torch, clo, layers, step_kind, passes):
    """Per-phase GPU times (ms per step): the step's kernels through the separate
    entry points, in order on one stream, with events between them."""
    import numpy as np

    names = ["reuse_test", "score_topk", "gather", "attention"]
    acc = {n: [] for n in names}
    torch.cuda.synchronize()
    for _ in range(passes):
        evs = []
        for bufs in layers:
            tau = bufs.tau if step_kind == 1 else math.inf
            query = bufs.q if step_kind == 1 else bufs.q_prev
            shape, layer = bufs.shape_with(tau), bufs.layer()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            ev[0].record()
            clo.clo_reuse_test(shape, query, bufs.q_prev, bufs.reuse, bufs.cos)
            ev[1].record()
            clo.clo_topk_select(shape, layer, query, bufs.reuse, bufs.ws)
            ev[2].record()
            clo.clo_gather_kv(shape, layer, bufs.reuse, bufs.ws)
            ev[3].record()
            clo.clo_sparse_attn(shape, layer, query, bufs.out, bufs.ws)
            ev[4].record()
            evs.append(ev)
        torch.cuda.synchronize()
        for j, n in enumerate(names):
            acc[n].append(sum(ev[j].elapsed_time(ev[j + 1]) for ev in evs))
    return {n: float(np.mean(v)) for n, v in acc.items()}


def select_phase_ms(torch, clo, loop, step_kind, passes) -> float:
    """ms per step of the loop's multi-layer selections alone (every layer, in the
    loop's batches, on one stream, nothing else running)."""
    plan = loop.sel_plans[step_kind == 0]
    e = loop.epoch  # flags keep their values: waits for e - 1 pass, signals store e again
    times = []
    for _ in range(passes):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        first = 0
        for n in loop.batches:
            clo.clo_select_layers(loop.layers[0].shape, plan, first, n, e - 1, e, error_word=loop.error)
            first += n
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    loop.check()
    return float(sorted(times)[len(times) // 2])


def growing_bench(torch, clo, workload, gen, cfg: int, steps: int) -> dict:
    """T steps over a growing context (the workload's context plus one appended
    token per step; k fixed at the workload's top-k), per reference policy.

    Timed per step (HIP events around the step's calls: append, decode, reference
    update).  Drift: after the timed pass, each step's output against a fresh
    top-k step (tau = +inf) at the same context with the same query, normwise per
    (sequence, query head): max_i |o_i - f_i| / max_i |f_i|."""
    import numpy as np

    base = gen.config(cfg)
    n0 = base.context
    p = gen.config(cfg, context=n0 + steps, topk=base.topk)
    log(f"growing context: N0={n0}, {steps} appended tokens, k={p.topk}; generating inputs")
    t0 = time.time()
    run = workload.GrowingRun(p, 0, steps, "previous")
    b = run.bufs
    fresh = workload.LayerBuffers(p.batch, p.hq, p.hkv, p.context, p.topk, p.dtype, b.mask, p.tau, share=b)
    log(f"inputs ready ({time.time() - t0:.1f} s)")
    eb = 4 if p.dtype == "f32" else 2
    host = np.array([not b.is_persistent(h) for h in range(b.Hkv)])[None, :]
    res = {}
    for policy in ("previous", "refresh"):
        run.reset(policy)
        outs = torch.empty((steps + 1,) + tuple(b.out.shape), dtype=b.out.dtype, device=b.out.device)
        reuse = torch.empty((steps + 1,) + tuple(b.reuse.shape), dtype=torch.uint8, device=b.out.device)
        run.step(0)
        torch.cuda.synchronize()
        evs = []
        for t in range(1, steps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run.step(t)
            e1.record()
            outs[t].copy_(b.out)
            reuse[t].copy_(b.reuse)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(z) for a, z in evs])
        drift_mean, drift_max = [], []
        for t in range(1, steps + 1):
            clo.clo_decode_step(run.shape(t, math.inf), fresh.layer(), run.qs[t], run.qs[t], fresh.out, fresh.reuse,
                                fresh.cos, fresh.ws)
            f = fresh.out.float()
            err = (outs[t].float() - f).abs().amax(-1) / f.abs().amax(-1).clamp_min(1e-30)
            drift_mean.append(float(err.mean()))
            drift_max.append(float(err.max()))
        torch.cuda.synchronize()
        r = reuse[1:].cpu().numpy().astype(bool)
        host_misses = (~r & host).sum(axis=(1, 2))
        host_bytes = host_misses * p.topk * 2 * HEAD_DIM * eb
        res[policy] = {
            "steps_per_s": round(1000.0 / float(ms.mean()), 3),
            "ms_per_step": round(float(ms.mean()), 4),
            "ms_per_step_min_max": [round(float(ms.min()), 4), round(float(ms.max()), 4)],
            "hit_rate": round(float(r.mean()), 4),
            "hit_rate_per_step": [round(float(x), 4) for x in r.mean(axis=(1, 2))],
            "host_gb_per_step": round(float(host_bytes.mean()) / 1e9, 4),
            "host_gbs": round(float(host_bytes.sum()) / (float(ms.sum()) / 1e3) / 1e9, 2),
            "drift_mean": round(float(np.mean(drift_mean)), 5),
            "drift_max": round(float(np.max(drift_max)), 5),
            "drift_mean_per_step": [round(x, 5) for x in drift_mean],
        }
        log(f"{policy}: {res[policy]['steps_per_s']} steps/s, hit rate {res[policy]['hit_rate']}, "
            f"drift mean {res[policy]['drift_mean']}")
    return {"n0": n0, "steps": steps, "topk": p.topk, "policies": res}


def profile_and_plan(torch, clo, gen, cfg: int, overrides: dict, instances: int) -> dict:
    """Profiling-based persistent heads: run the reuse test (on the GPU, through
    the C ABI) on `instances` separately seeded copies of the workload that share
    its volatile slots, average each (data layer, KV head) slot's cosine, and let
    clo_plan_persistent mark the slots with the lowest mean as persistent -- as
    many as the seeded draw has."""
    import numpy as np

    from top_sparse_attention_02_amd import workload

    base = gen.config(cfg, **overrides)
    L, H = base.layers, base.hkv
    period = base.data_layers or L
    n = int(base.persistent[:period].sum())
    sums = np.zeros((period, H))
    counts = np.zeros((period, H))
    for i in range(instances):
        pi = gen.config(cfg, **{**overrides, "seed": base.seed + 7919 * (i + 1), "slot_seed": base.seed})
        shape = clo.Shape(pi.batch, pi.hq, pi.hkv, pi.context, pi.topk, pi.tau, workload.clo_dtype(pi.dtype))
        cos = torch.zeros(pi.batch, H, dtype=torch.float32, device="cuda")
        reuse = torch.zeros(pi.batch, H, dtype=torch.uint8, device="cuda")
        for l in range(L):
            q = workload.stored_tensor(pi.q(l), pi.dtype)
            qp = workload.stored_tensor(pi.q_prev(l), pi.dtype)
            clo.clo_reuse_test(shape, q, qp, reuse, cos)
            sums[l % period] += cos.sum(0).cpu().numpy()
            counts[l % period] += pi.batch
    s_hat = (sums / counts).astype(np.float32)
    masks = clo.clo_plan_persistent(s_hat, n)
    plan = np.array([[(m >> h) & 1 for h in range(H)] for m in masks], dtype=bool)
    vol = base.volatile_slots()[:period]
    log(f"profiled {instances} instances: {n} persistent slots, {int((plan & vol).sum())} of {int(vol.sum())} "
        f"volatile slots among them (seeded draw: {int((base.persistent[:period] & vol).sum())})")
    return {"persistent": np.stack([plan[l % period] for l in range(L)]), "n_persistent_slots": n,
            "profile_instances": instances, "volatile_slots": int(vol.sum()),
            "volatile_persistent_planned": int((plan & vol).sum()),
            "volatile_persistent_seeded": int((base.persistent[:period] & vol).sum())}


def compare_tokens(torch, bufs, step_kind: int) -> dict:
    """Block selection against token selection on the same layer: the same step
    with block_size 1, normwise output deviation per (sequence, query head) and
    the fraction of the block-selected tokens that token selection also takes."""
    out_b = bufs.out.float().clone()
    idx_b = bufs.idx.clone()
    bs = bufs.shape.block_size
    bufs.set_block_size(0)
    bufs.step0()
    if step_kind == 1:
        bufs.step1()
    torch.cuda.synchronize()
    n = bufs.out.float()
    dev = (out_b - n).abs().amax(-1) / n.abs().amax(-1).clamp_min(1e-30)
    ib, it = idx_b.cpu().numpy(), bufs.idx.cpu().numpy()
    overlap = float(sum(len(set(ib[b, h]) & set(it[b, h])) for b in range(ib.shape[0]) for h in range(ib.shape[1]))
                    / ib.size)
    bufs.set_block_size(bs)
    return {"out_dev_mean": float(dev.mean()), "out_dev_max": float(dev.max()), "selection_overlap": overlap}


def compare_native(torch, workload, p, q8_layer, step_kind: int, flags) -> dict:
    """Output of the quantized-host-KV step against the same step with native host
    rows (the same inputs loaded a second time): normwise relative deviation per
    (sequence, query head), max_i |o_i - n_i| / max_i |n_i|, and how many
    selections differ (none can: scoring reads the exact keys in both)."""
    nat = workload.load_layer(p, 0, host_flags=flags)
    for bufs in (nat, q8_layer):
        bufs.step0()
        if step_kind == 1:
            bufs.step1()
    torch.cuda.synchronize()
    o, n = q8_layer.out.float(), nat.out.float()
    dev = (o - n).abs().amax(-1) / n.abs().amax(-1).clamp_min(1e-30)
    res = {"out_dev_mean": float(dev.mean()), "out_dev_max": float(dev.max()),
           "selections_equal": bool(torch.equal(q8_layer.idx, nat.idx))}
    del nat
    return res


def sync_probe(torch, clo, rounds: int = 500, trials: int = 3) -> dict:
    """Cross-stream hand-off latency.  Two streams take turns, 2 x rounds turns in
    all; each turn is one small library call (the reuse test of one sequence with
    2 KV heads, fp32: one short kernel) that may start only after the other
    stream's previous call.  The hand-off is made (a) with HIP events
    (hipStreamWaitEvent), (b) with the command processor's stream memory
    operations (hipStreamWriteValue32 after a call, hipStreamWaitValue32 before
    the next, on a word of signal memory), and (c) with the library's device
    flags (the clo_sync signal store after a call and the polling wait before
    the next, one kernel each).  The same calls back to back on one stream give
    the work alone; a turn's time minus that is the hand-off's cost.  Every
    producer is enqueued before its consumer, so every wait ends."""
    from top_sparse_attention_02_amd import hip_host

    shape = clo.Shape(1, 8, 2, 64, 7, 0.8, clo.CLO_F32)
    q = torch.randn(1, 8, HEAD_DIM, device="cuda")
    qp = torch.randn_like(q)
    reuse = torch.zeros(1, 2, dtype=torch.uint8, device="cuda")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    streams = (sa, sb)
    turns = 2 * rounds
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    cp_ok = hip_host.can_wait_value()
    sig = hip_host.signal_word() if cp_ok else None
    events = [torch.cuda.Event() for _ in range(turns)]
    base = [0]

    def work(s, sync=None):
        clo.clo_reuse_test(shape, q, qp, reuse, sync=sync, stream=s)

    def one_stream():
        for _ in range(turns):
            work(sa)

    def by_events():
        for t in range(turns):
            s = streams[t % 2]
            if t:
                s.wait_event(events[t - 1])
            work(s)
            events[t].record(s)

    def by_stream_ops():
        b = base[0]
        for t in range(turns):
            s = streams[t % 2]
            if t:
                hip_host.stream_wait_value32(s.cuda_stream, sig, b + t)
            work(s)
            hip_host.stream_write_value32(s.cuda_stream, sig, b + t + 1)
        base[0] = b + turns + 1

    def by_flags():
        b = base[0]
        for t in range(turns):
            s = streams[t % 2]
            work(s, clo.Sync(wait_flag=flag if t else None, wait_value=b + t, signal_flag=flag,
                             signal_value=b + t + 1))
        base[0] = b + turns + 1

    def timed(fn) -> float:
        best = math.inf
        for _ in range(trials):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(sa)
            sb.wait_stream(sa)
            fn()
            sa.wait_stream(sb)
            e1.record(sa)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / turns)
        return best

    if cp_ok:
        hip_host.stream_write_value32(sa.cuda_stream, sig, 0)
    torch.cuda.synchronize()
    alone = timed(one_stream)
    res = {"work_alone_us": round(alone, 2)}
    for name, fn in (("events", by_events), ("stream_wait_value", by_stream_ops if cp_ok else None),
                     ("device_flags", by_flags)):
        if fn is None:
            res[name] = None
            continue
        us = timed(fn)
        res[name] = {"us_per_turn": round(us, 2), "handoff_us": round(us - alone, 2)}
    res["turns"] = turns
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path has no "
              f"multi-GPU exchange: units shard by sequence or KV head, one process per GPU).", file=sys.stderr)
        sys.exit(2)
    if args.counters:
        if args.config in (4, 5) and args.layer is None:
            print("--counters: the 48-layer loop's streams wait on each other's flags; pass --layer L",
                  file=sys.stderr)
            sys.exit(2)
        os.environ["CLO_STEP_IN_ORDER"] = "1"  # read by the library at its first decode step
    import torch

    import gen
    from top_sparse_attention_02_amd import clo, workload

    torch.cuda.set_device(0)
    clo.load()
    if args.growing:
        if args.config not in (1, 2, 3):
            print("--growing runs a single-layer workload (configs 1-3)", file=sys.stderr)
            sys.exit(2)
        g = growing_bench(torch, clo, workload, gen, args.config, args.growing)
        prev = g["policies"]["previous"]
        print(json.dumps({
            "metric": "sparse-attn decode steps/s over a growing context (one appended token per step)",
            "value": prev["steps_per_s"], "unit": "steps/s", "n_gpus": 1, "steps": args.growing, "warmup": 1,
            "ms_per_step": prev["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": gen.config(args.config).dtype, "data": "synthetic (seeded; query walk with the 80/20 cosine model)",
            "config": {"workload": f"config {args.config}: " + WORKLOADS[args.config] +
                       f", {args.growing} decode steps with one appended token each, reference = previous query"},
            "growing": g}), flush=True)
        return
    if args.sync_probe:
        r = sync_probe(torch, clo)
        log(f"hand-off per turn: {r}")
        print(json.dumps({
            "metric": "cross-stream hand-off latency on the GPU (library device flags), us per turn",
            "value": r["device_flags"]["handoff_us"], "unit": "us", "n_gpus": 1, "steps": r["turns"],
            "warmup": 0, "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic", "config": {"workload": "two streams taking turns, one small call per turn"},
            "sync_probe": r}), flush=True)
        return
    overrides = {}
    if args.config in (4, 5):
        # distinct K/V layer buffers: 8 for B=8 (36 GB of offloaded K/V in pinned host
        # memory; 16 would need 72 GB, past the 64 GiB a process can pin on these
        # hosts), 16 for B=1
        overrides["data_layers"] = args.data_layers or (8 if args.config == 4 else 16)
    if args.volatile:
        overrides["volatile_frac"] = args.volatile
    if args.block_size > 1:
        overrides["topk"] = gen.config(args.config).topk // args.block_size * args.block_size
    plan = None
    if args.plan_persistent:
        plan = profile_and_plan(torch, clo, gen, args.config, overrides, args.profile_instances)
        overrides["persistent"] = plan["persistent"]
    p = gen.config(args.config, **overrides)
    if args.layer is not None and not (args.config in (4, 5) and 0 <= args.layer < p.layers):
        print(f"--layer takes a layer 0..{p.layers - 1} of config 4 or 5", file=sys.stderr)
        sys.exit(2)
    multi = p.layers > 1 and args.layer is None
    n_layers = p.layers if multi else 1
    log(f"config {args.config}: L={p.layers} B={p.batch} Hq={p.hq} Hkv={p.hkv} N={p.context} k={p.topk} "
        f"{p.dtype} data layers={p.data_layers or p.layers}")
    from top_sparse_attention_02_amd import hip_host

    flags = {"mapped": hip_host.hipHostMallocMapped,
             "coherent": hip_host.hipHostMallocMapped | hip_host.hipHostMallocCoherent,
             "noncoherent": hip_host.hipHostMallocMapped | hip_host.hipHostMallocNonCoherent}[args.host_memory]
    t0 = time.time()
    host_format = {"native": clo.CLO_HOST_NATIVE, "int8": clo.CLO_HOST_INT8,
                   "int4": clo.CLO_HOST_INT4}[args.host_kv]
    if multi:
        layers = workload.load_layers(p, log=log, host_flags=flags, host_format=host_format)
    else:
        layers = [workload.load_layer(p, args.layer or 0, log=log if p.batch >= 16 else None, host_flags=flags,
                                      host_format=host_format)]
    log(f"inputs generated and resident ({time.time() - t0:.1f} s)")

    mk = Markers()
    probe = None
    mk.push("probes")
    if not args.no_probe:
        probe = probe_host_link(torch)
        log(f"host link: memcpy {probe['memcpy_h2d_gbs']:.1f} GB/s, zero-copy stream "
            f"{probe['zero_copy_stream_gbs']:.1f} GB/s")

    hbm_probe = None
    if not args.no_probe:
        hbm_probe = probe_hbm_read(torch)
        log(f"HBM read ceiling: {hbm_probe['read_gbs']:.0f} GB/s ({hbm_probe['blocks']} blocks)")
    mk.pop()

    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy done: 1 GiB read + 1 GiB written")

    if args.block_size > 1:
        for bufs in layers:
            bufs.set_block_size(args.block_size)
    mk.push("cold step and warmup")
    if multi:
        att_batches = tuple(int(x) for x in args.attend_batches.split(",")) if args.attend_batches else None
        sel_batches = tuple(int(x) for x in args.select_batches.split(",")) if args.select_batches else None
        loop = workload.LayerLoop(layers, select_streams=args.select_streams, select=args.select,
                                  attend=args.attend, attend_batches=att_batches, gather_blocks=args.gather_blocks,
                                  select_batches=sel_batches)
        loop.step(cold=True)
        step = (lambda: loop.step()) if args.step == 1 else (lambda: loop.step(cold=True))
    else:
        layers[0].step0()
        step = layers[0].step1 if args.step == 1 else layers[0].step0
    torch.cuda.synchronize()
    if args.graph:
        if multi:
            print("--graph is for single-layer configs (the 48-layer loop waits on device flags)", file=sys.stderr)
            sys.exit(2)
        graph = workload.capture_step(step)
        step = graph.replay
        log("step captured into a HIP graph; timing its replays")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    mk.pop()

    # timed region: K whole decode steps (all layers)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    mk.push("timed steps")
    t_wall = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    mk.pop()
    # a second pass of K steps with an event after every step, for the per-step
    # median and minimum (kept out of the timed region above: at tens of
    # microseconds per step the extra events would show in it)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    mk.push("per-step pass")
    ev[0].record()
    for i in range(args.steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    mk.pop()
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    # host time to enqueue one step (argument checks and launches) onto an idle
    # GPU, median of K: while it stays below ms_per_step the GPU side is the limit
    # (and, for an overlapped single-layer step, the GPU time of the gather inside
    # each of these steps, from events the library records on its gather streams)
    sched = None if multi else clo.clo_decode_step_schedule(layers[0].shape, layers[0].mask, host_format)
    in_step = sched is not None and sched["mode"] != "in order" and not args.graph and not args.counters
    enq, gather_in_step = [], []
    mk.push("enqueue pass")
    for _ in range(args.steps):
        torch.cuda.synchronize()
        if in_step and enq:
            gather_in_step.append(clo.clo_last_step_gather_ms())
        t0 = time.perf_counter()
        step()
        enq.append(time.perf_counter() - t0)
    torch.cuda.synchronize()
    if in_step:
        gather_in_step.append(clo.clo_last_step_gather_ms())
    mk.pop()
    enqueue_us = sorted(enq)[len(enq) // 2] * 1e6
    if multi:
        loop.check()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    alg = algorithmic_bytes(layers)

    blocks = None
    if args.block_size > 1 and not multi:
        blocks = compare_tokens(torch, layers[0], args.step)
        log(f"blocks of {args.block_size} vs tokens: output deviation mean {blocks['out_dev_mean']:.3f}, "
            f"selection overlap {blocks['selection_overlap']:.3f}")
    quant = None
    if host_format != clo.CLO_HOST_NATIVE and not multi and not args.no_compare_native:
        quant = compare_native(torch, workload, p, layers[0], args.step, flags)
        log(f"{args.host_kv} host KV vs native: output deviation mean {quant['out_dev_mean']:.2e}, "
            f"max {quant['out_dev_max']:.2e}")
    mk.push("phase passes")
    phases = phase_times(torch, clo, layers, args.step, passes=args.steps if not multi else 2)
    if multi and loop.select == "batched":
        phases["select_batched"] = select_phase_ms(torch, clo, loop, args.step, passes=3)
    torch.cuda.synchronize()
    mk.pop()
    gather_s = phases["gather"] / 1e3
    host_gbs = alg["host_bytes"] / gather_s / 1e9 if alg["host_bytes"] else 0.0
    score_s = phases["score_topk"] / 1e3
    score_gbs = alg["score_bytes"] / score_s / 1e9 if alg["score_bytes"] else 0.0
    attn_gbs = alg["attn_bytes"] / (phases["attention"] / 1e3) / 1e9
    step_s = ms_per_step / 1e3
    if alg["host_bytes"] and gather_in_step:
        # the dominant kernel as it runs inside the timed step: the resident
        # range gather (or the range gathers on two streams), event-timed on the
        # library's gather streams, averaged over K steps
        g_ms = sum(gather_in_step) / len(gather_in_step)
        g_gbs = alg["host_bytes"] / (g_ms / 1e3) / 1e9
        resident = sched["mode"] == "one resident gather launch"
        roofline = {"bound": "host-link",
                    "kernel": "gather_ranges_kernel" if resident else
                              f"gather_kernel ({sched['ranges']} range launches on two streams)",
                    "achieved": round(g_gbs, 2), "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                    "frac": round(g_gbs / HOST_LINK_PEAK_GBS, 4), "traffic": None,
                    "bytes_per_launch": alg["host_bytes"], "launch_ms": round(g_ms, 4),
                    "launch_ms_median": round(sorted(gather_in_step)[len(gather_in_step) // 2], 4),
                    "launches_timed": len(gather_in_step),
                    "standalone": {"kernel": "gather_kernel", "launch_ms": round(phases["gather"], 4),
                                   "achieved": round(host_gbs, 2),
                                   "frac": round(host_gbs / HOST_LINK_PEAK_GBS, 4)}}
    elif alg["host_bytes"]:
        roofline = {"bound": "host-link", "kernel": "gather_kernel", "achieved": round(host_gbs, 2),
                    "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s", "frac": round(host_gbs / HOST_LINK_PEAK_GBS, 4),
                    "traffic": None, "bytes_per_launch": alg["host_bytes"] // len(layers),
                    "launch_ms": round(phases["gather"] / len(layers), 4)}
    if alg["host_bytes"]:
        # the committed record covers the native-format token gather of the steady step only
        same_launch = not multi and args.step == 1 and args.host_kv == "native" and args.block_size <= 1
        rec = profiled_traffic("gather_kernel", args.config, args.layer) if same_launch else None
        if rec:
            roofline["traffic"] = rec["traffic_bytes_per_launch"]
            roofline["traffic_detail"] = {"read_bytes": rec["read_bytes_per_launch"],
                                          "write_bytes": rec["write_bytes_per_launch"],
                                          "fetch_scale": rec["fetch_scale"], "write_scale": rec["write_scale"],
                                          "source": rec["path"]}
            if gather_in_step:
                roofline["traffic_detail"]["of"] = (
                    "the standalone gather_kernel launch over the same rows: counter runs execute one kernel "
                    "at a time, under which the step's overlapped gather cannot run")
        if probe:
            roofline["peak_measured"] = round(probe["h_meas_gbs"], 2)
            roofline["frac_measured"] = round(roofline["achieved"] / probe["h_meas_gbs"], 4)
    else:
        roofline = {"bound": "hbm", "kernel": "attn_partial_kernel", "achieved": round(attn_gbs, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                    "traffic": None}
        if hbm_probe:
            roofline["peak_measured"] = round(hbm_probe["read_gbs"], 1)
            roofline["frac_measured"] = round(attn_gbs / hbm_probe["read_gbs"], 4)

    # how the gather runs: its grid and the host bytes its loads keep in flight
    # (the gather grids sit near measured cliffs, so a change shows here)
    per_block = clo.clo_decode_step_schedule(layers[0].shape, layers[0].mask,
                                             host_format)["host_bytes_per_gather_block"]
    if multi:
        gb = loop.plan_blocks if loop.gather == "resident" else None
        gather_schedule = {"mode": "48-layer loop, " + ("one resident gather launch per step" if gb else
                                                          "a gather launch per layer"),
                           "gather_blocks": gb, "host_bytes_in_flight": gb * per_block if gb else None}
    else:
        gather_schedule = clo.clo_decode_step_schedule(layers[0].shape, layers[0].mask, host_format)
        if args.graph:
            gather_schedule["mode"] = "in order (graph capture)"
        if args.counters:
            gather_schedule["mode"] = "in order (--counters)"

    # the step's lower bounds from its algorithmic bytes: the host link at the
    # rate measured in this run (without the probe, at the link's published
    # peak), HBM at the published peak and at the measured read ceiling; the
    # step can overlap the two, so its bound is the larger
    host_bound_ms = alg["host_bytes"] / (probe["h_meas_gbs"] * 1e9) * 1e3 if probe else None
    host_bound_peak_ms = alg["host_bytes"] / (HOST_LINK_PEAK_GBS * 1e9) * 1e3
    hbm_bound_ms = alg["hbm_bytes"] / (HBM_PEAK_GBS * 1e9) * 1e3
    hbm_bound_meas_ms = alg["hbm_bytes"] / (hbm_probe["read_gbs"] * 1e9) * 1e3 if hbm_probe else None
    step_bound_ms = max(host_bound_ms or host_bound_peak_ms, hbm_bound_meas_ms or hbm_bound_ms)
    bounds = {"host_bytes": alg["host_bytes"], "hbm_bytes": alg["hbm_bytes"],
              "host_bound_ms": round(host_bound_ms, 4) if host_bound_ms is not None else None,
              "host_bound_ms_at_peak": round(host_bound_peak_ms, 4),
              "hbm_bound_ms_at_peak": round(hbm_bound_ms, 4),
              "hbm_bound_ms_at_read_ceiling": round(hbm_bound_meas_ms, 4) if hbm_bound_meas_ms else None,
              "step_bound_ms": round(step_bound_ms, 4),
              "frac_of_step_bound": round(step_bound_ms / ms_per_step, 4),
              "host_enqueue_us_per_step": round(enqueue_us, 2)}

    result = {
        "metric": METRIC,
        "value": round(1.0 / step_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(per_step[len(per_step) // 2], 4),
        "ms_per_step_min": round(per_step[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic (seeded N(0,1) keys/values and queries; no model weights)",
        "config": {"workload": f"config {args.config}: " + WORKLOADS[args.config] +
                   (", steady step (80/20 reuse)" if args.step == 1 else ", cold step (all miss)") +
                   (f", {args.volatile:.0%} volatile (layer, KV head) slots" if args.volatile else "") +
                   (", persistent heads from profiling" if plan else "") +
                   (f", {args.host_kv} host KV (power-of-two row scales)" if args.host_kv != "native" else "") +
                   (f", selection in blocks of {args.block_size} tokens, k={p.topk}" if args.block_size > 1 else "") +
                   (f", layer {args.layer} alone (single-layer fused step)" if args.layer is not None else ""),
                   "layers": n_layers, "batch": p.batch, "q_heads": p.hq, "kv_heads": p.hkv, "head_dim": HEAD_DIM,
                   "context": p.context, "topk": p.topk, "tau": p.tau, "step": args.step,
                   "data_layers": p.data_layers or p.layers, "host_memory": args.host_memory,
                   **({"graph": True} if args.graph else {}),
                   **({"step_schedule": "in order on one stream (--counters)"} if args.counters else {}),
                   **({"select_streams": args.select_streams, "select": loop.select,
                       **({"select_batches": list(loop.batches)} if loop.select == "batched" else {}),
                       "attend": loop.attend,
                       **({"attend_batches": list(loop.att_batches)} if loop.attend == "batched" else {})}
                      if multi else {})},
        "host_bound_ms": bounds["host_bound_ms"],
        "frac_of_host_bound": round(host_bound_ms / ms_per_step, 4) if host_bound_ms else None,
        "bounds": bounds,
        "roofline": roofline,
        "gather_schedule": gather_schedule,
        "persistent_plan": None if plan is None else {k: v for k, v in plan.items() if k != "persistent"},
        "block_size": args.block_size or 1,
        "blocks_vs_tokens": blocks,
        "host_kv": args.host_kv,
        "host_kv_vs_native": quant,
        "volatile_frac": args.volatile,
        "roofline_score": score_roofline(score_gbs, alg, args, multi, hbm_probe),
        # the loop's multi-layer selections alone: the same scoring bytes over their time
        "select_batched_gbs": (round(alg["score_bytes"] / (phases["select_batched"] / 1e3) / 1e9, 1)
                               if "select_batched" in phases else None),
        "attention_hbm_gbs": round(attn_gbs, 1),
        "attention_frac_measured": round(attn_gbs / hbm_probe["read_gbs"], 4) if hbm_probe else None,
        "step_hbm_gbs": round(alg["hbm_bytes"] / step_s / 1e9, 1),
        "step_host_gbs": round(alg["host_bytes"] / step_s / 1e9, 2),
        "phases_ms": {k: round(v, 4) for k, v in phases.items()},
        "units": {k: alg[k] for k in ("misses", "misses_persistent", "misses_host", "hits")},
        "host_link_probe": {k: round(v, 2) for k, v in probe.items()} if probe else None,
        "hbm_read_probe": ({"read_gbs": round(hbm_probe["read_gbs"], 1), "blocks": hbm_probe["blocks"],
                            "bytes": hbm_probe["bytes"]} if hbm_probe else None),
        "wall_s": round(wall, 3),
    }
    if multi:
        result["layer_steps_per_s"] = round(p.layers / step_s, 2)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of units")
        if args.host_kv != "native" or args.layer is not None:
            # the oracle reads stored rows of the step's dtype (the quantized host copy
            # holds none, so the native-format baseline is the one to compare with); a
            # single layer of a 48-layer workload is compared with in the full run
            result["cpu_baseline"] = None
        else:
            mk.push("cpu baseline")
            result["cpu_baseline"] = cpu_baseline(p, layers, args.cpu_sample_seconds, args.step,
                                                  full_step=not multi, one_thread=args.config in (1, 2))
            mk.pop()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
