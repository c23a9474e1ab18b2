"""Benchmark of the fused quantized linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch: for every linear of
the workload, LayerNorm + token-wise INT8 quantization (QKV and FFN1 inputs)
or plain token-wise quantization (attn-out and FFN2 inputs), then the INT8
GEMM with the fused dequant/bias(/GeLU) epilogue.  Default workload: the
GPT-NeoX-20B-shaped linears at 2048 tokens (prefill), hidden 6144, INT8
attention weights (QKV 18432x6144, out 6144x6144) and nibble-packed INT4
feed-forward weights (FFN1 24576x6144 with GeLU, FFN2 6144x24576), 128-row
weight groups: the largest of the five workloads that fits one GPU.  Its
activations follow the GPT-J recipe (0.5% outlier channels x30): its value
recipe is borrowed from another workload, and that reference is read as
counting workloads from zero.

Memory: R rotating sets of weights, inputs, intermediates and outputs (each
set one "layer") make the working set larger than twice the 256 MB Infinity
Cache, so every step reads its inputs from HBM.  Steps are replayed from HIP
graphs, one per set (the pages replay CUDA graphs for small models).

Prints one JSON line (stdout).  Details go to stderr.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0   # MI355X dense INT8 MFMA, 5.0 POP/s
FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, 2.5 PFLOP/s
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, 8 TB/s
METRIC = ("fused W8A8/W4A8 GEMM TOPS (% INT8 peak); decode GB/s (% HBM peak)")
ROTATE_BYTES = 600 * 2 ** 20   # > 2 x 256 MB Infinity Cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="neox-20b")
    ap.add_argument("--m-index", type=int, default=None,
                    help="which token count of the workload (default: largest)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU-oracle baseline")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode (GPT-J-6B, M=1) secondary figure")
    ap.add_argument("--no-fp16", action="store_true",
                    help="skip the fp16 torch.matmul comparator")
    ap.add_argument("--no-w8a16", action="store_true",
                    help="skip the W8A16 (fp16 activation) figure")
    ap.add_argument("--no-static", action="store_true",
                    help="skip the static per-tensor quantization comparator")
    ap.add_argument("--quant-on-load", action="store_true",
                    help="step: attn-out and FFN2 as quantize-on-load calls "
                         "(zq_gemm_*_xq) where they run as one kernel (one "
                         "token); with --summarize, summarize such a run")
    ap.add_argument("--chunked", action="store_true",
                    help="step (at most 16 tokens): the GEMMs on weights in "
                         "the chunk-contiguous decode layout (zq_pack_chunked, "
                         "zq_gemm_*_chunked); with --summarize, summarize "
                         "such a run")
    ap.add_argument("--no-xq", action="store_true",
                    help="skip the one-token quantize-on-load figure")
    ap.add_argument("--no-chain", action="store_true",
                    help="skip the layer-chain graph / schedule-table figure")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill GEMM figure of the larger workloads")
    ap.add_argument("--no-quantizers", action="store_true",
                    help="skip the row-quantizer figure of every workload")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles",
                                                      "traffic.json"))
    ap.add_argument("--only", default=None,
                    help="(profiling) run only the step loop, no extras")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="(profiling) first run a plain 256 MiB device copy "
                         "3 times, the reference for the HBM byte counters")
    ap.add_argument("--summarize", default=None, metavar="DIR",
                    help="summarize rocprofv3 CSV output in DIR (kernel trace "
                         "and/or --pmc FETCH_SIZE / WRITE_SIZE runs); no GPU")
    ap.add_argument("--write-traffic", default=None, metavar="JSON",
                    help="with --summarize: write the per-launch HBM traffic "
                         "of the GEMM and quantization kernels to JSON")
    return ap.parse_args()


# ------------------------------------------------------------------ setup --
class LinearSet:
    """Device buffers of one linear for one rotating set."""


def gemm_bytes(M, N, K, bits, G):
    return M * K + N * K * bits // 8 + 4 * (N // G) + 4 * M + 2 * N + 2 * M * N


def xq_bytes(M, N, K, bits, G):
    """The quantize-on-load linear: reads the fp16 activation (2MK) instead of
    codes and scales, and writes the codes (MK) and scales (4M) besides y."""
    return gemm_bytes(M, N, K, bits, G) + 2 * M * K


# the step's attn-out and FFN2 as quantize-on-load calls (--quant-on-load)
STEP_XQ = False


# the step's GEMMs on the chunk-contiguous decode layout (--chunked)
STEP_CHUNKED = False


def step_chunked(M):
    """Whether the step runs its GEMMs on the chunked decode layout."""
    return STEP_CHUNKED and M <= 16


def step_xq(zq, L, M):
    """Whether the step runs linear L as one quantize-on-load kernel."""
    return STEP_XQ and not L.ln and zq.gemm_xq_plan(
        M, L.N, L.K, L.bits).startswith("quantize-on-load")


def quant_bytes(M, K, ln=False):
    """Read x (2MK), write the codes (MK) and scales (4M); LayerNorm rows
    also read gamma and beta (4K)."""
    return 2 * M * K + M * K + 4 * M + (4 * K if ln else 0)


def pct_attainable(ops, nbytes, seconds):
    """Percent of the attainable roofline: min(INT8 MFMA peak, arithmetic
    intensity x HBM peak) for a GEMM, the HBM peak for a kernel with no
    contraction (ops = 0)."""
    if ops:
        att = min(INT8_PEAK_TOPS * 1e12, ops / nbytes * HBM_PEAK_GBS * 1e9)
        return round(100 * ops / seconds / att, 1)
    return round(100 * nbytes / seconds / (HBM_PEAK_GBS * 1e9), 1)


def build_sets(wl, M, dev, rotate_bytes):
    import torch
    import int4_quantized_transformer_amd as zq
    from int4_quantized_transformer_amd import workloads as W

    base = []
    for li, L in enumerate(wl.linears):
        w, b = W.gen_weights(wl, li)
        x = W.gen_activations(wl, li, M=M, m_index=list(wl.M).index(M))
        wd = w.to(dev)
        qw, sw = zq.quantize_weights(wd, wl.G, L.bits)
        del wd
        if step_chunked(M):
            qw = zq.pack_chunked(qw, L.bits)
        base.append(dict(L=L, x=x.to(dev), qw=qw, sw=sw, b=b.to(dev),
                         w_cpu=w, b_cpu=b, x_cpu=x))
    per_set = 0
    for d in base:
        L = d["L"]
        per_set += (d["qw"].numel() + d["x"].numel() * 2 + M * L.K
                    + 2 * M * L.N + 4 * M)
    R = max(1, -(-rotate_bytes // per_set))
    sets = []
    for r in range(R):
        lins = []
        for d in base:
            L = d["L"]
            s = LinearSet()
            s.L = L
            s.x = d["x"] if r == 0 else d["x"].clone()
            s.qw = d["qw"] if r == 0 else d["qw"].clone()
            s.sw = d["sw"] if r == 0 else d["sw"].clone()
            s.b = d["b"] if r == 0 else d["b"].clone()
            s.qx = torch.empty(M, L.K, dtype=torch.int8, device=dev)
            s.sx = torch.empty(M, dtype=torch.float32, device=dev)
            s.y = torch.empty(M, L.N, dtype=torch.float16, device=dev)
            lins.append(s)
        sets.append(lins)
    torch.cuda.synchronize()
    return base, sets, R, per_set


def clone_set(lins, M):
    """Another rotating set: copies of a set's inputs, weights and scales,
    and outputs of its own."""
    import torch
    out = []
    for d in lins:
        s = LinearSet()
        s.L = d.L
        s.x, s.qw, s.sw, s.b = d.x.clone(), d.qw.clone(), d.sw.clone(), d.b.clone()
        s.qx = torch.empty_like(d.qx)
        s.sx = torch.empty_like(d.sx)
        s.y = torch.empty_like(d.y)
        out.append(s)
    return out


ENTRY_MIN_SETS = 8


def make_step(zq, lins, wl, M, stream_ptr):
    """Pre-marshalled launches of one step: a list of (name, fn, args)."""
    import ctypes
    L_ = zq.lib()
    P = ctypes.c_void_p
    st = P(stream_ptr)
    calls = []
    for s in lins:
        L = s.L
        if step_xq(zq, L, M):
            fn = L_.zq_gemm_w8a8_xq if L.bits == 8 else L_.zq_gemm_w4a8_xq
            calls.append((f"{L.name}.gemm_w{L.bits}a8_xq", fn,
                          (P(s.x.data_ptr()), P(s.qw.data_ptr()),
                           P(s.sw.data_ptr()), wl.G, P(s.b.data_ptr()),
                           int(L.gelu), M, L.N, L.K, P(s.y.data_ptr()),
                           P(s.qx.data_ptr()), P(s.sx.data_ptr()), st)))
            continue
        if L.ln:
            calls.append((f"{L.name}.ln_quant", L_.zq_ln_quant_act,
                          (P(s.x.data_ptr()), None, None,
                           ctypes.c_float(wl.ln_eps), M, L.K,
                           P(s.qx.data_ptr()), P(s.sx.data_ptr()), None, st)))
        else:
            calls.append((f"{L.name}.quant", L_.zq_quant_act,
                          (P(s.x.data_ptr()), M, L.K, P(s.qx.data_ptr()),
                           P(s.sx.data_ptr()), st)))
        if step_chunked(M):
            fn = (L_.zq_gemm_w8a8_chunked if L.bits == 8
                  else L_.zq_gemm_w4a8_chunked)
        else:
            fn = L_.zq_gemm_w8a8 if L.bits == 8 else L_.zq_gemm_w4a8
        calls.append((f"{L.name}.gemm_w{L.bits}a8", fn,
                      (P(s.qx.data_ptr()), P(s.sx.data_ptr()),
                       P(s.qw.data_ptr()), P(s.sw.data_ptr()), wl.G,
                       P(s.b.data_ptr()), int(L.gelu), M, L.N, L.K,
                       P(s.y.data_ptr()), st)))
    return calls


def make_chain(zq, lins, wl, M):
    """The same step as a chain of the library's own executor (zq_chain),
    whose eager run launches the calls from native code."""
    c = zq.Chain(M)
    for s in lins:
        L = s.L
        if step_xq(zq, L, M):
            c.gemm_xq(s.x, s.qw, s.sw, wl.G, s.y, s.qx, s.sx, s.b, int(L.gelu))
            continue
        if L.ln:
            c.ln_quant(s.x, s.qx, s.sx, None, None, wl.ln_eps)
        else:
            c.quant(s.x, s.qx, s.sx)
        if step_chunked(M):
            c.gemm_chunked(s.qx, s.sx, s.qw, s.sw, wl.G, s.y, s.b, int(L.gelu))
        else:
            c.gemm(s.qx, s.sx, s.qw, s.sw, wl.G, s.y, s.b, int(L.gelu))
    return c


def timed_native(torch, chains, M, steps, stream):
    """Exactly `steps` steps launched one call at a time from native code
    (zq_chain_run_eager over the rotating sets); events around them."""
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        chains[i % len(chains)].run_eager(M, stream=stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall * 1e3 / steps


def run_calls(calls):
    for name, fn, args in calls:
        rc = fn(*args)
        if rc != 0:
            raise RuntimeError(f"{name} failed with status {rc}")


def kernel_work(name, L, M, G):
    """(ops, bytes, bound) of one launch."""
    if name.endswith("_xq"):
        return (2 * M * L.N * L.K, xq_bytes(M, L.N, L.K, L.bits, G), "mfma")
    if ".gemm" in name:
        return (2 * M * L.N * L.K, gemm_bytes(M, L.N, L.K, L.bits, G), "mfma")
    return (0, quant_bytes(M, L.K, L.ln), "hbm")


# ------------------------------------------------------------- CPU oracle --
def cpu_baseline(base, wl, M, target_s=12.0):
    """The CPU oracle, untuned, on a bounded sample of the same step."""
    import oracle
    ops_per_token = sum(2 * d["L"].N * d["L"].K for d in base)
    prepared = []
    for d in base:
        q, sw = oracle.quantize_weights(d["w_cpu"].numpy(), wl.G, d["L"].bits)
        prepared.append((d, q, sw))

    def run(S):
        t0 = time.perf_counter()
        for d, q, sw in prepared:
            L = d["L"]
            oracle.linear(d["x_cpu"].numpy()[:S], q, sw, wl.G,
                          d["b_cpu"].numpy(), int(L.gelu), ln=L.ln,
                          eps=wl.ln_eps)
        return time.perf_counter() - t0

    S = min(M, 64)
    t = run(S)
    S = int(min(M, max(S, S * target_s / max(t, 1e-3))))
    t = run(S)
    tops = ops_per_token * S / t / 1e12
    threads = oracle.threads()
    # once more on one thread, over a sample sized for about a third of the
    # time above
    S1 = max(16, min(S, int(S / threads / 3)))
    oracle.set_threads(1)
    try:
        t1 = run(S1)
    finally:
        oracle.set_threads(threads)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f
                          if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(tops, 6), "unit": "TOPS", "cores": threads,
            "kind": "oracle",
            "sample": (f"first {S} of {M} tokens through all {len(base)} "
                       f"linears (LN/quant, int64 GEMM, fp64 epilogue); "
                       f"{t:.1f} s"),
            "single_thread": {"value": round(ops_per_token * S1 / t1 / 1e12, 6),
                              "sample": f"first {S1} tokens; {t1:.1f} s"},
            "host": {"cpu": model, "nproc": os.cpu_count()}}


# ----------------------------------------------------------------- timing --
def timed_graphs(torch, graphs, steps, stream):
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall * 1e3 / steps


def timed_steps(torch, g_all, R, graphs, steps, stream):
    """Exactly `steps` steps: steps // R replays of the graph holding all R
    rotating steps, then the remaining steps from the one-step graphs;
    events around them on the replay stream."""
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps // R):
        g_all.replay()
    for i in range(steps % R):
        graphs[i].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall * 1e3 / steps


def timed_eager(torch, step_calls, steps, stream):
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        run_calls(step_calls[i % len(step_calls)])
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def replay_percentiles(torch, g, n, stream, per):
    """p10 / p50 / p90 over n replays of graph g, each between its own pair
    of events, divided by the `per` launches a replay holds (ms)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(n):
        g.replay()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(evs[i].elapsed_time(evs[i + 1]) / per for i in range(n))
    return [ts[min(n - 1, int(f * n))] for f in (0.1, 0.5, 0.9)]


def entry_timings(torch, zq, sets, wl, M, steps):
    """Average duration of each step entry's launch: one HIP graph per entry
    holding that launch for every rotating set (so its inputs come from HBM
    as in the step), replayed `steps` times and timed with events around
    the replays.  The sets are topped up with copies to ENTRY_MIN_SETS, so
    that a replay's own launch cost is spread over that many launches (with
    one launch per graph it added about 5 us to each, a third of a
    quantizer launch); graph launches carry no host gaps, so this is the
    kernel's own duration plus the small inter-kernel gap of a graph.  Also
    returns p10 / p50 / p90 of the per-launch time over separately timed
    replays."""
    sets = list(sets)
    while len(sets) < ENTRY_MIN_SETS:
        sets.append(clone_set(sets[0], M))
    names = [c[0] for c in make_step(zq, sets[0], wl, M, 0)]
    out, pct = {}, {}
    for j, name in enumerate(names):
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cs):
            for s in sets:
                call = make_step(zq, s, wl, M, cs.cuda_stream)[j]
                run_calls([call])
        stream = torch.cuda.current_stream()
        for _ in range(3):
            g.replay()
        ms, _ = timed_graphs(torch, [g], steps, stream)
        out[name] = ms / len(sets)
        pct[name] = replay_percentiles(torch, g, steps, stream, len(sets))
        del g
    return out, pct


def grid_threads(name, L, M, G, zq):
    """Launch grid (threads) of the kernel behind a step entry, as the
    kernel trace reports it (used to find that launch in rocprofv3 output)."""
    plan = zq.gemm_plan(M, L.N, L.K, L.bits) if ".gemm" in name else ""
    if ".gemm" in name and step_chunked(M):
        plan = zq.gemm_chunked_plan(M, L.N, L.K, L.bits).replace("chunked ", "")
    if name.endswith("_xq"):
        plan = zq.gemm_xq_plan(M, L.N, L.K, L.bits).replace(
            "quantize-on-load ", "")
    if plan.startswith("gemv") or plan.startswith("stream"):
        return int(plan.split("grid=")[1].split()[0]) * 64 * \
            int(plan.split("NW=")[1].split()[0])
    if plan.startswith("tiled"):
        # workgroups: one per tile, or (persistent kernel) the grid it reports
        wgs = int(plan.split("grid=")[1].split()[0]) if "grid=" in plan else \
            int(plan.split("tiles=")[1].split()[0])
        nt = 64 * (int(plan.split("BN=")[1].split()[0]) // int(plan.split("WN=")[1].split()[0])) \
            * (int(plan.split("BM=")[1].split()[0]) // int(plan.split("WM=")[1].split()[0]))
        return wgs * nt
    return None


KERNEL_SOURCES = ("zq_gemm.hip", "zq_quant.hip", "zq_index.h", "zq_internal.h")


def source_shas():
    out = {}
    for n in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "int4_quantized_transformer_amd", "csrc",
                               n), "rb") as f:
            out[n] = hashlib.sha256(f.read()).hexdigest()
    return out


def traffic_for(path, step, entry, grid):
    """HBM bytes per launch of one step entry ("<workload> M=<tokens>",
    entry name) from committed rocprofv3 counter runs, or None if absent,
    taken on other kernel sources, or on another launch grid."""
    try:
        with open(path) as f:
            t = json.load(f)
        shas = source_shas()
    except (OSError, ValueError):
        return None
    e = t.get("steps", {}).get(step, {}).get(entry)
    if not e or t.get("sources") != shas or e.get("grid") != grid:
        return None
    return e.get("hbm_bytes_per_launch")


def step_entries(zq, wl, M):
    """The launches of one step, in order: name, kernel, grid (threads; GEMMs
    only), algorithmic ops and bytes."""
    out = []
    for L in wl.linears:
        if step_xq(zq, L, M):
            gn = f"{L.name}.gemm_w{L.bits}a8_xq"
            ops = 2 * M * L.N * L.K
            nbytes = xq_bytes(M, L.N, L.K, L.bits, wl.G)
            xplan = zq.gemm_xq_plan(M, L.N, L.K, L.bits)
            out.append({"name": gn, "kernel": "gemm_gemv_kernel",
                        "grid": grid_threads(gn, L, M, wl.G, zq),
                        "block": 64 * int(xplan.split("NW=")[1].split()[0]),
                        "ops": ops, "bytes": nbytes,
                        "read_bytes": nbytes - 2 * M * L.N - M * L.K - 4 * M,
                        "roof_s": max(ops / (INT8_PEAK_TOPS * 1e12),
                                      nbytes / (HBM_PEAK_GBS * 1e9))})
            continue
        qn = f"{L.name}.ln_quant" if L.ln else f"{L.name}.quant"
        out.append({"name": qn, "kernel": "row_quant_kernel", "grid": None,
                    "ops": 0, "bytes": quant_bytes(M, L.K, L.ln)})
        gn = f"{L.name}.gemm_w{L.bits}a8"
        plan = zq.gemm_plan(M, L.N, L.K, L.bits)
        if step_chunked(M):
            plan = zq.gemm_chunked_plan(M, L.N, L.K, L.bits).replace(
                "chunked ", "")
        kern = {"tiled": "gemm_tiled_kernel", "stream": "gemm_stream_kernel",
                "gemv": "gemm_gemv_kernel", "skinny": "gemm_skinny_kernel"}[
                    plan.split()[0]]
        if step_chunked(M) and plan.startswith("gemv"):
            kern = "gemm_chunk_gemv_kernel"
        if "ping-pong" in plan:
            kern = "gemm_pingpong_kernel"
        ops = 2 * M * L.N * L.K
        nbytes = gemm_bytes(M, L.N, L.K, L.bits, wl.G)
        out.append({"name": gn, "kernel": kern,
                    "grid": grid_threads(gn, L, M, wl.G, zq),
                    "block": 64 * int(plan.split("NW=")[1].split()[0])
                    if plan.startswith("gemv") else None,
                    "ops": ops, "bytes": nbytes,
                    "read_bytes": nbytes - 2 * M * L.N,
                    # roofline time: what orders the durations of launches
                    # that share a kernel and grid (ops at prefill, bytes at
                    # decode)
                    "roof_s": max(ops / (INT8_PEAK_TOPS * 1e12),
                                  nbytes / (HBM_PEAK_GBS * 1e9))})
    return out


# ----------------------------------------------------- fp16 comparator --
def fp16_linear_us(torch, dev, wl, li, M, steps=20):
    """torch fp16 addmm + bias (+ GeLU) of linear `li` of `wl` at M tokens,
    with fp16 weights (run as a library, never inspected): the average
    launch from a CUDA graph holding one call per rotating weight copy, the
    copies together larger than twice the Infinity Cache, as for the INT8
    kernels."""
    from int4_quantized_transformer_amd import workloads as W
    L = wl.linears[li]
    w, b = W.gen_weights(wl, li)
    wd, bd = w.to(dev), b.to(dev)
    x = W.gen_activations(wl, li, M=M, m_index=list(wl.M).index(M)).to(dev)
    R = max(1, -(-ROTATE_BYTES // (2 * L.N * L.K)))
    ws = [wd] + [wd.clone() for _ in range(R - 1)]
    y = torch.empty(M, L.N, dtype=torch.float16, device=dev)

    def run():
        for w_ in ws:
            torch.addmm(bd, x, w_.t(), out=y)
            if L.gelu:
                torch.nn.functional.gelu(y)

    stream = torch.cuda.current_stream()
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cs):
        run()
    g.replay()
    ms, _ = timed_graphs(torch, [g], steps, stream)
    del g, ws, wd
    torch.cuda.empty_cache()
    return ms * 1e3 / R


# ------------------------------------------------------------------ decode --
def decode_case(torch, zq, dev, name, M, steps=100, with_fp16=True,
                chunked=False):
    """One decoder layer's four linears at decode-sized M: GEMM GB/s against
    HBM for the layer (graph replay of the four launches over rotating
    weight sets larger than the Infinity Cache) and per linear.  chunked:
    the weights repacked into the chunk-contiguous decode layout and the
    _chunked calls (no fp16 comparator)."""
    from int4_quantized_transformer_amd import workloads as W
    wl = W.workload(name)
    mi = list(wl.M).index(M)
    lin = []
    for li, L in enumerate(wl.linears):
        w, b = W.gen_weights(wl, li)
        x = W.gen_activations(wl, li, m_index=mi)
        qw, sw = zq.quantize_weights(w.to(dev), wl.G, L.bits)
        if chunked:
            qw = zq.pack_chunked(qw, L.bits)
        qx, sx = zq.quant_act(x.to(dev))
        lin.append((L, qx, sx, qw, sw, b.to(dev)))
        del w
    wbytes = sum(l[3].numel() for l in lin)
    # at least ENTRY_MIN_SETS sets, so that a graph of one linear's launches
    # spreads its own launch cost over as many kernels
    R = max(ENTRY_MIN_SETS, -(-ROTATE_BYTES // wbytes))
    sets = [lin] + [[(L, qx, sx, qw.clone(), sw, b) for (L, qx, sx, qw, sw, b)
                     in lin] for _ in range(R - 1)]
    ys = [torch.empty(M, l[0].N, dtype=torch.float16, device=dev) for l in lin]
    # the calls with a workspace (decode-sized M over few weight tiles splits
    # K); one workspace per linear, reused by every rotating set
    wss = []
    for (L, *_r) in lin:
        need = zq.gemm_workspace_bytes(M, L.N, L.K, L.bits)
        wss.append(torch.empty(need, dtype=torch.uint8, device=dev) if need else None)
    wsidx = {id(y): i for i, y in enumerate(ys)}

    def call(entry, y):
        L, qx, sx, qw, sw, b = entry
        if chunked:
            g = zq.gemm_w8a8_chunked if L.bits == 8 else zq.gemm_w4a8_chunked
            g(qx, sx, qw, sw, wl.G, b, int(L.gelu), y=y)
            return
        g = zq.gemm_w8a8_ws if L.bits == 8 else zq.gemm_w4a8_ws
        g(qx, sx, qw, sw, wl.G, b, int(L.gelu), y=y, ws=wss[wsidx[id(y)]])

    def graph(which):
        # every rotating set in one graph (consecutive layers, each with its
        # own weights)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for s_ in sets:
                for i in which:
                    call(s_[i], ys[i])
        return gr

    stream = torch.cuda.current_stream()
    for i in range(2 * R):
        for e, y in zip(sets[i % R], ys):
            call(e, y)
    ms_g, _ = timed_graphs(torch, [graph(range(4))], steps, stream)
    ms_g /= R
    # the same launches from native code (the library's chain executor)
    chains = []
    for s_ in sets:
        c = zq.Chain(M)
        for (L, qx, sx, qw, sw, b), y, ws in zip(s_, ys, wss):
            if chunked:
                c.gemm_chunked(qx, sx, qw, sw, wl.G, y, b, int(L.gelu))
            else:
                c.gemm_ws(qx, sx, qw, sw, wl.G, y, ws, b, int(L.gelu))
        chains.append(c)
    for c in chains:
        c.run_eager(M, stream=stream.cuda_stream)
    ms_n, _ = timed_native(torch, chains, M, steps * R, stream)
    by_launch = {"graph": round(ms_g * 1e3, 2),
                 "native_eager": round(ms_n * 1e3, 2)}
    ms = min(ms_g, ms_n)
    nbytes = sum(gemm_bytes(M, L.N, L.K, L.bits, wl.G) for (L, *_r) in lin)
    gbs = nbytes / (ms * 1e-3) / 1e9
    per = {}
    for i, (L, *_r) in enumerate(lin):
        mi_, _ = timed_graphs(torch, [graph([i])], steps, stream)
        mi_ /= R
        b_ = gemm_bytes(M, L.N, L.K, L.bits, wl.G)
        per[f"{L.name} W{L.bits}"] = {
            "us": round(mi_ * 1e3, 2),
            "GB_per_s": round(b_ / (mi_ * 1e-3) / 1e9, 1),
            "pct_attainable": pct_attainable(2 * M * L.N * L.K, b_, mi_ * 1e-3),
            "plan": (zq.gemm_chunked_plan(M, L.N, L.K, L.bits) if chunked
                     else zq.gemm_ws_plan(M, L.N, L.K, L.bits)).split(" W")[0],
            "bytes": b_}
    del sets, chains
    torch.cuda.empty_cache()
    fp16 = {}
    if with_fp16 and not chunked:
        for i, (L, *_r) in enumerate(lin):
            fp16[f"{L.name}"] = round(fp16_linear_us(torch, dev, wl, i, M,
                                                     steps // 4 or 1), 2)
        fp16["layer"] = round(sum(fp16.values()), 2)
    out = {"GB_per_s": round(gbs, 1),
           "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
           "us_per_step": round(ms * 1e3, 2), "us_by_launch": by_launch,
           "bytes_per_step": nbytes, "rotating_sets": R, "per_linear": per}
    if fp16:
        out["torch_fp16_us"] = fp16
        out["speedup_vs_fp16"] = round(fp16["layer"] / (ms * 1e3), 2)
    return out


def decode_figure(torch, zq, dev, steps=100, with_fp16=True):
    """Decoder linears at decode-sized M (QKV, out, FFN1+GeLU, FFN2): GPT-J-6B
    (W8A8, 128-row groups) at M = 1, 16 and 64, and GPT-NeoX-20B (W8 attention,
    W4 FFN) at M = 1 and 16; GEMM GB/s against 8 TB/s."""
    out = {"workload": "decoder linears (QKV, out, FFN1+GeLU, FFN2), "
                       "one HIP graph over all rotating weight sets (as "
                       "consecutive layers); bytes = the GEMMs' algorithmic "
                       "bytes"}
    for name, ms in (("gptj-6b", (1, 16, 64)), ("neox-20b", (1, 16))):
        for M in ms:
            out[f"{name} M={M}"] = decode_case(torch, zq, dev, name, M, steps,
                                               with_fp16)
            torch.cuda.empty_cache()
    # the same layers with the weights in the chunk-contiguous decode layout
    # (zq_pack_chunked): the rings at 16 tokens, the chunked GEMV at one
    for name in ("gptj-6b", "neox-20b"):
        for M in (1, 16):
            out[f"{name} M={M} chunked"] = decode_case(
                torch, zq, dev, name, M, steps, False, chunked=True)
            torch.cuda.empty_cache()
    return out


def xq_figure(torch, zq, dev, steps=20):
    """The linears whose input is not LayerNorm'd (attn-out, FFN2) at one
    token: the quantizer launch followed by the GEMM against the
    quantize-on-load call (one kernel: the GEMV quantizes the fp16 row as it
    stages it), both in one HIP graph over rotating weight sets, the same
    fp16 input, bias, y, codes and scales."""
    from int4_quantized_transformer_amd import workloads as W
    out = {"workload": "GPT-J-6B and GPT-NeoX-20B attn-out and FFN2 at one "
                       "token; input = the linear's fp16 activation"}
    stream = torch.cuda.current_stream()
    saved = 0.0
    for name in ("gptj-6b", "neox-20b"):
        wl = W.workload(name)
        for li, L in enumerate(wl.linears):
            if L.name not in ("attn_out", "ffn2"):
                continue
            w, b = W.gen_weights(wl, li)
            qw, sw = zq.quantize_weights(w.to(dev), wl.G, L.bits)
            del w
            x = W.gen_activations(wl, li, m_index=list(wl.M).index(1)).to(dev)
            qx, sx = zq.quant_act(x)
            R = max(2, -(-ROTATE_BYTES // qw.numel()))
            qws = [qw] + [qw.clone() for _ in range(R - 1)]
            y = torch.empty(1, L.N, dtype=torch.float16, device=dev)
            bd = b.to(dev)
            g8 = zq.gemm_w8a8 if L.bits == 8 else zq.gemm_w4a8
            gx = zq.gemm_w8a8_xq if L.bits == 8 else zq.gemm_w4a8_xq

            def two():
                for w_ in qws:
                    zq.quant_act(x, qx=qx, sx=sx)
                    g8(qx, sx, w_, sw, wl.G, bd, 0, y=y)

            def one():
                for w_ in qws:
                    gx(x, w_, sw, wl.G, bd, 0, y=y, qx=qx, sx=sx)

            us = {}
            for key, fn in (("quant_then_gemm", two), ("quantize_on_load", one)):
                fn()
                torch.cuda.synchronize()
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    fn()
                ms, _ = timed_graphs(torch, [gr], steps, stream)
                us[key] = round(ms * 1e3 / R, 2)
                del gr
            b_ = gemm_bytes(1, L.N, L.K, L.bits, wl.G)
            us["GB_per_s_quantize_on_load"] = round(
                b_ / (us["quantize_on_load"] * 1e-6) / 1e9, 1)
            us["plan"] = zq.gemm_xq_plan(1, L.N, L.K, L.bits).split(" NW")[0]
            out[f"{name} {L.name} W{L.bits}"] = us
            saved += us["quant_then_gemm"] - us["quantize_on_load"]
            del qws
            torch.cuda.empty_cache()
    out["us_saved_total"] = round(saved, 2)
    return out


def quantizer_figure(torch, zq, dev, steps=20):
    """The row quantizers at every workload's token counts: LayerNorm +
    quantization (QKV / FFN1 inputs, affine gamma / beta) and quantization
    alone (attn-out / FFN2 inputs), each from one HIP graph over rotating
    inputs, against torch's fp16 -> int8 cast of the same tensor, which
    reads and writes the same bytes (2MK, MK) with no arithmetic to speak
    of: the cost of moving them with a library elementwise kernel."""
    from int4_quantized_transformer_amd import workloads as W
    out = {"note": "us per launch (graph over rotating inputs; decode-sized "
                   "rows are launch-bound, at most 64 input copies); "
                   "GB_per_s = algorithmic bytes (2MK read + MK + 4M "
                   "written, + 4K gamma/beta with LN) / time; torch_cast = "
                   "int8 tensor .copy_(fp16 tensor) of the same shape"}
    stream = torch.cuda.current_stream()
    for wl in W.WORKLOADS:
        seen = set()
        for mi, M in enumerate(wl.M):
            for li, L in enumerate(wl.linears):
                key = (M, L.K, L.ln)
                if key in seen:
                    continue
                seen.add(key)
                x = W.gen_activations(wl, li, m_index=mi).to(dev)
                nb = quant_bytes(M, L.K, L.ln)
                R = min(64, max(8, -(-ROTATE_BYTES // (3 * M * L.K))))
                xs = [x] + [x.clone() for _ in range(R - 1)]
                qx = torch.empty(M, L.K, dtype=torch.int8, device=dev)
                sx = torch.empty(M, dtype=torch.float32, device=dev)
                gam = torch.ones(L.K, dtype=torch.float16, device=dev)
                bet = torch.zeros(L.K, dtype=torch.float16, device=dev)
                qc = torch.empty(M, L.K, dtype=torch.int8, device=dev)

                def zq_call():
                    for x_ in xs:
                        if L.ln:
                            zq.ln_quant_act(x_, gam, bet, wl.ln_eps, qx=qx,
                                            sx=sx)
                        else:
                            zq.quant_act(x_, qx=qx, sx=sx)

                def cast():
                    for x_ in xs:
                        qc.copy_(x_)

                us = {}
                for name, fn in (("us", zq_call), ("torch_cast_us", cast)):
                    fn()
                    torch.cuda.synchronize()
                    gr = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(gr):
                        fn()
                    ms, _ = timed_graphs(torch, [gr], steps, stream)
                    us[name] = round(ms * 1e3 / R, 2)
                    del gr
                kind = "ln_quant" if L.ln else "quant"
                out[f"{wl.name} {kind} {M}x{L.K}"] = {
                    "us": us["us"],
                    "GB_per_s": round(nb / (us["us"] * 1e-6) / 1e9, 1),
                    "pct_hbm_peak": pct_attainable(0, nb, us["us"] * 1e-6),
                    "torch_cast_us": us["torch_cast_us"],
                    "vs_torch_cast": round(us["torch_cast_us"] / us["us"], 2),
                }
                del xs, x
                torch.cuda.empty_cache()
    return out


def prefill_figure(torch, zq, dev, steps=20):
    """Fused W8A8 / W4A8 GEMMs at the prefill token counts of the other
    large workloads (BERT-large 8192 tokens with W4 FFN, GPT-J-6B 2048; the
    GPT-NeoX-20B step is the headline): per linear, the average launch from
    a graph holding it for every rotating set, TOPS and % of the 5.0 POP/s
    INT8 peak, beside the torch fp16 matmul of the same shape."""
    from int4_quantized_transformer_amd import workloads as W
    stream = torch.cuda.current_stream()
    out = {"note": "GEMM with the fused epilogue only (inputs already "
                   "quantized); one graph per linear over rotating sets"}
    for name, M in (("bert-large", 8192), ("gptj-6b", 2048)):
        wl = W.workload(name)
        mi = list(wl.M).index(M)
        res = {}
        tot_ops = tot_us = tot_f16 = 0.0
        for li, L in enumerate(wl.linears):
            w, b = W.gen_weights(wl, li)
            qw, sw = zq.quantize_weights(w.to(dev), wl.G, L.bits)
            del w
            qx, sx = zq.quant_act(W.gen_activations(wl, li, m_index=mi).to(dev))
            per = qw.numel() + qx.numel() + 2 * M * L.N
            R = max(2, -(-ROTATE_BYTES // per))
            sets = [(qx, sx, qw, b.to(dev))] + [
                (qx.clone(), sx.clone(), qw.clone(), b.to(dev)) for _ in range(R - 1)]
            y = torch.empty(M, L.N, dtype=torch.float16, device=dev)
            g8 = zq.gemm_w8a8 if L.bits == 8 else zq.gemm_w4a8
            for (a_, s_, w_, b_) in sets:
                g8(a_, s_, w_, sw, wl.G, b_, int(L.gelu), y=y)
            gr = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            with torch.cuda.graph(gr, stream=cs):
                for (a_, s_, w_, b_) in sets:
                    g8(a_, s_, w_, sw, wl.G, b_, int(L.gelu), y=y)
            gr.replay()
            ms, _ = timed_graphs(torch, [gr], steps, stream)
            us = ms * 1e3 / R
            ops = 2.0 * M * L.N * L.K
            tops = ops / (us * 1e-6) / 1e12
            res[f"{L.name} {L.N}x{L.K} W{L.bits}"] = {
                "us": round(us, 2), "TOPS": round(tops, 1),
                "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 1),
                "pct_attainable": pct_attainable(
                    ops, gemm_bytes(M, L.N, L.K, L.bits, wl.G), us * 1e-6),
                "plan": zq.gemm_plan(M, L.N, L.K, L.bits).split(" W")[0]}
            tot_ops += ops
            tot_us += us
            del sets, gr, y
            torch.cuda.empty_cache()
            f16 = fp16_linear_us(torch, dev, wl, li, M, steps)
            e = res[f"{L.name} {L.N}x{L.K} W{L.bits}"]
            e["torch_fp16_us"] = round(f16, 2)
            e["speedup_vs_fp16"] = round(f16 / us, 2)
            tot_f16 += f16
        tops = tot_ops / (tot_us * 1e-6) / 1e12
        res["all four"] = {"TOPS": round(tops, 1),
                           "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 1),
                           "torch_fp16_TFLOPS": round(tot_ops / (tot_f16 * 1e-6) / 1e12, 1),
                           "speedup_vs_fp16": round(tot_f16 / tot_us, 2)}
        out[f"{name} M={M}"] = res
    return out


def w8a16_figure(torch, zq, dev, steps=20):
    """GPT-NeoX20B QKV (18432 x 6144) with INT8 weights and fp16 activations
    (the pages' W8A8/16 scheme keeps NeoX's attention inputs in fp16), at
    prefill (M = 2048: TFLOP/s against the fp16 MFMA peak) and decode (M = 16
    and 1: GB/s against HBM); the torch fp16 matmul of the same shape beside
    it."""
    from int4_quantized_transformer_amd import workloads as W
    wl = W.workload("neox-20b")
    L = wl.linears[0]
    N, K, G = L.N, L.K, wl.G
    w, b = W.gen_weights(wl, 0)
    wd = w.to(dev)
    qw, sw = zq.quantize_weights(wd, G, 8)
    bd = b.to(dev)
    R = max(2, -(-ROTATE_BYTES // (N * K)))
    qws = [qw] + [qw.clone() for _ in range(R - 1)]
    out = {"workload": f"neox-20b QKV {N}x{K} W8A16, {G}-row groups, "
                       "HIP-graph replay over rotating weight sets"}
    for M in (2048, 16, 1):
        x = W.gen_activations(wl, 0, M=M, m_index=list(wl.M).index(M)).to(dev)
        y = torch.empty(M, N, dtype=torch.float16, device=dev)
        for i in range(R):
            zq.gemm_w8a16(x, qws[i], sw, G, bd, 0, y=y)
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cs):
            for i in range(R):
                zq.gemm_w8a16(x, qws[i], sw, G, bd, 0, y=y)
        stream = torch.cuda.current_stream()
        g.replay()
        ms, _ = timed_graphs(torch, [g], steps, stream)
        us = ms * 1e3 / R
        nbytes = N * K + 2 * M * K + 2 * M * N + 4 * (N // G) + 2 * N
        e = {"us": round(us, 2), "plan": zq.gemm_w8a16_plan(M, N, K)}
        if M > 64:
            tf = 2 * M * N * K / (us * 1e-6) / 1e12
            e["TFLOPS"] = round(tf, 1)
            e["pct_fp16_peak"] = round(100 * tf / FP16_PEAK_TFLOPS, 1)
        else:
            gbs = nbytes / (us * 1e-6) / 1e9
            e["GB_per_s"] = round(gbs, 1)
            e["pct_hbm_peak"] = round(100 * gbs / HBM_PEAK_GBS, 1)
        # torch fp16 matmul + bias at the same shape (fp16 weights)
        ws16 = [wd] + [wd.clone() for _ in range(max(1, R // 2) - 1)]
        R2 = len(ws16)
        for i in range(R2):
            torch.addmm(bd, x, ws16[i].t())
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps * R2):
            torch.addmm(bd, x, ws16[i % R2].t())
        e1.record(stream)
        torch.cuda.synchronize()
        e["torch_fp16_us"] = round(e0.elapsed_time(e1) * 1e3 / (steps * R2), 2)
        out[f"M={M}"] = e
        del ws16, g
    return out


def static_figure(torch, zq, dev, batches=100, steps=50):
    """Static per-tensor vs token-wise INT8 activations on the BERT-base FFN1
    linear (4096 tokens x 768 -> 3072, W8 weights): the range is calibrated
    as a moving average over `batches` seeded synthetic batches, then a
    held-out batch goes through both quantizers and the same INT8 GEMM; the
    relative RMS error of each output against the fp32 product, and the
    static quantizer's own bandwidth."""
    from int4_quantized_transformer_amd import workloads as W
    wl = W.workload("bert-base")
    L = wl.linears[2]
    M, K, N = 4096, L.K, L.N

    oc = W.outlier_channels(wl, 2)

    def batch(seed):
        # N(0,1) tokens with the workload's outlier channels scaled, each
        # token's range multiplied by a log-uniform factor in [1, 4]
        g = torch.Generator().manual_seed(seed)
        x = torch.randn(M, K, generator=g)
        x[:, oc] *= wl.outlier_factor
        x *= torch.exp(torch.rand(M, 1, generator=g) * math.log(4.0))
        return x.half().to(dev)

    st = None
    for i in range(batches):
        st = zq.calibrate_minmax(batch(1000 + i), st)
    x = batch(7)
    w, b = W.gen_weights(wl, 2)
    wd, bd = w.to(dev), b.to(dev)
    qw, sw = zq.quantize_weights(wd, wl.G, 8)
    ref = torch.addmm(bd.float(), x.float(), wd.float().t())
    qt, sxt = zq.quant_act(x)
    yt = zq.gemm_w8a8(qt, sxt, qw, sw, wl.G, bd, 0).float()
    qs, s = zq.quant_act_static(x, st)
    ys = zq.gemm_w8a8(qs, s.expand(M).contiguous(), qw, sw, wl.G, bd, 0).float()
    rel = lambda y: float(torch.linalg.norm(y - ref) / torch.linalg.norm(ref))
    xq_t = (qt.float() * sxt[:, None]).sub(x.float()).pow(2).mean().sqrt()
    xq_s = (qs.float() * s).sub(x.float()).pow(2).mean().sqrt()
    # static quantizer bandwidth (inputs rotated past the Infinity Cache)
    R = max(2, -(-ROTATE_BYTES // (3 * M * K)))
    xs = [x] + [x.clone() for _ in range(R - 1)]
    q = torch.empty_like(qs)
    so = torch.empty(1, dtype=torch.float32, device=dev)
    st_ = torch.empty(M, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    times = {}
    for name, call in (("static", lambda i: zq.quant_act_static(xs[i], st, qx=q,
                                                                s_out=so)),
                       ("token_wise", lambda i: zq.quant_act(xs[i], qx=q, sx=st_))):
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cs):
            for i in range(R):
                call(i)
        g.replay()
        ms, _ = timed_graphs(torch, [g], steps, stream)
        times[name] = ms * 1e3 / R
        del g
    us = times["static"]
    return {"workload": "bert-base FFN1 input 4096x768 (outlier channels, token "
                        "ranges varying up to 4x), W8 FFN1 weights; range "
                        f"calibrated over {batches} batches, momentum 0.95",
            "rel_rms_error_output": {"token_wise": round(rel(yt), 5),
                                     "static_per_tensor": round(rel(ys), 5)},
            "rms_error_activations": {"token_wise": round(float(xq_t), 5),
                                      "static_per_tensor": round(float(xq_s), 5)},
            "static_quant_us": round(us, 2),
            "static_quant_GB_per_s": round(3 * M * K / (us * 1e-6) / 1e9, 1),
            "token_wise_quant_us": round(times["token_wise"], 2)}


def chain_figure(torch, zq, dev, steps=50, reps=20):
    """Encoder layers' linear chains (per layer: LN+quant -> QKV, quant ->
    attention output, LN+quant -> FFN1 with quantized output -> FFN2, seven
    launches) launched one call at a time from native code, replayed as one
    HIP graph per token count, and replayed again after tuning the schedule
    table at those token counts: a 12-layer BERT-base stack at seq 128 with
    batch 1, 16 and 128 (the pages' Table 6 shapes), one BERT-base layer,
    and a 4-layer GPT-J decode stack, also with attn-out and FFN2 as
    quantize-on-load calls (six launches per layer; one kernel each at one
    token).  Times are per stack, from events
    around `steps` back-to-back runs (so launch gaps count), with the host
    time per run beside them."""
    from int4_quantized_transformer_amd import workloads as W
    stream = torch.cuda.current_stream()

    def per_run_us(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        host = (time.perf_counter() - t0) * 1e6 / steps
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps, host

    out = {"note": "layers of a stack share one layer's weights and buffers "
                   "(cache-resident across runs): a launch-overhead figure"}
    for name, layers, ms, xq in (("bert-base", 12, (128, 2048, 16384), False),
                                 ("bert-base", 1, (128,), False),
                                 ("gptj-6b", 4, (1, 16, 64), False),
                                 ("gptj-6b", 4, (1, 16, 64), True)):
        wl = W.workload(name)
        zq.sched_clear()
        c, B = W.layer_chain(wl, max(ms), dev, seed=1, layers=layers,
                             quant_on_load=xq)
        c.run_eager(max(ms))
        res = {"launches": len(c)}
        for M in ms:
            ge, he = per_run_us(lambda: c.run_eager(M))
            gg, hg = per_run_us(lambda: c.run(M))
            res[f"M={M}"] = {"eager_us": round(ge, 2), "eager_host_us": round(he, 2),
                             "graph_us": round(gg, 2), "graph_host_us": round(hg, 2)}
        # tune each GEMM of the layer at these token counts
        yq = B["ws"].view(torch.float16)
        for i, L in enumerate(wl.linears):
            y = {0: B["y_qkv"], 1: B["y_ao"], 3: B["y_out"]}.get(i)
            if y is None:
                y = yq[: max(ms) * L.N].view(max(ms), L.N)
            zq.gemm_tune(B[f"qx{i}"], B[f"sx{i}"], B[f"qw{i}"], B[f"sw{i}"],
                         wl.G, ms, bias=B[f"b{i}"],
                         act=zq.ACT_GELU if L.gelu else zq.ACT_NONE, y=y,
                         reps=reps)
        for M in ms:
            gt, _ = per_run_us(lambda: c.run(M))
            e = res[f"M={M}"]
            e["tuned_graph_us"] = round(gt, 2)
            e["tuned_plans"] = [zq.gemm_plan(M, L.N, L.K, L.bits).split(" W")[0]
                                for L in wl.linears]
        out[f"{name} x{layers}" + (" quant-on-load" if xq else "")] = res
        zq.sched_clear()
        c.close()
        del B
    return out


# -------------------------------------------------------------------- main --
# -------------------------------------------------------- profile summary --
COPY_BYTES = 256 * 2 ** 20


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _short(name):
    for key in ("gemm_tiled_kernel", "gemm_skinny_kernel", "gemm_stream_kernel",
                "gemm_gemv_kernel", "gemm_pingpong_kernel", "row_quant_kernel",
                "weight_quant_kernel", "splitk_reduce_kernel"):
        if key in name:
            return key
    if "neg_kernel" in name:
        return "copy"
    return name[:40]


def _split(values, entries, key):
    """Attribute the dispatches of one (kernel, grid) to the step entries that
    launch it.  Every entry launches it equally often; sorted by the measured
    value (duration, or fetched bytes), the i-th equal share goes to the entry
    with the i-th smallest expected value `key` (entries with equal keys are
    interchangeable).  Returns {entry name: [values]}, or None if the count
    does not divide or two populations that should differ overlap."""
    k = len(entries)
    if k == 0 or len(values) % k:
        return None
    n = len(values) // k
    vs = sorted(values)
    es = sorted(entries, key=lambda e: e[key])
    # entries whose expected values differ by more than 2% must form
    # populations that differ (durations are quantized and the counters
    # coarse, so equal values may meet at a boundary; equal group means
    # would mean the entries cannot be told apart)
    for i in range(k - 1):
        a, b = es[i][key], es[i + 1][key]
        if b > 1.02 * a:
            ga, gb = vs[i * n:(i + 1) * n], vs[(i + 1) * n:(i + 2) * n]
            # (two groups of one and the same constant value read the same
            # either way round: a coarse counter)
            if not sum(gb) > sum(ga) and not (ga[0] == ga[-1] == gb[0] == gb[-1]):
                return None
    return {e["name"]: vs[i * n:(i + 1) * n] for i, e in enumerate(es)}


def summarize(d, traffic_out=None, workload="neox-20b", m_index=None):
    """Per step entry: durations from the kernel trace and, when present,
    FETCH_SIZE / WRITE_SIZE per dispatch scaled by the same counters of the
    plain copy of COPY_BYTES bytes (GEMM entries; quantizer launches are
    listed per kernel)."""
    import glob
    import statistics as st
    import int4_quantized_transformer_amd as zq
    from int4_quantized_transformer_amd import workloads as W
    wl = W.workload(workload)
    M = wl.M[-1] if m_index is None else wl.M[m_index]
    entries = step_entries(zq, wl, M)
    gemm_e = [e for e in entries if e["grid"] is not None]
    lines = [f"step entries ({wl.name}, M={M}): " + ", ".join(
        f"{e['name']} -> {e['kernel']}@{e['grid']}" if e["grid"] else
        f"{e['name']} -> {e['kernel']}" for e in entries), ""]
    for tr in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"),
                               recursive=True)):
        groups = {}
        for r in _read_csv(tr):
            k = (_short(r["Kernel_Name"]),
                 int(r.get("Grid_Size_X") or r.get("Grid_Size")),
                 int(r.get("Workgroup_Size_X") or r.get("Workgroup_Size")))
            groups.setdefault(k, []).append(
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        lines.append(f"kernel trace {os.path.relpath(tr, d)}")
        lines.append("| kernel | grid (threads) | block | calls | avg us | "
                     "median us |")
        lines.append("|---|---|---|---|---|---|")
        for (k, g, w), v in sorted(groups.items(), key=lambda x: -sum(x[1])):
            lines.append(f"| {k} | {g} | {w} | {len(v)} | "
                         f"{st.mean(v) / 1e3:.2f} | {st.median(v) / 1e3:.2f} |")
        lines.append("")
        lines.append("GEMM step entries (dispatches of one kernel and grid "
                     "split equally by sorted duration, matched to the "
                     "entries' roofline times max(ops / INT8 peak, bytes / HBM "
                     "peak))")
        lines.append("| entry | kernel@grid | calls | avg us | median us |")
        lines.append("|---|---|---|---|---|")
        for (k, g, w), v in sorted(groups.items()):
            es = [e for e in gemm_e if e["kernel"] == k and e["grid"] == g
                  and e.get("block") in (None, w)]
            sp = _split(v, es, "roof_s") if es else None
            for name, vv in (sp or {}).items():
                lines.append(f"| {name} | {k}@{g} | {len(vv)} | "
                             f"{st.mean(vv) / 1e3:.2f} | "
                             f"{st.median(vv) / 1e3:.2f} |")
    pmc = {}
    for cc in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"),
                               recursive=True)):
        for r in _read_csv(cc):
            cname = r["Counter_Name"]
            if cname not in ("FETCH_SIZE", "WRITE_SIZE"):
                continue
            k = (_short(r["Kernel_Name"]), int(r["Grid_Size"]),
                 int(r["Workgroup_Size"]))
            pmc.setdefault(cname, {}).setdefault(k, {}).setdefault(
                r["Dispatch_Id"], 0.0)
            pmc[cname][k][r["Dispatch_Id"]] += float(r["Counter_Value"])
    traffic = {}
    if pmc:
        lines.append("")
        lines.append("HBM counters (KiB per dispatch; factor = counter / true "
                     f"bytes of the {COPY_BYTES >> 20} MiB copy)")
        factors = {}
        for cname, per in pmc.items():
            cp = [v for (k, g, w), dd in per.items() if k == "copy"
                  for v in dd.values()]
            if cp:
                factors[cname] = st.median(cp) * 1024 / COPY_BYTES
        lines.append(f"factors: {json.dumps(factors)}")
        lines.append("| counter | kernel | grid | dispatches | median KiB | "
                     "scaled bytes |")
        lines.append("|---|---|---|---|---|---|")
        for cname, per in pmc.items():
            f = factors.get(cname)
            for (k, g, w), dd in sorted(per.items()):
                med = st.median(dd.values())
                scaled = med * 1024 / f if f else None
                lines.append(f"| {cname} | {k} | {g} | {len(dd)} | {med:.0f} | "
                             f"{'' if scaled is None else f'{scaled:.0f}'} |")
        lines.append("")
        lines.append("GEMM step entries (dispatches of one kernel and grid "
                     "split equally by sorted counter value, matched to the "
                     "entries' algorithmic read / write bytes)")
        lines.append("| entry | counter | dispatches | median KiB | scaled "
                     "bytes | algorithmic bytes |")
        lines.append("|---|---|---|---|---|---|")
        for cname, per in pmc.items():
            f = factors.get(cname)
            if not f:
                continue
            for (k, g, w), dd in sorted(per.items()):
                es = [dict(e, write_bytes=e["bytes"] - e["read_bytes"])
                      for e in gemm_e if e["kernel"] == k and e["grid"] == g
                      and e.get("block") in (None, w)]
                key = "read_bytes" if cname == "FETCH_SIZE" else "write_bytes"
                sp = _split(list(dd.values()), es, key) if es else None
                for name, vv in (sp or {}).items():
                    med = st.median(vv)
                    scaled = med * 1024 / f
                    alg = [e[key] for e in es if e["name"] == name][0]
                    lines.append(f"| {name} | {cname} | {len(vv)} | {med:.0f} |"
                                 f" {scaled:.0f} | {alg} |")
                    traffic.setdefault(name, {"grid": g})[cname] = scaled
    mfma_lines(d, gemm_e, lines)
    print("\n".join(lines))
    if traffic_out and traffic:
        # one file for every profiled step; entries of other steps are kept
        # when they were taken on the same kernel sources
        out = {"sources": source_shas(), "steps": {}}
        try:
            with open(traffic_out) as f:
                old = json.load(f)
            if old.get("sources") == out["sources"]:
                out["steps"] = old.get("steps", {})
        except (OSError, ValueError):
            pass
        step = out["steps"][step_key(wl, M)] = {}
        for name, v in traffic.items():
            if "FETCH_SIZE" in v and "WRITE_SIZE" in v:
                step[name] = {
                    "grid": v["grid"],
                    "hbm_bytes_per_launch": round(v["FETCH_SIZE"] + v["WRITE_SIZE"]),
                    "fetch_bytes": round(v["FETCH_SIZE"]),
                    "write_bytes": round(v["WRITE_SIZE"])}
        with open(traffic_out, "w") as f:
            json.dump(out, f, indent=1)


def step_key(wl, M):
    """Name of a profiled step in the traffic file."""
    return (f"{wl.name} M={M}" + (" quant-on-load" if STEP_XQ else "")
            + (" chunked" if step_chunked(M) else ""))


def mfma_lines(d, gemm_e, lines):
    """Clock and MFMA utilisation per GEMM entry from a --pmc run with
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE: GRBM_GUI_ACTIVE is summed
    over the 8 XCDs (clock = GRBM / 8 / kernel duration); the MFMA busy
    cycles are summed over the 1024 SIMDs (busy = MFMA / 1024 / (GRBM / 8)),
    i.e. the achieved INT8 rate as a fraction of the peak at the measured
    clock."""
    import glob
    import statistics as st
    per = {}
    for cc in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"),
                               recursive=True)):
        for r in _read_csv(cc):
            if r["Counter_Name"] not in ("SQ_VALU_MFMA_BUSY_CYCLES",
                                         "GRBM_GUI_ACTIVE"):
                continue
            k = (_short(r["Kernel_Name"]), int(r["Grid_Size"]),
                 int(r["Workgroup_Size"]))
            dd = per.setdefault(k, {}).setdefault(r["Dispatch_Id"], {})
            dd[r["Counter_Name"]] = dd.get(r["Counter_Name"], 0.0) + \
                float(r["Counter_Value"])
            dd["us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    if not per:
        return
    lines.append("")
    lines.append("MFMA utilisation (per dispatch of a GEMM entry; the dispatches "
                 "of one kernel and grid split equally by sorted MFMA busy "
                 "cycles, matched to the entries' ops)")
    lines.append("| entry | dispatches | median us (under counters) | clock GHz "
                 "| MFMA busy | INT8 POP/s |")
    lines.append("|---|---|---|---|---|---|")
    for (k, g, w), dd in sorted(per.items()):
        es = [e for e in gemm_e if e["kernel"] == k and e["grid"] == g
              and e.get("block") in (None, w)]
        rows = [v for v in dd.values() if "SQ_VALU_MFMA_BUSY_CYCLES" in v
                and "GRBM_GUI_ACTIVE" in v]
        if not es or not rows:
            continue
        sp = _split([r["SQ_VALU_MFMA_BUSY_CYCLES"] for r in rows], es, "ops")
        for name, vv in (sp or {}).items():
            sel = [r for r in rows if r["SQ_VALU_MFMA_BUSY_CYCLES"] in vv]
            ops = [e["ops"] for e in es if e["name"] == name][0]
            us = st.median(r["us"] for r in sel)
            clk = st.median(r["GRBM_GUI_ACTIVE"] / 8 / (r["us"] * 1e3)
                            for r in sel)
            busy = st.median(r["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 /
                             (r["GRBM_GUI_ACTIVE"] / 8) for r in sel)
            lines.append(f"| {name} | {len(sel)} | {us:.1f} | {clk:.2f} | "
                         f"{busy:.3f} | {ops / us / 1e9:.2f} |")


def copy_calibration(torch, dev):
    """A plain elementwise kernel that reads COPY_BYTES and writes
    COPY_BYTES (torch.neg), three times."""
    a = torch.empty(COPY_BYTES // 2, dtype=torch.float16, device=dev).normal_()
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


def main():
    global STEP_XQ, STEP_CHUNKED
    args = parse()
    STEP_XQ = args.quant_on_load
    STEP_CHUNKED = args.chunked
    if args.summarize:
        summarize(args.summarize, args.write_traffic, args.workload,
                  args.m_index)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); the fused linear shards over tokens: each "
              "GPU runs the same layer on its own token rows with the weights "
              "replicated, and needs no communication", file=sys.stderr)
        sys.exit(2)

    import torch
    import int4_quantized_transformer_amd as zq
    from int4_quantized_transformer_amd import workloads as W

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    wl = W.workload(args.workload)
    M = wl.M[-1] if args.m_index is None else wl.M[args.m_index]
    zq.lib()

    if args.copy_calibration:
        copy_calibration(torch, dev)
    base, sets, R, per_set = build_sets(wl, M, dev, ROTATE_BYTES)
    stream = torch.cuda.current_stream()
    step_calls = [make_step(zq, s, wl, M, stream.cuda_stream) for s in sets]
    log(f"workload {wl.name} M={M}: {R} rotating sets x "
        f"{per_set / 2**20:.1f} MiB")

    run_calls(step_calls[0])
    torch.cuda.synchronize()

    for i in range(args.warmup):
        run_calls(step_calls[i % R])
    torch.cuda.synchronize()

    graphs = []
    if not args.no_graph:
        for calls in step_calls:
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            with torch.cuda.graph(g, stream=s):
                run_calls(make_step(zq, [c for c in sets[len(graphs)]], wl, M,
                                    s.cuda_stream))
            graphs.append(g)
        # the R steps back to back in one graph, each with its own weights
        # and inputs, as consecutive layers of a model are: the pages replay
        # a whole model's launch sequence as one graph
        g_all = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.graph(g_all, stream=s):
            for r in range(R):
                run_calls(make_step(zq, [c for c in sets[r]], wl, M,
                                    s.cuda_stream))
        for i in range(args.warmup):
            graphs[i % R].replay()
        g_all.replay()
        torch.cuda.synchronize()
        ms_g, wall_g = timed_steps(torch, g_all, R, graphs, args.steps, stream)
    # the same K steps launched from native code by the library's chain
    # executor; the step is timed both ways and `value` takes the faster
    # (on this runtime a graph node costs more than a native launch once
    # the host keeps ahead of the GPU)
    chains = [make_chain(zq, sets[r], wl, M) for r in range(R)]
    for i in range(args.warmup):
        chains[i % R].run_eager(M, stream=stream.cuda_stream)
    ms_n, wall_n = timed_native(torch, chains, M, args.steps, stream)
    by_launch = {"native_eager": round(ms_n, 5)}
    if not args.no_graph:
        by_launch["graph"] = round(ms_g, 5)
    launch = min(by_launch, key=by_launch.get)
    ms, wall_ms = (ms_g, wall_g) if launch == "graph" else (ms_n, wall_n)
    if args.only:
        print(json.dumps({"ms_per_step": ms}))
        return

    eager_ms = timed_eager(torch, step_calls, max(20, args.steps // 4), stream)
    bd, bdq = entry_timings(torch, zq, sets, wl, M, max(20, args.steps // 4))

    ops_step = sum(2 * M * d["L"].N * d["L"].K for d in base)
    tops = ops_step / (ms * 1e-3) / 1e12
    lin_by = {d["L"].name: d["L"] for d in base}
    breakdown = {}
    for n, t in bd.items():
        L = lin_by[n.split(".")[0]]
        ops, nbytes, bound = kernel_work(n, L, M, wl.G)
        e = {"us": round(t * 1e3, 2)}
        if ops:
            e["TOPS"] = round(ops / (t * 1e-3) / 1e12, 1)
            e["pct_int8_peak"] = round(100 * e["TOPS"] / INT8_PEAK_TOPS, 1)
        e["GB_per_s"] = round(nbytes / (t * 1e-3) / 1e9, 1)
        e["pct_attainable"] = pct_attainable(ops, nbytes, t * 1e-3)
        e["us_p10_p50_p90"] = [round(v * 1e3, 2) for v in bdq[n]]
        breakdown[n] = e
    dom = max(bd, key=bd.get)
    Ld = lin_by[dom.split(".")[0]]
    ops, nbytes, bound = kernel_work(dom, Ld, M, wl.G)
    t_dom = bd[dom] * 1e-3
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(ops / t_dom / 1e12, 1),
                "peak": INT8_PEAK_TOPS, "unit": "TOPS"}
    else:
        roof = {"bound": "hbm", "achieved": round(nbytes / t_dom / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = dom
    roof["avg_launch_us"] = round(bd[dom] * 1e3, 2)
    roof["algorithmic"] = {"ops": ops, "bytes": nbytes}
    roof["grid_threads"] = grid_threads(dom, Ld, M, wl.G, zq)
    roof["traffic"] = traffic_for(args.traffic, step_key(wl, M), dom,
                                  roof["grid_threads"])
    roof["timing"] = ("per-launch average from a HIP graph of this launch "
                      f"over {max(R, ENTRY_MIN_SETS)} rotating sets, events "
                      "around the replays")

    out = {
        "metric": METRIC, "value": round(tops, 2), "unit": "TOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": (f"{wl.name} encoder linears"
                                if wl.name.startswith("bert") else
                                f"{wl.name} decoder linears ("
                                + ("prefill" if M > 64 else "decode") + ")")
                   + ("; attn-out and FFN2 quantize-on-load" if STEP_XQ
                      else ""),
                   "tokens": M, "hidden": wl.linears[0].K, "group_rows": wl.G,
                   "linears": {L.name: f"{L.N}x{L.K} W{L.bits}A8"
                               + (" +LN" if L.ln else "")
                               + (" +GeLU" if L.gelu else "")
                               for L in wl.linears},
                   "rotating_sets": R, "launch": launch,
                   "steps_per_graph_replay": R if not args.no_graph else 0,
                   "activations": (
                       f"N(0,1), {wl.n_outliers(wl.linears[0].K)} of "
                       f"{wl.linears[0].K} channels x{wl.outlier_factor:g}"
                       + ("; value recipe of another workload, its "
                          "reference read as counting from zero: GPT-J's "
                          "recipe for NeoX, BERT-base's for BERT-large"
                          if wl.name in ("neox-20b", "bert-large") else ""))},
        "roofline": roof,
    }
    extras = {"ms_per_step_by_launch": by_launch,
              "eager_ms_per_step": round(eager_ms, 5),
              "host_wall_ms_per_step": round(wall_ms, 5),
              "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 2),
              "breakdown": breakdown}
    if not args.no_fp16:
        extras["fp16_matmul"] = fp16_comparator(torch, zq, dev, wl, M, ms,
                                                max(10, args.steps // 2))
    if not args.no_decode:
        extras["decode"] = decode_figure(torch, zq, dev,
                                         with_fp16=not args.no_fp16)
        out["roofline_decode"] = decode_roofline(extras["decode"], args.traffic)
    if not args.no_prefill:
        extras["prefill"] = prefill_figure(torch, zq, dev)
    if not args.no_quantizers:
        extras["quantizers"] = quantizer_figure(torch, zq, dev)
    if not args.no_w8a16:
        extras["w8a16"] = w8a16_figure(torch, zq, dev)
    if not args.no_static:
        extras["static_vs_tokenwise"] = static_figure(torch, zq, dev)
    if not args.no_xq:
        extras["quant_on_load"] = xq_figure(torch, zq, dev)
    if not args.no_chain:
        extras["layer_chain"] = chain_figure(torch, zq, dev)
    out["extras"] = extras
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(base, wl, M)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def fp16_comparator(torch, zq, dev, wl, M, int8_ms, steps):
    """torch fp16 matmul + bias (+GeLU) of the step's linears at the same
    shapes, with fp16 weights (library run), each from a CUDA graph over
    rotating weight copies as the INT8 step rotates its sets; the step time
    is the sum of the four."""
    per = {L.name: fp16_linear_us(torch, dev, wl, i, M, steps)
           for i, L in enumerate(wl.linears)}
    ms = sum(per.values()) / 1e3
    ops = sum(2 * M * L.N * L.K for L in wl.linears)
    return {"ms_per_step": round(ms, 5),
            "TFLOPS": round(ops / (ms * 1e-3) / 1e12, 1),
            "pct_fp16_peak": round(100 * ops / (ms * 1e-3) / 1e12
                                   / FP16_PEAK_TFLOPS, 1),
            "us_by_linear": {k: round(v, 2) for k, v in per.items()},
            "int8_step_speedup": round(ms / int8_ms, 3),
            "note": "torch.addmm fp16 + bias (+gelu), graph replay over "
                    "rotating fp16 weight copies, same shapes, no "
                    "quantization; the INT8 step includes its LN+quant and "
                    "quant launches"}


def decode_roofline(dec, traffic_path):
    """Roofline entry of the decode regime: the slowest GEMM of the
    GPT-NeoX-20B one-token layer (weight streaming, HBM-bound)."""
    case = dec.get("neox-20b M=1")
    if not case:
        return None
    name, e = max(case["per_linear"].items(), key=lambda kv: kv[1]["us"])
    t = e["us"] * 1e-6
    achieved = e["bytes"] / t / 1e9
    import int4_quantized_transformer_amd as zq
    from int4_quantized_transformer_amd import workloads as W
    wl = W.workload("neox-20b")
    lin = {L.name: L for L in wl.linears}[name.split()[0]]
    entry = f"{lin.name}.gemm_w{lin.bits}a8"
    tr = traffic_for(traffic_path, "neox-20b M=1", entry,
                     grid_threads(entry, lin, 1, wl.G, zq))
    return {"bound": "hbm", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": tr,
            "kernel": f"neox-20b M=1 {name} ({e['plan']})",
            "avg_launch_us": e["us"], "algorithmic": {"bytes": e["bytes"]},
            "layer_GB_per_s": case["GB_per_s"],
            "layer_pct_hbm_peak": case["pct_hbm_peak"],
            "timing": "per-launch average from a HIP graph of this launch "
                      "over rotating weight sets, events around the replays"}


if __name__ == "__main__":
    main()
