"""Throughput of one hybrid-batch decoder-layer forward on one MI355X.

Workload (default): a Llama-2-70B-shaped layer (H=8192, 64 q / 8 kv heads,
head_dim 128, SwiGLU FFN 28672, bf16 weights N(0, 0.01)) over a hybrid batch
of the last 512-token chunk of a 4096-token prompt (3584 tokens already
cached) plus Bd=64 decodes with contexts drawn from U{512..4096}; pages of 16
tokens; rows padded to 16.  This is the largest layer of the workloads that
fits one GPU unsharded.  Synthetic, seeded inputs (seed 0).  The
Mistral-7B-shaped layer (Lp=256 after 768 cached + Bd=32 decodes,
contexts U{128..2048}) is timed briefly beside it (`extra`).

A step is one layer call as it runs inside a stack of layers
(``hl_layer_forward_chain``): every kernel of the layer, with the layer's
input RMSNorm already formed by the previous layer's down-projection reduce
and this call's reduce forming the next layer's -- one RMSNorm per call, as
in the stand-alone ``hl_layer_forward``, which is timed beside it
(`standalone_call`; ``--plain`` makes it the timed step).  Inputs are
resident in HBM before the timed region; R copies of the weights and of
the KV pool are rotated so that the 256 MB MALL cannot hold one call's
working set for the next.  Before the W warmup steps the layer runs for
about --settle-ms of GPU time so that the clocks have left their ramp (the
first ~25 ms of calls run several percent slow); the timed region is exactly
K steps.

Printed: one JSON line with tokens/s per layer (real rows / time), the
dominant kernel's roofline figures, the time of every kernel slot of the
layer against the roofline model T = max(T_math, T_mem), and the CPU
oracle's rate on the host (median of --cpu-runs full calls, plus a one-thread
figure on a bounded sample), and the HBM read rate a plain streaming read
attains on this GPU (`hbm_read_attained`; an HBM-bound dominant kernel also
gets its fraction of that rate).  Kernel times come from HIP events that the
library records between its kernels on the stream it launches on.  `parts`
times the batch's chunk and its decodes as separate calls beside the hybrid
call (alternating rounds): the saving of one hybrid call over the two, and
what the piggybacked decodes add as a fraction of their own call.

``--cpu-table PATH`` only times the CPU oracle over the other measured
configurations (no GPU use) and writes a markdown table.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "hybrid-batch tokens/s per layer (Lp+Bd); % peak MFMA (linear), % HBM BW (attn)"
WORKLOADS = ["llama70", "mistral", "tiny", "llama70_tp8", "mistral_tp4", "decode128"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--settle-ms", type=float, default=100.0,
                   help="GPU time of untimed layer calls before the warmup steps")
    p.add_argument("--workload", choices=WORKLOADS, default="llama70")
    p.add_argument("--extra", default="mistral",
                   help="comma-separated workloads timed briefly beside the main one ('' for none)")
    p.add_argument("--pad", type=int, default=16)
    p.add_argument("--rotate", type=int, default=4)
    p.add_argument("--no-graph", action="store_true", help="skip the graph-replay timing")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-runs", type=int, default=3)
    p.add_argument("--cpu-table", metavar="PATH",
                   help="only time the CPU oracle over the sweep configurations (no GPU) and "
                        "write the markdown table to PATH")
    p.add_argument("--no-standalone", action="store_true",
                   help="skip the stand-alone call's timing (profiling runs)")
    p.add_argument("--no-parts", action="store_true",
                   help="skip timing the batch's chunk and its decodes as separate calls")
    p.add_argument("--plain", action="store_true",
                   help="time the stand-alone layer call instead of the call inside a stack")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run one 256 MiB device-to-device copy first (PMC byte-counter scale)")
    return p.parse_args()


def make_batch(name, seed=0, **kw):
    """(batch, description, sample builder for the one-thread oracle figure)."""
    from chunked_prefill_hybrid_rmsnorm_amd import inputs as I
    if name == "mistral":
        return I.mistral_batch(seed=seed, **kw), (
            "mistral7b-shaped layer: Lp=256 (768 cached) + Bd=32 decodes, ctx U[128,2048]")
    if name == "llama70":
        return I.llama70_batch(seed=seed, **kw), (
            "llama2-70b-shaped layer: Lp=512 (3584 cached) + Bd=64 decodes, ctx U[512,4096]")
    if name == "llama70_tp8":
        return I.llama70_tp8_batch(seed=seed, **kw), (
            "llama2-70b layer, one GPU's tensor-parallel share (T=8: 8 q / 1 kv heads, F=3584): "
            "Lp=512 (3584 cached) + Bd=64 decodes, ctx U[512,4096]")
    if name == "mistral_tp4":
        return I.mistral_tp4_batch(seed=seed, **kw), (
            "mistral7b layer, one GPU's tensor-parallel share (T=4: 8 q / 2 kv heads, F=3584): "
            "Lp=256 (768 cached) + Bd=32 decodes, ctx U[128,2048]")
    if name == "decode128":
        return I.make_hybrid_batch(I.MISTRAL_7B, chunk_lens=[], chunk_starts=[], n_decodes=128,
                                   ctx_range=(128, 4096), seed=seed, weight_std=0.02), (
            "mistral7b-shaped layer, decodes only: Bd=128 decodes, ctx U[128,4096]")
    return I.tiny_batch(seed=seed), "tiny layer H=256: Lp=64 (64 cached) + Bd=4 decodes, ctx U[16,128]"


def time_loop(fn, steps, warmup, settle_ms=0.0):
    """Average ms per call, HIP events on the current stream (the one the
    library launches on).  Untimed: calls for about `settle_ms` of GPU time,
    then `warmup` calls."""
    import torch
    if settle_ms > 0:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(0)
        b.record()
        torch.cuda.synchronize()
        for i in range(int(settle_ms / max(a.elapsed_time(b), 1e-3))):
            fn(i)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(hb, name, runs):
    """The oracle as it stands, on the host cores: `runs` full calls of the
    benchmarked batch with every BLAS thread, and one call of a bounded
    sample of the same layer (16 chunk rows at the end of the same cached
    prefix plus 4 decodes, same weights) on one thread."""
    import numpy as np
    from chunked_prefill_hybrid_rmsnorm_amd import inputs as I
    from oracle import layer_forward
    from tests.oracle_inputs import oracle_args
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = os.cpu_count() or 1
    args = oracle_args(hb)
    times = []
    for _ in range(runs):
        t = time.perf_counter()
        layer_forward(*args)
        times.append(time.perf_counter() - t)
    t_med = sorted(times)[len(times) // 2]
    M = hb.x.shape[0]
    res = {"value": round(M / t_med, 2), "unit": "tokens/s", "cores": int(threads),
           "kind": "oracle",
           "sample": f"{runs} full call(s) of the benchmarked hybrid batch (M={M} rows), float64 "
                     f"numpy oracle with {threads} BLAS threads, median {t_med:.2f} s/call",
           "cpu_model": _cpu_model(), "host_cpu_count": os.cpu_count(),
           "run_seconds": [round(t, 3) for t in times]}
    # one thread, on a bounded sample of the same layer (same weights and
    # cached-prefix length, fewer rows)
    c0 = hb.chunks[0] if hb.chunks else None
    ctx = hb.decodes.ctx_lens
    lo, hi = (int(ctx.min()), int(ctx.max())) if len(ctx) else (16, 128)
    n_rows = min(16, c0.length) if c0 else 0
    sample = I.make_hybrid_batch(hb.shape, chunk_lens=[n_rows] if n_rows else [],
                                 chunk_starts=[c0.start_pos + c0.length - n_rows] if n_rows else [],
                                 n_decodes=4, ctx_range=(lo, hi), seed=1, weights=hb.weights)
    sargs = oracle_args(sample)
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t = time.perf_counter()
            layer_forward(*sargs)
            t1 = time.perf_counter() - t
        ms = sample.x.shape[0]
        res["one_thread"] = {"value": round(ms / t1, 2), "unit": "tokens/s", "cores": 1,
                             "sample": f"{n_rows} chunk rows after {c0.start_pos + c0.length - n_rows if c0 else 0} "
                                       f"cached tokens + 4 decodes (ctx U[{lo},{hi}]) of the same "
                                       f"layer and weights, M={ms}, one call {t1:.2f} s"}
    return res


def cpu_table(runs, path, keys=None, prompt_chunks=(1, 16)):
    """The oracle as it stands on the host cores (every BLAS thread) over the
    configurations the GPU path is measured on: the tiny, Mistral-shaped and
    Llama-70B-shaped batches, three points of the token-budget grid, and the
    2048-token prompt prefilled in 1 and in 16 chunks (each chunk's call
    reading the pages the earlier calls wrote).  Median of `runs` calls per
    batch; one pass of each prompt.  `keys` picks a subset of the batches
    (tiny, mistral, grid256, grid128d128, grid512d16, llama70) and
    `prompt_chunks` the prompt splits."""
    import numpy as np
    from chunked_prefill_hybrid_rmsnorm_amd import inputs as I
    from oracle import layer_forward
    from tests.oracle_inputs import oracle_args, oracle_weights, widen
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    M7 = I.MISTRAL_7B
    grid = lambda lp, bd: I.make_hybrid_batch(M7, chunk_lens=[lp] if lp else [],
                                              chunk_starts=[0] if lp else [], n_decodes=bd,
                                              ctx_range=(128, 4096), seed=0)
    batches = [
        ("tiny", "tiny layer (H=256): Lp=64 (64 cached) + Bd=4", lambda: I.tiny_batch(seed=0)),
        ("mistral", "Mistral-7B-shaped: Lp=256 (768 cached) + Bd=32",
         lambda: I.mistral_batch(seed=0)),
        ("grid256", "Mistral-7B-shaped grid point: Lp=256 + Bd=0", lambda: grid(256, 0)),
        ("grid128d128", "Mistral-7B-shaped grid point: Lp=128 + Bd=128", lambda: grid(128, 128)),
        ("grid512d16", "Mistral-7B-shaped grid point: Lp=512 + Bd=16", lambda: grid(512, 16)),
        ("llama70", "Llama-2-70B-shaped: Lp=512 (3584 cached) + Bd=64",
         lambda: I.llama70_batch(seed=0)),
    ]
    rows = []
    for key, desc, make in batches:
        if keys is not None and key not in keys:
            continue
        hb = make()
        args = oracle_args(hb)
        times = []
        for _ in range(runs):
            t = time.perf_counter()
            layer_forward(*args)
            times.append(time.perf_counter() - t)
        t_med = sorted(times)[len(times) // 2]
        M = hb.x.shape[0]
        rows.append((desc, M, f"median of {runs}", t_med, M / t_med))
        log(f"{desc}: {t_med:.3f} s/call")
    for n in prompt_chunks:
        seq = I.make_prompt_sequence(M7, 2048, n, seed=0)
        w = oracle_weights(seq.weights)
        kv = widen(seq.kv_pages)
        t = time.perf_counter()
        for k in range(n):
            c = seq.chunk(k)
            kv = layer_forward(seq.shape, w, widen(seq.chunk_rows(k)),
                               [(c.length, c.start_pos, c.block_table)], [], [], kv).kv_pages
        dt = time.perf_counter() - t
        rows.append((f"Mistral-7B-shaped 2048-token prompt in {n} chunk(s)", 2048,
                     f"{n} call(s), one pass", dt, 2048 / dt))
        log(f"2048-token prompt in {n} chunk(s): {dt:.2f} s")
    lines = ["# CPU oracle on the measured configurations", "",
             "Command (run from the repository root):", "",
             f"    python bench.py --cpu-table {path} --cpu-runs {runs}", "",
             f"float64 NumPy oracle (`oracle/`), {threads} BLAS threads, host CPU "
             f"`{_cpu_model()}` ({os.cpu_count()} logical CPUs). Seeded synthetic inputs, the "
             "same recipes as the GPU measurements. A reported baseline, not a target.", "",
             "| batch | rows | timing | s | tokens/s |", "|---|---:|---|---:|---:|"]
    for desc, M, how, dt, tps in rows:
        lines.append(f"| {desc} | {M} | {how} | {dt:.3f} | {tps:.1f} |")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps({"cpu_table": path, "threads": threads,
                      "rows": [{"batch": r[0], "rows": r[1], "seconds": round(r[3], 4),
                                "tokens_per_s": round(r[4], 2)} for r in rows]}), flush=True)


def hbm_read_attained(gib=1, copies=4, calls=16):
    """HBM read rate of the library's plain streaming read (hl_read_stream)
    over `copies` buffers of `gib` GiB read in turn, together far past the
    256 MB MALL: the bandwidth this GPU attains, beside the 8 TB/s of the data
    sheet that `roofline.peak` uses."""
    import torch
    from chunked_prefill_hybrid_rmsnorm_amd import binding as B
    n = gib << 30
    bufs = [torch.full((n // 4,), 0x01020304, dtype=torch.int32, device="cuda")
            for _ in range(copies)]
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    for b in bufs:
        B.hl_read_stream(b, n, sink)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(calls):
        B.hl_read_stream(bufs[i % copies], n, sink)
    t1.record()
    torch.cuda.synchronize()
    sec = t0.elapsed_time(t1) * 1e-3
    del bufs
    torch.cuda.empty_cache()
    return {"value": round(n * calls / sec / 1e12, 3), "unit": "TB/s", "bytes_per_call": n,
            "calls": calls, "buffers": copies,
            "kernel": "hl_read_stream: 16-byte non-temporal loads, 8192 workgroups x 256 lanes"}


def measure(a, name, steps, warmup, settle_ms, graph, key):
    """Layer time, graph replay, per-call spread, per-slot times and the
    dominant slot's roofline for one workload."""
    import torch
    from chunked_prefill_hybrid_rmsnorm_amd import binding as B
    from chunked_prefill_hybrid_rmsnorm_amd import profiling as P
    from chunked_prefill_hybrid_rmsnorm_amd import roofline as RL
    log(f"generating {name} inputs ...")
    hb, desc = make_batch(name)
    db = B.DeviceBatch(hb, pad=a.pad)
    log("uploading rotation copies ...")
    copies = [((db.wt, db.weights), db.kv)]
    keep = []
    for _ in range(a.rotate - 1):
        wt = {k: v.clone() for k, v in db.wt.items()}
        wstruct = B.hl_weights(*(wt[k].data_ptr() for k in
                                 ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "g_attn", "g_ffn")))
        kvt = db.kv_t.clone()
        keep.append((wt, kvt))
        copies.append(((wt, wstruct), B.hl_kv(kvt.data_ptr(), db.kv.num_pages)))
    torch.cuda.synchronize()

    # a layer inside a stack: its input RMSNorm (xn_in) was formed by the
    # previous layer's down-projection reduce, and its own reduce forms the
    # next layer's (xn_next) -- one RMSNorm per call, as in the plain call
    H = hb.shape.hidden
    xn_in = torch.empty((db.Mp, H), dtype=torch.bfloat16, device="cuda")
    B.hl_rmsnorm(db.x, db.wt["g_attn"], xn_in, db.M, db.Mp, H, hb.shape.rms_eps)
    xn_next = torch.empty_like(xn_in)

    def plain(i):
        (wt, ws), kv = copies[i % len(copies)]
        B.hl_layer_forward(db.cfg, ws, db.x, db.chunks, db.dec, kv, db.out, db.ws, db.ws_bytes,
                           a.pad)

    def chained(i, events=None):
        (wt, ws), kv = copies[i % len(copies)]
        B.hl_layer_forward_chain(db.cfg, ws, db.x, db.chunks, db.dec, kv, db.out, db.ws,
                                 db.ws_bytes, a.pad, xn_in=xn_in, g_next=wt["g_attn"],
                                 xn_next=xn_next, events=events)

    layer = plain if a.plain else chained

    log(f"layer: settle {settle_ms:.0f} ms + {warmup} warmup + {steps} timed steps ...")
    ms = time_loop(layer, steps, warmup, settle_ms)
    M = db.M
    tok_s = M / (ms / 1e3)
    log(f"layer {ms * 1e3:.1f} us/step, {tok_s / 1e6:.3f} M tokens/s")

    # one graph holding one call per rotation copy, replayed: the host launch
    # cost of the layer's kernels and of the graph launch itself is spread
    # over the calls it holds
    g_res = None
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(len(copies)):
                layer(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        reps = max(1, steps // len(copies))
        gms = time_loop(lambda i: g.replay(), reps, max(1, warmup // len(copies))) / len(copies)
        g_res = {"ms_per_step": round(gms, 5), "value": round(M / (gms / 1e3), 1),
                 "calls_per_graph": len(copies)}
        log(f"layer (graph replay, {len(copies)} calls per graph) {gms * 1e3:.1f} us/step")
        # eager calls and replays in alternating blocks, so that a clock that
        # drifts over the run weighs on both alike; medians over the rounds
        blk = max(1, steps // 4 // len(copies)) * len(copies)
        e_t, g_t = [], []
        for _ in range(4):
            e_t.append(time_loop(layer, blk, 0))
            g_t.append(time_loop(lambda i: g.replay(), blk // len(copies), 0) / len(copies))
        med = lambda v: (sorted(v)[1] + sorted(v)[2]) / 2  # noqa: E731  (four rounds)
        e_med, g_med = med(e_t), med(g_t)
        g_res["interleaved"] = {"eager_ms_per_step": round(e_med, 5),
                                "replay_ms_per_step": round(g_med, 5), "rounds": 4,
                                "calls_per_block": blk}
        log(f"interleaved blocks of {blk} calls: eager {e_med * 1e3:.1f} us/step, "
            f"graph replay {g_med * 1e3:.1f} us/step")

    # spread of single calls: one event between consecutive calls
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    for i in range(warmup):
        layer(i)
    bounds[0].record()
    for i in range(steps):
        layer(i)
        bounds[i + 1].record()
    torch.cuda.synchronize()
    per_call = sorted(bounds[i].elapsed_time(bounds[i + 1]) * 1e3 for i in range(steps))

    def pct(q):
        return round(per_call[min(len(per_call) - 1, int(q * len(per_call)))], 2)

    spread = {"p10_us": pct(0.1), "p50_us": pct(0.5), "p90_us": pct(0.9)}
    log(f"per call: p10 {spread['p10_us']} us, p50 {spread['p50_us']} us, p90 {spread['p90_us']} us")

    # per-slot times inside the real layer sequence: HIP events recorded by
    # the library between its kernels, on the stream it launches on
    log("per-slot timing with stage events ...")
    names = B.stage_names()
    ns = len(names)

    def make_events():
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)]
        for e in evs:  # materialise the underlying HIP events
            e.record()
        return evs

    ev_sets = [make_events() for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(warmup):
        layer(i)
    for i in range(steps):
        if a.plain:
            (wt, ws), kv = copies[i % len(copies)]
            B.hl_layer_forward_timed(db.cfg, ws, db.x, db.chunks, db.dec, kv, db.out, db.ws,
                                     db.ws_bytes, a.pad, ev_sets[i])
        else:
            chained(i, ev_sets[i])
    torch.cuda.synchronize()
    lens = [c.length for c in hb.chunks]
    starts = [c.start_pos for c in hb.chunks]
    stages = {s.name: s for s in RL.layer_stages(hb.shape.hidden, hb.shape.n_q_heads,
                                                  hb.shape.n_kv_heads, hb.shape.head_dim,
                                                  hb.shape.ffn, lens, starts,
                                                  [int(c) for c in hb.decodes.ctx_lens], a.pad,
                                                  chained=not a.plain)}
    table = {}
    for k, sname in enumerate(names):
        t = sum(ev[k].elapsed_time(ev[k + 1]) for ev in ev_sets) / steps * 1e-3
        st = stages[sname]
        work = st.flops > 0 or st.bytes > 0
        table[sname] = {
            "us": round(t * 1e6, 2),
            "bound": st.bound if work else "none (launch-shape overhead)",
            "t_roof_us": round(st.t_roof() * 1e6, 2),
            "roof_frac": round(st.t_roof() / t, 4) if t > 0 and work else None,
            "GB/s": round(st.bytes / t / 1e9, 1) if t > 0 and work else None,
            "TFLOP/s": round(st.flops / t / 1e12, 2) if t > 0 and work else None,
        }
        log(f"  {sname:24s} {t * 1e6:8.1f} us  roof {st.t_roof() * 1e6:7.1f} us  "
            f"({table[sname]['bound']}, frac {table[sname]['roof_frac']})")
    # dominant kernel: the slot with the longest average duration
    dom = max(table, key=lambda k: table[k]["us"])
    st = stages[dom]
    t_dom = table[dom]["us"] * 1e-6
    if st.bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(st.bytes / t_dom / 1e9, 1),
                "peak": RL.PEAK_HBM_BPS / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(st.flops / t_dom / 1e12, 2),
                "peak": RL.PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = P.stored_traffic(TRAFFIC_FILE, dom, key)
    roof["kernel"] = dom
    roof["kernel_us"] = table[dom]["us"]
    roof["algorithmic_per_launch"] = st.bytes if st.bound == "hbm" else st.flops
    roof["algorithmic_bytes"] = st.bytes
    roof["algorithmic_flops"] = st.flops
    t_roof = RL.layer_roofline_time(list(stages.values()))
    other = None
    if not a.plain and not a.no_standalone:
        # the stand-alone call (its own first RMSNorm, no next-layer norm)
        pms = time_loop(plain, max(steps // 2, 1), max(warmup // 2, 1))
        other = {"ms_per_step": round(pms, 5), "value": round(M / (pms / 1e3), 1)}
        log(f"stand-alone call (own first RMSNorm) {pms * 1e3:.1f} us/step")
    parts = None
    if not a.plain and not a.no_parts and hb.chunks and db.dec.n > 0:
        parts = time_parts(db, hb, copies, steps, a.pad)
        log(f"parts: hybrid {parts['hybrid_ms'] * 1e3:.1f} us, chunk alone "
            f"{parts['chunk_alone_ms'] * 1e3:.1f} us, decodes alone "
            f"{parts['decodes_alone_ms'] * 1e3:.1f} us")
    return hb, desc, {
        "ms": ms, "tok_s": tok_s, "M": M, "Mp": db.Mp, "roofline": roof, "stages": table,
        "layer_roofline": {"t_roof_us": round(t_roof * 1e6, 2), "t_us": round(ms * 1e3, 2),
                           "frac": round(t_roof / (ms * 1e-3), 4)},
        "graph_replay": g_res, "per_call": spread, "standalone_call": other, "parts": parts}


def time_parts(db, hb, copies, steps, pad):
    """The hybrid call against its parts: the chunk rows alone and the decode
    rows alone, each as a call inside a layer stack on the same weights,
    pages and contexts, timed in three alternating rounds (medians), so that
    clock drift weighs on all three alike.  The pages' claim is that the
    decodes cost far less piggybacked on the chunk than in a call of their own
    (Sarathi-Serve digest, section 2; intelliparadigm.com article, section 3.1)."""
    import torch
    from chunked_prefill_hybrid_rmsnorm_amd import binding as B
    H = hb.shape.hidden
    Lp = sum(c.length for c in hb.chunks)
    M = db.M
    none = B.hl_decodes(0, None, None, 0, 0)

    def setup(x_rows):
        m = x_rows.shape[0]
        mp = -(-m // pad) * pad
        xn = torch.empty((mp, H), dtype=torch.bfloat16, device="cuda")
        B.hl_rmsnorm(x_rows, db.wt["g_attn"], xn, m, mp, H, hb.shape.rms_eps)
        return xn, torch.empty_like(xn), torch.empty_like(x_rows)

    full = (db.x, db.chunks, db.dec) + setup(db.x)
    chunk = (db.x[:Lp], db.chunks, none) + setup(db.x[:Lp])
    decs = (db.x[Lp:M], [], db.dec) + setup(db.x[Lp:M])

    def caller(spec):
        x, chunks, dec, xn_in, xn_next, out = spec

        def call(i):
            (wt, ws), kv = copies[i % len(copies)]
            B.hl_layer_forward_chain(db.cfg, ws, x, chunks, dec, kv, out, db.ws, db.ws_bytes,
                                     pad, xn_in=xn_in, g_next=wt["g_attn"], xn_next=xn_next)
        return call

    calls = [caller(full), caller(chunk), caller(decs)]
    blk = max(len(copies), steps // 4 // len(copies) * len(copies))
    for c in calls:  # warm each call (one round of the rotation copies)
        for i in range(len(copies)):
            c(i)
    t = [[], [], []]
    for _ in range(3):
        for k, c in enumerate(calls):
            t[k].append(time_loop(c, blk, 0))
    med = [sorted(v)[1] for v in t]
    return {"hybrid_ms": round(med[0], 5), "chunk_alone_ms": round(med[1], 5),
            "decodes_alone_ms": round(med[2], 5),
            "saving": round(1 - med[0] / (med[1] + med[2]), 4),
            "decodes_added_frac": round((med[0] - med[1]) / med[2], 4),
            "rounds": 3, "calls_per_block": blk}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        log("bench.py: only --gpus 1 is supported (single-GPU build)")
        sys.exit(2)
    if a.cpu_table:
        cpu_table(a.cpu_runs, a.cpu_table)
        return
    import torch
    from chunked_prefill_hybrid_rmsnorm_amd import binding as B
    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    B.load()
    torch.cuda.set_device(0)

    if a.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    hb, desc, r = measure(a, a.workload, a.steps, a.warmup, a.settle_ms, not a.no_graph, a.workload)
    extra = {}
    for name in [w for w in a.extra.split(",") if w and w != a.workload]:
        if name not in WORKLOADS:
            log(f"unknown extra workload {name}")
            sys.exit(2)
        _, edesc, er = measure(a, name, min(a.steps, 100), min(a.warmup, 50), a.settle_ms, False,
                               name)
        extra[name] = {"workload": edesc, "value": round(er["tok_s"], 1), "unit": "tokens/s",
                       "ms_per_step": round(er["ms"], 5), "rows": er["M"],
                       "roofline": er["roofline"], "layer_roofline": er["layer_roofline"],
                       "stages": {k: v["us"] for k, v in er["stages"].items()},
                       "parts": er["parts"]}
        torch.cuda.empty_cache()

    result = {
        "metric": METRIC, "value": round(r["tok_s"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": desc, "rows": r["M"], "rows_padded": r["Mp"], "pad": a.pad,
                   "rotated_copies": a.rotate, "clock_settle_ms": a.settle_ms,
                   "layer_call": ("stand-alone (own first RMSNorm)" if a.plain else
                                  "inside a layer stack: first RMSNorm formed by the previous "
                                  "layer's down reduce, this call's reduce forms the next one")},
        "roofline": r["roofline"],
        "layer_roofline": r["layer_roofline"],
        "stages": r["stages"],
        "graph_replay": r["graph_replay"],
        "per_call": r["per_call"],
        "standalone_call": r["standalone_call"],
        "parts": r["parts"],
        "extra": extra,
    }
    log("timing the streaming read ...")
    att = hbm_read_attained()
    result["hbm_read_attained"] = att
    if r["roofline"] and r["roofline"].get("bound") == "hbm":
        # the dominant kernel's rate against the attained read rate as well
        result["roofline"]["frac_of_attained"] = round(
            r["roofline"]["achieved"] / (att["value"] * 1e3), 4)
    if not a.no_cpu_baseline:
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(hb, a.workload, a.cpu_runs)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
