#!/usr/bin/env python3
"""Benchmark of the MoDA forward on one MI355X.

One step = the whole MoDA path over one batch of synthetic input already in
HBM: moda_pack_depth_cache (depth repack) + moda_fwd (fused forward).  The
causal-only mode (moda_causal_fwd) is timed on the same Q/K/V for the
MoDA / causal-only time ratio, depth attention alone (moda_depth_fwd) on the
same packed cache for its HBM rate, and the forward straight from the natural
depth layout (moda_fwd_natural), from the layer-major one (moda_fwd_layers)
and, with --ablation, as a masked scan of the flat depth axis
(moda_fwd_masked_scan, T <= 16384 only), group-unaware (each query head of a
group in its own moda_fwd launch, so each reads the depth span itself) and as
a naive per-token loop (T decode calls, T <= 16384 only) for the layout
ablation, the decode step
(moda_decode: the last token over the whole cache) and the depth-stream write
of one entry per token into the packed cache (moda_append_depth) for their
HBM rates.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--config long_64k] [--no-cpu-baseline]
    python bench.py --sweep            # one JSON line per sweep point (no oracle)
    python bench.py --sweep --sweep-bwd   # ... with the backward timed too
    python bench.py --sweep --results sweep.jsonl   # ... appended to a file; a rerun skips
                                                    # the points already there
    python bench.py --decode-sweep     # one JSON line per decode shape
    python bench.py --stack --config layer_1p5b   # a stack of layers growing the depth stream

FLOP convention (algorithmic, per query head): 4 * d * (T(T+1)/2 + T*L), the
diagonal counted, exponentials not counted.  The backward (moda_bwd, timed
after the step, not part of it) is credited 2.5x that: five products per
(query, entry) pair (S recomputed, dP, dV, dQ, dK) against the forward's two.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA (published)
MALL_BYTES = 256 << 20      # MI355X last-level (Infinity) cache, memory side
METRIC = "MoDA fwd TFLOP/s + % bf16 MFMA peak at T=64K; time ratio vs causal-only"
KERNEL_SOURCES = [os.path.join(ROOT, "depth_wise_kv_amd", "csrc", f)
                  for f in ("moda_kernels.hip", "moda_device.h", "moda_internal.h")]


def flops(c, L=None):
    L = c["L"] if L is None else L
    return 4.0 * c["d"] * c["B"] * c["Hq"] * (c["T"] * (c["T"] + 1) / 2.0 + c["T"] * L)


def es(c):
    return 2 if c["dtype"] == "bf16" else 4


def fused_bytes(c, L=None):
    """Q, O, sequence K/V and depth K/V each moved once (no LSE)."""
    L = c["L"] if L is None else L
    B, Hq, Hkv, T, d = c["B"], c["Hq"], c["Hkv"], c["T"], c["d"]
    return es(c) * (2 * B * Hq * T * d + 2 * B * Hkv * T * d + 2 * B * Hkv * T * L * d)


def depth_bytes(c):
    """Depth attention alone: Q and O once, depth K/V once (no LSE)."""
    B, Hq, Hkv, T, L, d = c["B"], c["Hq"], c["Hkv"], c["T"], c["L"], c["d"]
    return es(c) * (2 * B * Hq * T * d + 2 * B * Hkv * T * L * d)


def pack_bytes(c):
    """Depth K/V read once and written once."""
    return 2 * (2 * c["B"] * c["Hkv"] * c["T"] * c["L"] * c["d"] * es(c))


def append_bytes(c, n=1):
    """Depth-stream write of n entries per token: new K/V read once, written once."""
    return 2 * (2 * c["B"] * c["Hkv"] * c["T"] * n * c["d"] * es(c))


def decode_bytes(c):
    """Decode step: the KV cache and the new token's depth K/V once, q and O."""
    B, Hq, Hkv, T, L, d = c["B"], c["Hq"], c["Hkv"], c["T"], c["L"], c["d"]
    return es(c) * (2 * B * Hkv * T * d + 2 * B * Hkv * L * d + 2 * B * Hq * d)


def fwd_kernel_name(c):
    """Name of the fused kernel instance moda_fwd launches for workload c."""
    from depth_wise_kv_amd import moda
    v = moda.moda_fwd_variant(moda.make_shape(c["B"], c["Hq"], c["Hkv"], c["T"], c["L"], c["d"],
                                              c["dtype"]))
    if v.startswith("mfma_bf16_d128"):
        return {"w4": "moda_fwd_mfma<1, 4, 128>", "w8": "moda_fwd_mfma<1, 8, 256>",
                "ks": "moda_fwd_mfma<1, 8, 128>"}[v.rsplit("_", 1)[1]]
    if v.startswith("mfma_"):  # the kernel for the other head dims and fp32
        e = "float" if c["dtype"] == "f32" else "unsigned short"
        return f"moda_fwd_small<{e}, {c['d']}, true, {'true' if c['L'] else 'false'}>"
    return "moda_fwd_generic"


def roofline(c, fwd_ms, traffic):
    """Roofline of the fused kernel: matrix-core-bound when its arithmetic
    intensity (algorithmic flops per algorithmic HBM byte) is above the ridge
    point of the two published peaks, HBM-bound below it."""
    ai = flops(c) / fused_bytes(c)
    peak = PEAK_BF16_TFLOPS if c["dtype"] == "bf16" else PEAK_F32_TFLOPS
    if ai >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        a = flops(c) / fwd_ms / 1e9
        return {"bound": "mfma", "kernel": fwd_kernel_name(c), "achieved": a,
                "peak": peak, "unit": "TFLOP/s", "frac": a / peak, "traffic": traffic}
    a = fused_bytes(c) / fwd_ms / 1e6
    return {"bound": "hbm", "kernel": fwd_kernel_name(c), "achieved": a,
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": a / PEAK_HBM_GBS, "traffic": traffic}


def kernel_src_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(name):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha") != kernel_src_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cold_cache(c):
    """True when a warm last-level cache could hold a noticeable share of what
    one call reads (algorithmic bytes between a quarter of it and 16 times it):
    such calls are timed cold, the cache overwritten before each."""
    return MALL_BYTES // 4 < fused_bytes(c) < 16 * MALL_BYTES


class CacheFlush:
    """Overwrites the last-level cache (and the L2s) with a 512 MiB fill."""

    def __init__(self, dev):
        import torch
        self.buf = torch.empty(2 * MALL_BYTES, dtype=torch.uint8, device=dev)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(self.n & 0xFF)


def timed(fn, steps, stream, graph=True, flush=None):
    """Durations (ms) of one call of fn, one sample per timed call or replay,
    from HIP events recorded on the stream the kernels run on.  Callers report
    the median (and the minimum where it is shown).
    - Calls of a millisecond or more: at least max(steps, 20) calls back to
      back, each between its own event pair.
    - Shorter calls, warm: `reps` calls are captured into a HIP graph and the
      graph is replayed max(steps, 100 // reps, 5) times, each replay between
      its own pair (issued one by one from Python, such calls would leave the
      GPU idle between kernels while the host prepares the next launch); the
      replays are timed twice and the second pass kept, since a process's
      first timed pass runs slow.  A sample is a replay's time over reps.
    - With `flush` (cold): each call runs after flush() on the same stream,
      at least max(steps, 20) calls (100 when under a millisecond), each
      between its own pair; the host enqueues ahead of the GPU, which is busy
      with the flush, so no launch gap enters the pair (timed that way without
      the flush, the pairs agree with the graph replay within 2%)."""
    import torch

    def pairs(n, body, before=None):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for ea, eb in evs:
            if before is not None:
                before()
            ea.record(stream)
            body()
            eb.record(stream)
        torch.cuda.synchronize()
        return np.array([ea.elapsed_time(eb) for ea, eb in evs])

    fn()
    torch.cuda.synchronize()
    est = float(pairs(1, fn)[0])
    if flush is not None:
        return pairs(max(steps, 20 if est >= 1.0 else 100), fn, flush)
    if graph and est < 1.0:
        reps = max(1, min(200, int(np.ceil(1.0 / max(est, 5e-3)))))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        n = max(steps, 100 // reps, 5)
        pairs(n, g.replay)
        t = pairs(n, g.replay) / reps
        del g
        return t
    return pairs(max(steps, 20), fn)


def finished_points(path):
    """Names of the sweep points whose lines a results file already holds
    (none if there is no file); a truncated last line counts as unfinished."""
    done = set()
    if not path or not os.path.exists(path):
        return done
    with open(path) as f:
        for line in f:
            try:
                rec = json.loads(line)
            except json.JSONDecodeError:
                continue
            if isinstance(rec, dict) and "config" in rec:
                done.add(rec["config"])
    return done


def emit_point(path, rec):
    """Print a sweep point's JSON line and, with a results file, append it
    there as one write followed by a flush to disk."""
    line = json.dumps(rec)
    print(line, flush=True)
    if path:
        # a run killed mid-write may have left a last line without its newline
        torn = False
        if os.path.exists(path) and os.path.getsize(path) > 0:
            with open(path, "rb") as f:
                f.seek(-1, os.SEEK_END)
                torn = f.read(1) != b"\n"
        with open(path, "a") as f:
            f.write(("\n" if torn else "") + line + "\n")
            f.flush()
            os.fsync(f.fileno())


def center(t, cold):
    """The duration a timing reports: the mean of warm samples (the average
    launch duration), the median of cold ones (a rare call after the cache
    overwrite stalls for milliseconds)."""
    return float(np.median(t) if cold else np.mean(t))


def cpu_baseline(cfg, d_in, budget_s=15.0, seed=0):
    """The fp64 oracle, as it stands, on a bounded random sample of rows."""
    import torch

    import oracle
    B, Hq, Hkv, T, L, d = (cfg[x] for x in ("B", "Hq", "Hkv", "T", "L", "d"))
    G = Hq // Hkv
    rng = np.random.default_rng(seed)

    def to_np(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
            else t.numpy()

    k, v = to_np(d_in["k"]), to_np(d_in["v"])

    def run(nrows):
        rows = np.stack([rng.integers(0, B, nrows), rng.integers(0, Hq, nrows),
                         rng.integers(0, T, nrows)], 1).astype(np.int64)
        rt = torch.from_numpy(rows).to(d_in["q"].device)
        b, h, t = rt[:, 0], rt[:, 1], rt[:, 2]
        qr = to_np(d_in["q"][b, h, t])
        kdr = to_np(d_in["kd"][b, h // G, t]) if L else None
        vdr = to_np(d_in["vd"][b, h // G, t]) if L else None
        t0 = time.perf_counter()
        oracle.moda_rows(rows, (B, Hq, Hkv, T, L, d), qr, k, v, kdr, vdr)
        dt = time.perf_counter() - t0
        work = 4.0 * d * float(np.sum(rows[:, 2] + 1 + L))
        return dt, work, nrows

    dt, work, n = run(32)                       # calibration
    rate_rows = n / max(dt, 1e-6)
    nrows = int(max(32, min(200000, rate_rows * budget_s)))
    dt, work, n = run(nrows)
    tflops = work / dt / 1e12
    full_s = flops(cfg) / (work / dt)
    # cores: the host CPUs this process may run on; threads: the OpenMP threads the
    # oracle ran with (OMP_NUM_THREADS, else one per core)
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": tflops, "unit": "TFLOP/s", "cores": cores,
            "threads": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} random (b,h,t) rows of the same workload, fp64, {dt:.1f} s; "
                      f"full workload extrapolated to {full_s:.0f} s",
            "rows": n, "seconds": dt, "rows_per_s": n / dt,
            "full_workload_s_extrapolated": full_s}


def decode_inputs(cfg, d_in):
    """Decode inputs cut from a forward case: the last token's query and depth
    rows; the whole K/V is the cache."""
    import torch
    from depth_wise_kv_amd import moda
    T, L = cfg["T"], cfg["L"]
    q = d_in["q"][:, :, T - 1].contiguous()
    kd = d_in["kd"][:, :, T - 1].contiguous() if L else None
    vd = d_in["vd"][:, :, T - 1].contiguous() if L else None
    shape = moda.make_shape(cfg["B"], cfg["Hq"], cfg["Hkv"], T, L, cfg["d"], cfg["dtype"])
    ws = torch.empty(max(16, moda.moda_decode_workspace_bytes(shape)), dtype=torch.uint8,
                     device=q.device)
    return q, kd, vd, ws


def time_decode(cfg, d_in, steps, stream, reps=20, given=None):
    """Mean duration of one decode call (both of its kernels), over steps*reps
    calls replayed from a graph."""
    import torch
    from depth_wise_kv_amd import moda
    if given is None:
        q, kd, vd, ws = decode_inputs(cfg, d_in)
    else:
        q, kd, vd = given
        shape = moda.make_shape(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], cfg["L"], cfg["d"],
                                cfg["dtype"])
        ws = torch.empty(max(16, moda.moda_decode_workspace_bytes(shape)), dtype=torch.uint8,
                         device=q.device)
    out = torch.empty_like(q)

    def dec():
        for _ in range(reps):
            moda.decode(q, d_in["k"], d_in["v"], kd, vd, out=out, workspace=ws)

    # replayed from a HIP graph, so the host's per-call launch cost (tens of
    # microseconds through Python) does not hide the device time
    dec()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dec()
    graph.replay()
    torch.cuda.synchronize()
    ms = float(np.mean(timed(graph.replay, steps, stream, graph=False))) / reps
    del graph
    return ms


# Decode shapes (B, Hq, Hkv, T, L): the forward workloads' heads and lengths,
# plus serving batches of many sequences.
DECODE_SWEEP = [(1, 16, 4, 65536, 32), (4, 32, 8, 8192, 128), (2, 16, 4, 4096, 24),
                (1, 16, 4, 4096, 24), (32, 16, 4, 8192, 24), (64, 16, 4, 4096, 24),
                (8, 32, 8, 32768, 64), (16, 16, 16, 16384, 32)]


def stack_run(cfg, steps):
    """A stack of L+1 layers at one layer's shape, each attending over the depth
    entries its predecessors wrote (layer l: L = l), three ways:
      layer-major stream: layer l writes its K/V as slice l of [L+1, B, Hkv, T, d]
        (zero-copy) and moda_fwd_layers reads the first l slices;
      packed, repacked per layer: the first l entries repacked, then moda_fwd;
      natural, per layer: moda_fwd_natural over a contiguous [B, Hkv, T, l, d];
      natural with room: layer l writes entry l of [B, Hkv, T, L+1, d] in place
        and moda_fwd_strided reads the first l entries of every token.
    Inputs are reused across layers (timing only).  Prints one JSON line."""
    import torch
    from depth_wise_kv_amd import moda
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    B, Hq, Hkv, T, NL, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], cfg["L"] + 1, cfg["d"]
    g = torch.Generator(device=dev)
    g.manual_seed(7000)
    r = lambda *sh: torch.randn(*sh, generator=g, device=dev).to(torch.bfloat16)
    q, k, v = r(B, Hq, T, d), r(B, Hkv, T, d), r(B, Hkv, T, d)
    kl, vl = r(NL, B, Hkv, T, d), r(NL, B, Hkv, T, d)
    out = torch.empty_like(q)
    nat = {l: (kl[:l].permute(1, 2, 3, 0, 4).contiguous(), vl[:l].permute(1, 2, 3, 0, 4).contiguous())
           for l in range(1, NL)}
    packed = {l: torch.empty(moda.moda_depth_cache_bytes(moda.make_shape(B, Hq, Hkv, T, l, d, "bf16")),
                             dtype=torch.uint8, device=dev) for l in range(1, NL)}

    def layer_major():
        for l in range(NL):
            moda.fwd_layers(q, k, v, kl if l else None, vl if l else None, l, out=out)

    def packed_per_layer():
        for l in range(NL):
            if l:
                shape = moda.make_shape(B, Hq, Hkv, T, l, d, "bf16")
                moda.pack_depth_cache(nat[l][0], nat[l][1], shape, out=packed[l])
                moda.fwd(q, k, v, packed[l], l, out=out)
            else:
                moda.fwd(q, k, v, None, 0, out=out)

    kc, vc = kl.permute(1, 2, 3, 0, 4).contiguous(), vl.permute(1, 2, 3, 0, 4).contiguous()

    def natural_room():
        for l in range(NL):
            moda.fwd_capacity(q, k, v, kc if l else None, vc if l else None, l, out=out)

    def natural_per_layer():
        for l in range(NL):
            moda.fwd_natural(q, k, v, nat[l][0] if l else None, nat[l][1] if l else None, out=out)

    res = {"stack": f"{NL} layers at B{B} Hq{Hq} Hkv{Hkv} T{T} d{d}, layer l reads l depth entries"}
    for name, fn in (("layer_major_ms", layer_major), ("packed_repack_per_layer_ms", packed_per_layer),
                     ("natural_per_layer_ms", natural_per_layer),
                     ("natural_with_room_ms", natural_room)):
        fn()
        res[name] = float(np.mean(timed(fn, steps, stream)))
    print(json.dumps(res), flush=True)


def decode_sweep(steps):
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(6000)
    for B, Hq, Hkv, T, L in DECODE_SWEEP:
        c = dict(B=B, Hq=Hq, Hkv=Hkv, T=T, L=L, d=128, dtype="bf16")
        r = lambda *sh: torch.randn(*sh, generator=g, device=dev).to(torch.bfloat16)
        d_in = {"q": None, "k": r(B, Hkv, T, 128), "v": r(B, Hkv, T, 128)}
        q = r(B, Hq, 128)
        kd, vd = (r(B, Hkv, L, 128), r(B, Hkv, L, 128)) if L else (None, None)
        ms = time_decode(c, d_in, steps, stream, given=(q, kd, vd))
        print(json.dumps({"decode": f"B{B}_Hq{Hq}_Hkv{Hkv}_T{T}_L{L}", "us": ms * 1e3,
                          "hbm_gbs": decode_bytes(c) / ms / 1e6,
                          "pct_hbm_peak": 100.0 * decode_bytes(c) / ms / 1e6 / PEAK_HBM_GBS}),
              flush=True)
        del d_in, q, kd, vd
        torch.cuda.empty_cache()


def bench_config(cfg, steps, warmup, with_cpu, causal=True, with_bwd=True, ablation=False):
    import torch
    from depth_wise_kv_amd import moda
    from synth import torch_inputs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    d_in = torch_inputs(cfg, dev)
    q, k, v, kd, vd = (d_in[n] for n in ("q", "k", "v", "kd", "vd"))
    L = cfg["L"]
    shape = moda.make_shape(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], L, cfg["d"], cfg["dtype"])
    packed = (torch.empty(moda.moda_depth_cache_bytes(shape), dtype=torch.uint8, device=dev)
              if L else None)
    out = torch.empty_like(q)
    # calls whose data a warm 256 MB last-level cache could partly hold are
    # timed cold (fwd, causal, pack, depth alone, natural and layer-major forms)
    fl = CacheFlush(dev) if cold_cache(cfg) else None
    torch.cuda.synchronize()

    def pack():
        if L:
            moda.pack_depth_cache(kd, vd, shape, out=packed)

    def fwd():
        moda.fwd(q, k, v, packed, L, out=out)

    def step():
        pack()
        fwd()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # whole-step wall clock over exactly `steps` steps
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    # per-kernel durations (HIP events on the stream the kernels run on)
    cold = fl is not None
    fwd_t = timed(fwd, steps, stream, flush=fl)
    fwd_ms = center(fwd_t, cold)
    fwd_median_ms, fwd_min_ms = float(np.median(fwd_t)), float(np.min(fwd_t))
    fwd_warm_ms = float(np.mean(timed(fwd, steps, stream))) if cold else None
    pack_ms = center(timed(pack, steps, stream, flush=fl), cold) if L else 0.0
    causal_ms = causal_min_ms = None
    if causal:
        cout = torch.empty_like(q)
        moda.causal_fwd(q, k, v, out=cout)
        causal_t = timed(lambda: moda.causal_fwd(q, k, v, out=cout), steps, stream, flush=fl)
        causal_ms, causal_min_ms = center(causal_t, cold), float(np.min(causal_t))
    natural_ms = None
    if L and cfg["dtype"] == "bf16" and cfg["d"] == 128:
        nout = torch.empty_like(q)
        moda.fwd_natural(q, k, v, kd, vd, out=nout)
        natural_ms = center(timed(lambda: moda.fwd_natural(q, k, v, kd, vd, out=nout),
                                  steps, stream, flush=fl), cold)
    scan_ms = None
    if ablation and L and cfg["dtype"] == "bf16" and cfg["d"] == 128 and cfg["T"] <= 16384:
        # layout ablation: the Flash-compatible masked scan over the flat depth axis
        sout = torch.empty_like(q)
        moda.fwd_masked_scan(q, k, v, kd, vd, out=sout)
        scan_ms = float(np.mean(timed(lambda: moda.fwd_masked_scan(q, k, v, kd, vd, out=sout),
                                      max(1, steps // 2), stream)))
        del sout
    unaware_ms = None
    G = cfg["Hq"] // cfg["Hkv"]
    if ablation and L and G > 1:
        # layout ablation, group-unaware: each query head of a group runs on its own (G
        # launches with one head per KV head), so every head reads the depth span itself
        q_heads = [q[:, j::G].contiguous() for j in range(G)]
        o_heads = [torch.empty_like(x) for x in q_heads]

        def unaware():
            for x, o in zip(q_heads, o_heads):
                moda.fwd(x, k, v, packed, L, out=o)

        unaware()
        unaware_ms = float(np.mean(timed(unaware, steps, stream)))
        del q_heads, o_heads
    pertoken_ms = None
    if (ablation and cfg["dtype"] == "bf16" and cfg["d"] == 128 and cfg["T"] <= 16384
            and cfg["Hq"] // cfg["Hkv"] <= 32):
        # layout ablation, naive per-token loop: token t alone (one decode call over the
        # cache's first t+1 keys and its own depth entries), T launches from the host
        T = cfg["T"]
        q_t = q.permute(2, 0, 1, 3).contiguous()
        kd_t = kd.permute(2, 0, 1, 3, 4).contiguous() if L else None
        vd_t = vd.permute(2, 0, 1, 3, 4).contiguous() if L else None
        lens = (torch.arange(1, T + 1, dtype=torch.int32, device=dev)[:, None]
                .expand(T, cfg["B"]).contiguous())
        o_t = torch.empty_like(q_t)
        ws = torch.empty(max(16, moda.moda_decode_workspace_bytes(shape)), dtype=torch.uint8,
                         device=dev)

        def pertoken():
            for t in range(T):
                moda.decode(q_t[t], k, v, kd_t[t] if L else None, vd_t[t] if L else None,
                            out=o_t[t], workspace=ws, cache_lens=lens[t])

        pertoken()
        pertoken_ms = float(np.mean(timed(pertoken, 2, stream, graph=False)))
        del q_t, kd_t, vd_t, lens, o_t, ws
    layers_ms = None
    if L and cfg["dtype"] == "bf16" and cfg["d"] == 128:
        # the same entries as per-layer slices [L,B,Hkv,T,d] (moda_fwd_layers)
        kl = kd.permute(3, 0, 1, 2, 4).contiguous()
        vl = vd.permute(3, 0, 1, 2, 4).contiguous()
        lout = torch.empty_like(q)
        moda.fwd_layers(q, k, v, kl, vl, out=lout)
        layers_ms = center(timed(lambda: moda.fwd_layers(q, k, v, kl, vl, out=lout),
                                 steps, stream, flush=fl), cold)
        del kl, vl, lout
    append_ms = None
    if L:
        # the depth-stream write of one layer: entry L-1 of every token, in place
        k_new = kd[:, :, :, L - 1].contiguous()
        v_new = vd[:, :, :, L - 1].contiguous()
        moda.append_depth(packed, shape, L - 1, k_new, v_new)
        append_ms = float(np.mean(timed(lambda: moda.append_depth(packed, shape, L - 1, k_new,
                                                                   v_new), steps, stream)))
        del k_new, v_new
    append2_ms = None
    if L >= 2:
        # a layer that writes two entries (attention K/V and the FFN's KV projection)
        k_new = kd[:, :, :, L - 2:].contiguous()
        v_new = vd[:, :, :, L - 2:].contiguous()
        moda.append_depth(packed, shape, L - 2, k_new, v_new)
        append2_ms = float(np.mean(timed(lambda: moda.append_depth(packed, shape, L - 2, k_new,
                                                                    v_new), steps, stream)))
        del k_new, v_new
    depth_ms = None
    if L:
        dout = torch.empty_like(q)
        moda.depth_fwd(q, packed, cfg["Hkv"], L, out=dout)
        depth_ms = center(timed(lambda: moda.depth_fwd(q, packed, cfg["Hkv"], L, out=dout),
                                steps, stream, flush=fl), cold)
    decode_ms = None
    if cfg["dtype"] == "bf16" and cfg["d"] == 128 and cfg["Hq"] // cfg["Hkv"] <= 32:
        decode_ms = time_decode(cfg, d_in, steps, stream)
    bwd_ms = None
    if with_bwd and cfg["dtype"] == "bf16" and cfg["d"] == 128 and cfg["Hq"] // cfg["Hkv"] <= 32:
        # backward of the same step: O, LSE from the forward, a seeded dO
        o_b, lse_b = moda.fwd(q, k, v, packed, L, with_lse=True)
        g = torch.Generator(device=dev)
        g.manual_seed(cfg.get("seed", 0) + 5)
        dout = torch.randn(q.shape, generator=g, device=dev, dtype=torch.float32).to(q.dtype)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty_like(kd) if L else None, torch.empty_like(vd) if L else None)
        delta = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        ws_n = moda.moda_bwd_workspace_bytes(shape)
        bwd_ws = torch.empty((ws_n,), dtype=torch.uint8, device=dev) if ws_n else None

        def bwd():
            moda.bwd(q, k, v, o_b, lse_b, dout, kd if L else None, vd if L else None, packed,
                     grads=grads, delta=delta, workspace=bwd_ws)

        bwd()
        bwd_ms = float(np.mean(timed(bwd, steps, stream)))
        del o_b, lse_b, dout, grads, delta, bwd_ws
    del fl
    res = dict(wall_ms=wall_ms, fwd_ms=fwd_ms, fwd_median_ms=fwd_median_ms, fwd_min_ms=fwd_min_ms,
               causal_min_ms=causal_min_ms,
               fwd_warm_ms=fwd_warm_ms, pack_ms=pack_ms,
               cache="cold" if cold_cache(cfg) else "warm", causal_ms=causal_ms,
               depth_ms=depth_ms, bwd_ms=bwd_ms, natural_ms=natural_ms, decode_ms=decode_ms,
               append_ms=append_ms, append2_ms=append2_ms, layers_ms=layers_ms,
               scan_ms=scan_ms, pertoken_ms=pertoken_ms,
               unaware_ms=unaware_ms)
    if with_cpu:
        res["cpu_baseline"] = cpu_baseline(cfg, d_in)
    del d_in, packed, out
    torch.cuda.empty_cache()
    return res


def profile_only(cfg, which, steps):
    """Launch one kernel `steps` times on the workload (for rocprofv3 --pmc)."""
    import torch
    from depth_wise_kv_amd import moda
    from synth import torch_inputs
    dev = torch.device("cuda:0")
    d_in = torch_inputs(cfg, dev)
    L = cfg["L"]
    shape = moda.make_shape(cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["T"], L, cfg["d"], cfg["dtype"])
    packed = moda.pack_depth_cache(d_in["kd"], d_in["vd"], shape) if L else None
    out = torch.empty_like(d_in["q"])
    if which == "bwd":
        o_b, lse_b = moda.fwd(d_in["q"], d_in["k"], d_in["v"], packed, L, with_lse=True)
        dout = torch.randn_like(d_in["q"], dtype=torch.float32).to(d_in["q"].dtype)
        kd, vd = (d_in["kd"], d_in["vd"]) if L else (None, None)
    if which == "decode":
        dq, dkd, dvd, dws = decode_inputs(cfg, d_in)
        dout_ = torch.empty_like(dq)
    if which == "append":
        k_new = d_in["kd"][:, :, :, L - 1].contiguous()
        v_new = d_in["vd"][:, :, :, L - 1].contiguous()
    torch.cuda.synchronize()
    for _ in range(steps):
        if which == "fwd":
            moda.fwd(d_in["q"], d_in["k"], d_in["v"], packed, L, out=out)
        elif which == "causal":
            moda.causal_fwd(d_in["q"], d_in["k"], d_in["v"], out=out)
        elif which == "depth":
            moda.depth_fwd(d_in["q"], packed, cfg["Hkv"], L, out=out)
        elif which == "decode":
            moda.decode(dq, d_in["k"], d_in["v"], dkd, dvd, out=dout_, workspace=dws)
        elif which == "append":
            moda.append_depth(packed, shape, L - 1, k_new, v_new)
        elif which == "bwd":
            moda.bwd(d_in["q"], d_in["k"], d_in["v"], o_b, lse_b, dout, kd, vd, packed)
        else:
            moda.pack_depth_cache(d_in["kd"], d_in["vd"], shape, out=packed)
    torch.cuda.synchronize()
    print(json.dumps({"profiled": which, "workload": cfg, "launches": steps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="long_64k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--sweep-bwd", action="store_true",
                    help="with --sweep: also time the backward at every point")
    ap.add_argument("--ablation", action="store_true",
                    help="also time the group-unaware and masked-scan layout ablations (the "
                         "group-unaware one launches moda_fwd's kernel at other shapes)")
    ap.add_argument("--stack", action="store_true",
                    help="time a stack of L+1 layers at the config's shape (layer l reads l depth "
                         "entries): layer-major stream vs per-layer repack vs natural layout")
    ap.add_argument("--decode-sweep", action="store_true",
                    help="time the decode step on the decode shapes (one JSON line each)")
    ap.add_argument("--only", default=None,
                    help="with --sweep: run only points whose name contains this string")
    ap.add_argument("--results", default=None,
                    help="with --sweep: also append each finished point's JSON line to this "
                         "file, and skip the points it already holds (an interrupted sweep "
                         "resumes where it stopped)")
    ap.add_argument("--profile-kernel", choices=["fwd", "causal", "pack", "depth", "bwd", "decode", "append"],
                    help="only launch this kernel (steps times) for counter collection")
    ap.add_argument("--gemm-reference", type=int, default=0, metavar="N",
                    help="time a bf16 N x N x N torch.matmul (hipBLASLt): the practical "
                         "matrix-core rate of this GPU under its power limit, for context")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="copy a 1 GiB buffer (steps times): HBM counter calibration")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); sharding over "
              "several GPUs is not implemented", file=sys.stderr)
        sys.exit(2)

    from synth import WORKLOADS, sweep_points

    if args.gemm_reference:
        import torch
        n = args.gemm_reference
        a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
        b_ = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16)
        for _ in range(max(args.warmup, 1)):
            c = a @ b_
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            c = a @ b_
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        del c
        print(json.dumps({"gemm": f"bf16 {n}x{n}x{n} torch.matmul", "ms": ms,
                          "tflops": 2.0 * n ** 3 / ms / 1e9,
                          "pct_bf16_peak": 100.0 * 2.0 * n ** 3 / ms / 1e9 / PEAK_BF16_TFLOPS}),
              flush=True)
        return
    if args.copy_calibration:
        import torch
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"copy_bytes_per_launch": n, "launches": args.steps + 1,
                          "ms_per_copy": ms, "read_plus_write_gbs": 2 * n / ms / 1e6}),
              flush=True)
        return
    named = dict(WORKLOADS)
    named.update({c["name"]: c for c in sweep_points()})
    if args.config not in named:
        print(f"bench.py: unknown config {args.config!r}", file=sys.stderr)
        sys.exit(2)
    if args.profile_kernel:
        profile_only(dict(named[args.config]), args.profile_kernel, args.steps)
        return

    if args.decode_sweep:
        decode_sweep(args.steps)
        return
    if args.stack:
        stack_run(dict(named[args.config]), args.steps)
        return
    if args.sweep:
        done = finished_points(args.results)
        for c in sweep_points():
            if args.only and args.only not in c["name"]:
                continue
            if c["name"] in done:
                print(f"bench.py: {c['name']} already in {args.results}; skipped",
                      file=sys.stderr, flush=True)
                continue
            r = bench_config(c, args.steps, args.warmup, False, causal=True,
                             with_bwd=args.sweep_bwd, ablation=args.ablation)
            emit_point(args.results, {"config": c["name"], "T": c["T"], "L": c["L"],
                              "G": c["Hq"] // c["Hkv"], "fwd_ms": r["fwd_ms"],
                              "fwd_warm_cache_ms": r["fwd_warm_ms"],
                              "kernel_timing_cache": r["cache"],
                              "pack_ms": r["pack_ms"], "causal_ms": r["causal_ms"],
                              "fwd_tflops": flops(c) / r["fwd_ms"] / 1e9,
                              "causal_tflops": flops(c, 0) / r["causal_ms"] / 1e9,
                              "ratio_fwd_over_causal": r["fwd_ms"] / r["causal_ms"],
                              "fwd_hbm_gbs": fused_bytes(c) / r["fwd_ms"] / 1e6,
                              "fwd_natural_layout_ms": r["natural_ms"],
                              "fwd_layer_major_ms": r["layers_ms"],
                              "fwd_masked_scan_ms": r["scan_ms"],
                              "fwd_group_unaware_ms": r["unaware_ms"],
                              "depth_only_ms": r["depth_ms"],
                              "depth_only_hbm_gbs": (depth_bytes(c) / r["depth_ms"] / 1e6
                                                     if r["depth_ms"] else None),
                              "decode_us": r["decode_ms"] * 1e3 if r["decode_ms"] else None,
                              "decode_hbm_gbs": (decode_bytes(c) / r["decode_ms"] / 1e6
                                                 if r["decode_ms"] else None),
                              "bwd_ms": r["bwd_ms"],
                              "bwd_tflops": (2.5 * flops(c) / r["bwd_ms"] / 1e9
                                             if r["bwd_ms"] else None)})
        return

    cfg = dict(named[args.config])
    r = bench_config(cfg, args.steps, args.warmup, not args.no_cpu_baseline,
                     ablation=args.ablation)
    F = flops(cfg)
    step_ms = r["wall_ms"]
    fwd_tflops = F / r["fwd_ms"] / 1e9
    traffic = load_traffic(f"fwd_{args.config}")
    line = {
        "metric": METRIC,
        "value": F / step_ms / 1e9,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": args.config, "B": cfg["B"], "Hq": cfg["Hq"], "Hkv": cfg["Hkv"],
                   "T": cfg["T"], "L": cfg["L"], "d": cfg["d"], "inputs": "N(0,1) seeded",
                   "step": "moda_pack_depth_cache + moda_fwd"},
        "fwd_ms": r["fwd_ms"],
        "fwd_median_ms": r["fwd_median_ms"],
        "fwd_min_ms": r["fwd_min_ms"],
        "fwd_warm_cache_ms": r["fwd_warm_ms"],
        "kernel_timing_cache": r["cache"],
        "pack_ms": r["pack_ms"],
        "causal_ms": r["causal_ms"],
        "causal_min_ms": r["causal_min_ms"],
        "fwd_tflops": fwd_tflops,
        "fwd_pct_bf16_peak": 100.0 * fwd_tflops / PEAK_BF16_TFLOPS,
        "step_pct_bf16_peak": 100.0 * (F / step_ms / 1e9) / PEAK_BF16_TFLOPS,
        "causal_tflops": flops(cfg, 0) / r["causal_ms"] / 1e9,
        "ratio_fwd_over_causal": r["fwd_ms"] / r["causal_ms"],
        "ratio_step_over_causal": step_ms / r["causal_ms"],
        "pack_hbm_gbs": pack_bytes(cfg) / r["pack_ms"] / 1e6 if r["pack_ms"] else None,
        "fwd_hbm_gbs": fused_bytes(cfg) / r["fwd_ms"] / 1e6,
        "depth_only_ms": r["depth_ms"],
        "depth_only_hbm_gbs": depth_bytes(cfg) / r["depth_ms"] / 1e6 if r["depth_ms"] else None,
        "fwd_natural_layout_ms": r["natural_ms"],
        "fwd_layer_major_ms": r["layers_ms"],
        "fwd_masked_scan_ms": r["scan_ms"],
        "fwd_group_unaware_ms": r["unaware_ms"],
        "fwd_per_token_loop_ms": r["pertoken_ms"],
        "bwd_ms": r["bwd_ms"],
        "bwd_tflops": 2.5 * F / r["bwd_ms"] / 1e9 if r["bwd_ms"] else None,
        "decode_us": r["decode_ms"] * 1e3 if r["decode_ms"] else None,
        "decode_hbm_gbs": decode_bytes(cfg) / r["decode_ms"] / 1e6 if r["decode_ms"] else None,
        "append_us": r["append_ms"] * 1e3 if r["append_ms"] else None,
        "append_hbm_gbs": append_bytes(cfg) / r["append_ms"] / 1e6 if r["append_ms"] else None,
        "append2_us": r["append2_ms"] * 1e3 if r["append2_ms"] else None,
        "append2_hbm_gbs": (append_bytes(cfg, 2) / r["append2_ms"] / 1e6
                            if r["append2_ms"] else None),
        "roofline": roofline(cfg, r["fwd_ms"], traffic),
    }
    if "cpu_baseline" in r:
        line["cpu_baseline"] = r["cpu_baseline"]
        # the forward's speedup over the oracle's extrapolated full-workload time
        line["cpu_baseline"]["gpu_fwd_speedup"] = (
            r["cpu_baseline"]["full_workload_s_extrapolated"] * 1e3 / r["fwd_ms"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
