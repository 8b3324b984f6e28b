#!/usr/bin/env python3
"""Benchmark of the routed MoE layer served from an elastic expert cache, one MI355X.

A step is one decode step through every layer of the stack: per layer the router,
the cache decisions and the fetch split, the fills of F over PCIe, the CPU
branch for C on the host cores, the grouped SwiGLU FFN of H and F, and the merge.
Headline workload: 43 stacked layers, d=4096, E=256, top-6, d_ff=2048, bf16
experts in pinned host memory, batch 1, GPU cache 11 % of the (layer, expert)
pairs (1210 slots), Zipf(1.1) popularity with 0.6 step-to-step reuse, fetch
fraction from B_P and B_H measured on this machine.  The cache is warmed by at
least 64 trace steps before timing, whatever --warmup says.  Inputs are seeded and
synthetic, resident in HBM (activations, router weights, routing masks) or pinned
host memory (the pool) before the timed region starts.

Also measured: the 40-layer d=2048, E=128, top-8, d_ff=768 stack (cache 37 %) at
batch 1, without the at-least-one-fill floor (min_fill = 0), and at batch 8
(unless --no-config2); one 8192-token prefill chunk through the 43-layer shape with
full-layer double buffering, and with the second buffer off (unless --no-prefill);
the same shape with MXFP4 experts: a 16384-token prefill as two 8192-token chunks on
the scaled MFMA, then batch-1 decode over a 512-step trace with the cache resized
from 1210 to 605 slots at step 256 (unless --no-mxfp4); the placement replay.

--counter-calibration runs only a plain device copy of known size (for scaling
rocprofv3's FETCH_SIZE and WRITE_SIZE to bytes) and prints its own JSON line.

Prints one JSON line.  --gpus N > 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE decode tok/s + 8k-token prefill tok/s (DSV4 shape); % of HBM/MFMA peak"
HEADLINE = "decode-L43-d4096-E256-top6"
CONFIG2 = "decode-L40-d2048-E128-top8"
CACHE_WARMUP_STEPS = 64  # trace steps that warm the cold cache before any timed step
# physical layers of the pinned pool when --l-phys is 0: the 43-layer bf16 pool
# (554 GB) does not fit host memory, so it aliases 4 physical layers (51.5 GB);
# keys, bytes moved and timing are those of the logical pool
L_PHYS_DEFAULT = {HEADLINE: 4}
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published (E4M3 x E2M1 runs at the fp8 rate)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str):
    """Hash of one kernel's definition in kernels.hip (from its signature to the first
    closing brace at column 0), so that counters stay valid while other kernels change."""
    src = open(os.path.join(ROOT, "moe_expert_offload_amd", "csrc", "kernels.hip")).read()
    at = src.find(f"void {kernel}(")
    if at < 0:
        return None
    end = src.find("\n}\n", at)
    return hashlib.sha256(src[at:end].encode()).hexdigest()[:16]


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were
    taken on the current kernel source (profiles/<kernel>__<workload>.counters.txt)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def default_l_phys(args, wl):
    s = wl.shape
    if args.l_phys > 0:
        return min(args.l_phys, s.L)
    return L_PHYS_DEFAULT.get(wl.name, s.L)


def phased_time(m, q, S, B_P, B_H):
    # fills at B_P; host branch at B_H - B_P while the link is busy, B_H after
    t_fill = q * S / B_P if q > 0 else 0.0
    rest = (m - q) * S
    done = max(B_H - B_P, 0.0) * t_fill
    return t_fill if done >= rest else t_fill + (rest - done) / B_H


def bw_profile(ft, fshape, pool, scratch, B_P, B_H):
    """The contended pair next to B_P and B_H: both fetch fractions and the 2x hybrid gate
    (the split itself uses Eq. 4, B_P / B_H)."""
    po, co = ft.ft_bench_bw_contended(fshape, pool.ptr, 64, scratch, 0)
    return {"pcie_ov_GBs": round(po / 1e9, 2), "cpu_ov_GBs": round(co / 1e9, 2),
            "frac_q16_eq4": ft.ft_frac_q16(B_P, B_H), "frac_q16_contended": ft.ft_frac_q16_contended(po, co),
            "hybrid_gate_2x": ft.ft_recommend_hybrid([B_P], [B_H], 2.0)}


def run_decode(args, torch, ft, synth, HostPool, workload=None, steps=None, warmup=None, overrides=None,
               pool=None):
    if workload is not None:  # a further decode leg with its own sizes
        args = argparse.Namespace(**{**vars(args), "workload": workload, "steps": steps, "warmup": warmup})
    if overrides:
        args = argparse.Namespace(**{**vars(args), **overrides})
    wl = synth.WORKLOADS[args.workload]
    s = wl.shape
    T = wl.T
    S = s.record_bytes
    # the cache starts cold: at least CACHE_WARMUP_STEPS trace steps run before timing
    warm = max(CACHE_WARMUP_STEPS, args.warmup)
    steps_total = warm + args.steps
    steps_gen = steps_total + args.steps  # a second pass over further steps carries the kernel timing
    L_phys = default_l_phys(args, wl)
    log(f"decode workload {wl.name}: pool {L_phys * s.E} records x {S / 1e6:.2f} MB = {L_phys * s.E * S / 1e9:.1f} GB")
    if pool is None:
        t = time.time()
        pool = HostPool(L_phys * s.E, s.record_bytes, s.pool_dtype)
        synth.fill_records_torch(pool.view, wl.seed_key, seed=args.seed)
        log(f"pool allocated and filled in {time.time() - t:.1f} s")

    fshape = ft.make_shape(s.L, s.E, s.d, s.d_ff, s.k)
    scratch = torch.empty(64 * S, dtype=torch.uint8, device="cuda")
    B_P, B_H = ft.ft_bench_bw(fshape, pool.ptr, 64, scratch, 0)
    bwp = bw_profile(ft, fshape, pool, scratch, B_P, B_H)
    del scratch
    fq = ft.ft_frac_q16(B_P, B_H) if args.frac_q16 < 0 else args.frac_q16
    log(f"B_P {B_P / 1e9:.1f} GB/s, B_H {B_H / 1e9:.1f} GB/s, frac_q16 {fq}")

    wr = [torch.from_numpy(synth.router_weights(wl, l, seed=args.seed).view(np.int16)).cuda() for l in range(s.L)]
    tr = synth.trace_for(wl, seed=args.seed, steps=steps_gen)
    allowed = np.zeros((steps_gen, s.L, T, s.E), dtype=np.uint8)
    st_i, l_i, b_i = np.meshgrid(np.arange(steps_gen), np.arange(s.L), np.arange(T), indexing="ij")
    for j in range(s.k):
        allowed[st_i, l_i, b_i, tr[:, :, :, j].astype(np.int64)] = 1
    allowed_d = torch.from_numpy(allowed).cuda()
    xh = np.empty((steps_gen, s.L, T, s.d), dtype=np.uint16)
    for st in range(steps_gen):
        for l in range(s.L):
            xh[st, l] = synth.tokens(wl, st, l, T=T, seed=args.seed)
    xs = torch.from_numpy(xh.view(np.int16)).cuda()
    del xh
    ys = torch.empty((s.L, T, s.d), dtype=torch.float32, device="cuda")

    N = wl.n_slots
    cfg = ft.make_config(frac_q16=fq, min_fill=args.min_fill, max_fetch=args.max_fetch, cpu_threads=args.cpu_threads,
                         prefill_overlap=0, T_max=T, L_phys=L_phys)
    slots = torch.empty(N * S, dtype=torch.uint8, device="cuda")
    wsb = ft.ft_workspace_bytes(fshape, T)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    ctx = ft.ft_create(fshape, cfg, pool.ptr, pool.nbytes, slots, N, ws, wsb)
    compute = torch.cuda.current_stream()
    st_call = ft.ft_step_stats()
    calls = []
    graph_mode = getattr(args, "mode", "eager") == "graph"
    graph = None
    if graph_mode:
        # fixed buffers the graph reads and writes; each step's inputs are copied in
        # (inside the timed region)
        xb = torch.empty((s.L, T, s.d), dtype=torch.int16, device="cuda")
        ab = torch.empty((s.L, T, s.E), dtype=torch.uint8, device="cuda")
        yb = torch.empty((s.L, T, s.d), dtype=torch.float32, device="cuda")
        graph = ft.ft_decode_graph_create(ctx, T, xb, wr, ab, yb)

    def step(st, record):
        if graph_mode:
            xb.copy_(xs[st])
            ab.copy_(allowed_d[st])
            ft.ft_decode_graph_launch(graph, compute)
            return
        for l in range(s.L):
            ft.ft_moe_decode_layer(ctx, l, xs[st, l], T, wr[l], allowed_d[st, l], ys[l], compute,
                                   None, st_call)
            if record:
                calls.append((st_call.hits, st_call.misses, st_call.q, st_call.n_c, st_call.t_cpu_us,
                               st_call.t_total_us, st_call.t_route_us, st_call.t_ctrl_us, st_call.t_issue_us,
                               st_call.t_cpu_work_us, st_call.cpu_caller_items, st_call.t_submit_us,
                               st_call.t_between_us))

    try:
        for st in range(warm):
            step(st, False)
        torch.cuda.synchronize()
        ft.ft_reset_stats(ctx)
        # timed region: the steps as they run in serving, no timing events
        t0 = time.perf_counter()
        for st in range(warm, steps_total):
            step(st, True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if graph_mode:
            ft.ft_decode_graph_status(graph)
        stats = ft.ft_get_stats(ctx)
        # second timed region over the next steps of the same trace: every grouped-FFN
        # kernel launched with start/stop events (for the roofline; eager calls only)
        prof = {"launches": 0, "ms_gateup": 0.0, "ms_down": 0.0, "bytes_gateup": 0.0, "bytes_down": 0.0}
        t2 = t3 = time.perf_counter()
        if not graph_mode:
            ft.ft_profile_enable(ctx, True)
            t2 = time.perf_counter()
            for st in range(steps_total, steps_total + args.steps):
                step(st, False)
            torch.cuda.synchronize()
            t3 = time.perf_counter()
            prof = ft.ft_profile_read(ctx)
            ft.ft_profile_enable(ctx, False)
    finally:
        if graph:
            ft.ft_decode_graph_destroy(graph)
        ft.ft_destroy(ctx)
    elapsed = t1 - t0
    ms_gu = prof["ms_gateup"] / max(prof["launches"], 1)
    ms_dn = prof["ms_down"] / max(prof["launches"], 1)
    bytes_gu = prof["bytes_gateup"] / max(prof["launches"], 1)
    bytes_dn = prof["bytes_down"] / max(prof["launches"], 1)
    gu_gbs = prof["bytes_gateup"] / (prof["ms_gateup"] * 1e-3) / 1e9 if prof["ms_gateup"] > 0 else 0.0
    dn_gbs = prof["bytes_down"] / (prof["ms_down"] * 1e-3) / 1e9 if prof["ms_down"] > 0 else 0.0
    # modelled floor of the timed steps: per call the slower of the GPU weight stream
    # and the miss path (fills at B_P next to the host branch, phase-aware)
    floor_s = 0.0
    for hits, misses, q, n_c, *_ in calls:
        floor_s += max((hits + q) * S / (HBM_PEAK_GBS * 1e9), phased_time(misses, q, S, B_P, B_H))
    reads = max(stats["reads"], 1)
    if graph_mode:
        # per-call records are not collected in graph mode: the floor from the counters
        floor_s = None
    res = {
        "mode": "graph" if graph_mode else "eager",
        "tok_s": args.steps * T / elapsed,
        "ms_per_step": elapsed / args.steps * 1e3,
        "workload": wl.name, "T": T, "L": s.L, "n_slots": N, "L_phys": L_phys, "cache_warmup_steps": warm,
        "timed_steps": args.steps,
        "B_P_GBs": B_P / 1e9, "B_H_GBs": B_H / 1e9, "frac_q16": fq, "bw_profile": bwp, "min_fill": args.min_fill,
        "cpu_threads": args.cpu_threads,
        "miss_rate_reads": 1.0 - stats["read_hits"] / reads,
        "miss_rate_unique": stats["unique_misses"] / max(stats["unique_hits"] + stats["unique_misses"], 1),
        "trace_reuse": trace_reuse(tr),
        "miss_rate_context": "the pages' LRU miss rates on their own traces: 16 % and 39 % (context, not a target)",
        "fills_per_step": stats["fills"] / args.steps, "cpu_experts_per_step": stats["cpu_experts"] / args.steps,
        "h2d_GB_per_step": stats["h2d_bytes"] / args.steps / 1e9,
        "modelled_floor_ms_per_step": floor_s / args.steps * 1e3 if floor_s is not None else None,
        "host_cpu_branch_ms_per_step": sum(c[4] for c in calls) / args.steps / 1e3,
        # rate of the host branch over its own work time (records of C per second)
        "cpu_branch_GBs": (sum(c[3] for c in calls) * S / (sum(c[9] for c in calls) * 1e-6) / 1e9
                           if calls and sum(c[9] for c in calls) > 0 else None),
        "host_call_us": {
            "route": float(np.mean([c[6] for c in calls])) if calls else 0.0,
            "ctrl": float(np.mean([c[7] for c in calls])) if calls else 0.0,
            "cpu_when_used": float(np.mean([c[4] for c in calls if c[3] > 0])) if any(c[3] > 0 for c in calls) else 0.0,
            "cpu_work_when_used": float(np.mean([c[9] for c in calls if c[3] > 0])) if any(c[3] > 0 for c in calls) else 0.0,
            "cpu_work_p50": float(np.percentile([c[9] for c in calls if c[3] > 0], 50)) if any(c[3] > 0 for c in calls) else 0.0,
            "cpu_work_p90": float(np.percentile([c[9] for c in calls if c[3] > 0], 90)) if any(c[3] > 0 for c in calls) else 0.0,
            "cpu_work_per_expert_p50": float(np.percentile([c[9] / c[3] for c in calls if c[3] > 0], 50)) if any(c[3] > 0 for c in calls) else 0.0,
            "issue": float(np.mean([c[8] for c in calls])) if calls else 0.0,
            "cpu_caller_items_when_used": float(np.mean([c[10] for c in calls if c[3] > 0])) if any(c[3] > 0 for c in calls) else 0.0,
            "cpu_items_when_used": float(np.mean([c[3] * 48 + 64 for c in calls if c[3] > 0])) if any(c[3] > 0 for c in calls) else 0.0,
            "issue_when_fill": float(np.mean([c[8] for c in calls if c[2] > 0])) if any(c[2] > 0 for c in calls) else 0.0,
            "total": float(np.mean([c[5] for c in calls])) if calls else 0.0,
            "submit": float(np.mean([c[11] for c in calls])) if calls else 0.0,
            "between_calls": float(np.mean([c[12] for c in calls])) if calls else 0.0,
        },
        "timed_with_kernel_events_ms_per_step": (t3 - t2) / args.steps * 1e3,
        "kernels": {
            "ffn_gateup_rows": {"avg_us": ms_gu * 1e3, "bytes_per_launch": bytes_gu, "GBs": gu_gbs,
                                "launches": prof["launches"]},
            "ffn_down_rows": {"avg_us": ms_dn * 1e3, "bytes_per_launch": bytes_dn, "GBs": dn_gbs},
        },
    }
    roofline = {"bound": "hbm", "kernel": "ffn_gateup_rows_kernel", "achieved": round(gu_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                "traffic": stored_traffic("ffn_gateup_rows_kernel", args.workload),
                "avg_launch_us": round(ms_gu * 1e3, 3), "algorithmic_bytes_per_launch": round(bytes_gu)}
    if T >= 4:
        # the library runs the hits' FFN beside the fills for 4 or more tokens
        roofline["schedule"] = "hits' FFN launched beside fill_kernel: durations include the overlap"
    return res, roofline, (pool, wl, tr, fq, L_phys)


def dma_h2d_rate(torch, nbytes=1 << 31, reps=3):
    """Rate of a plain pinned host -> device copy (the copy engine path the prefill's
    layer loads take), best of a few."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    best = 0.0
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src, non_blocking=True)
        b.record()
        b.synchronize()
        best = max(best, nbytes / (a.elapsed_time(b) * 1e-3))
    del src, dst
    return best


def trace_reuse(tr):
    """Empirical step-to-step reuse of a routing trace [steps, L, B, k]: the fraction of a
    step's experts (steps 1..) that its stream also took at the step before (the kept ones
    plus chance redraws)."""
    prev, cur = tr[:-1], tr[1:]
    hit = (cur[..., :, None] == prev[..., None, :]).any(axis=-1)
    return float(hit.mean()) if hit.size else None


def measured_peaks(torch, reps=5):
    """The box's own ceilings next to the rated ones: an HBM copy of 2 GiB (read + write
    bytes), a bf16 GEMM of 8192^3 (the library's), and a pinned host -> device copy; medians
    over `reps` after a warm-up.  (A read stream of LDS-direct loads at one block per compute
    unit, probed separately, reaches 6.0-6.4 TB/s.)"""
    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return sorted(ts)[len(ts) // 2]
    n = 1 << 31
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src))
    del src, dst
    m = 8192
    a = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    b = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    t_gemm = timed(lambda: torch.matmul(a, b))
    del a, b
    return {"hbm_copy_GBs": round(2 * n / t_copy / 1e9, 1),
            "bf16_gemm_TFLOPs": round(2.0 * m ** 3 / t_gemm / 1e12, 1),
            "h2d_copy_GBs": round(dma_h2d_rate(torch) / 1e9, 1),
            "rated": {"hbm_GBs": HBM_PEAK_GBS, "bf16_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                      "fp8_TFLOPs": MFMA_FP8_PEAK_TFLOPS, "pcie_gen5_x16_GBs": 63.0},
            "note": "copy: read + write bytes of a 2 GiB device copy; GEMM: torch.matmul (hipBLASLt), "
                    "contiguous operands; host copy: pinned memory by the copy engine"}


def run_prefill(args, torch, ft, synth, HostPool):
    wl = synth.WORKLOADS["prefill8k-L43-d4096-E256-top6"]
    s = wl.shape
    T = wl.T
    S = s.record_bytes
    L_phys = max(1, min(args.prefill_l_phys, s.L))
    log(f"prefill workload {wl.name}: pool {L_phys * s.E} records = {L_phys * s.E * S / 1e9:.1f} GB (aliased)")
    t = time.time()
    pool = HostPool(L_phys * s.E, s.record_bytes, s.pool_dtype)
    synth.fill_records_torch(pool.view, wl.seed_key, seed=args.seed)
    log(f"pool allocated and filled in {time.time() - t:.1f} s")
    try:
        fshape = ft.make_shape(s.L, s.E, s.d, s.d_ff, s.k)
        N = wl.n_slots
        cfg = ft.make_config(frac_q16=0, min_fill=0, max_fetch=0, cpu_threads=2, prefill_overlap=1, T_max=T,
                             L_phys=L_phys)
        slots = torch.empty(N * S, dtype=torch.uint8, device="cuda")
        wsb = ft.ft_workspace_bytes(fshape, T)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        wr = [torch.from_numpy(synth.router_weights(wl, l, seed=args.seed).view(np.int16)).cuda() for l in range(s.L)]
        xs = [synth.tokens_torch(wl.seed_key, 0, l, T, s.d, seed=args.seed) for l in range(s.L)]
        y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
        ctx = ft.ft_create(fshape, cfg, pool.ptr, pool.nbytes, slots, N, ws, wsb)
        compute = torch.cuda.current_stream()
        copy = torch.cuda.Stream()
        try:
            # warm-up: two layers
            ft.ft_moe_prefill_begin(ctx, copy)
            for l in range(2):
                ft.ft_moe_prefill_layer(ctx, l, xs[l], T, wr[l], y, compute, copy)
            ft.ft_moe_prefill_end(ctx)
            torch.cuda.synchronize()
            ft.ft_profile_enable(ctx, True)
            t0 = time.perf_counter()
            ft.ft_moe_prefill_begin(ctx, copy)
            for l in range(s.L):
                ft.ft_moe_prefill_layer(ctx, l, xs[l], T, wr[l], y, compute, copy)
            ft.ft_moe_prefill_end(ctx)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            prof = ft.ft_profile_read(ctx)
            ft.ft_profile_enable(ctx, False)
        finally:
            ft.ft_destroy(ctx)
        el_off = None
        if args.prefill_ablation:
            # the second buffer disabled: each layer's routed experts load on demand after
            # its routing, serialised against its compute
            cfg_off = ft.make_config(frac_q16=0, min_fill=0, max_fetch=0, cpu_threads=2, prefill_overlap=0, T_max=T,
                                     L_phys=L_phys)
            ctx = ft.ft_create(fshape, cfg_off, pool.ptr, pool.nbytes, slots, N, ws, wsb)
            try:
                log("prefill with overlap off (on-demand loading)")
                t2 = time.perf_counter()
                ft.ft_moe_prefill_begin(ctx, copy)
                for l in range(s.L):
                    ft.ft_moe_prefill_layer(ctx, l, xs[l], T, wr[l], y, compute, copy)
                ft.ft_moe_prefill_end(ctx)
                torch.cuda.synchronize()
                el_off = time.perf_counter() - t2
            finally:
                ft.ft_destroy(ctx)
        b_dma = dma_h2d_rate(torch)
    finally:
        pool.free()
    el = t1 - t0
    ms = prof["ms_gateup"] + prof["ms_down"]
    fl = prof["flops_gateup"] + prof["flops_down"]
    tflops = fl / (ms * 1e-3) / 1e12 if ms > 0 else 0.0
    by = prof["bytes_gateup"] + prof["bytes_down"]
    h2d = s.L * s.E * S
    t_xfer = h2d / b_dma
    t_comp_last = ms / max(prof["launches"], 1) * 1e-3
    # attainable at this shape: the weight stream at peak HBM bandwidth times the flops per weight byte
    ai = fl / max(prof["bytes_gateup"] + prof["bytes_down"], 1.0)
    attainable = min(MFMA_BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
    return {
        "tok_s": T / el, "s_per_chunk": el, "T": T, "L": s.L, "L_phys": L_phys, "n_slots": N,
        "h2d_GB": h2d / 1e9, "h2d_GBs_effective": h2d / el / 1e9,
        # overlap efficiency (sum of transfer times at the measured copy rate, plus the last
        # layer's compute) / wall time
        "dma_h2d_GBs": round(b_dma / 1e9, 2), "transfer_floor_s": round(t_xfer, 4),
        "overlap_efficiency": round((t_xfer + t_comp_last) / el, 4),
        "ffn_kernel_ms_per_layer": ms / max(prof["launches"], 1),
        "ffn_mfma": {"bound_note": "weight stream: HBM-bound at this shape", "TFLOPs": round(tflops, 1),
                     "frac_of_bf16_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "flop_per_byte": round(ai, 1), "attainable_TFLOPs": round(attainable, 1),
                     "frac_of_attainable": round(tflops / attainable, 4),
                     "GBs": round(by / (ms * 1e-3) / 1e9, 1) if ms > 0 else 0.0,
                     "gateup_ms_per_layer": prof["ms_gateup"] / max(prof["launches"], 1),
                     "down_ms_per_layer": prof["ms_down"] / max(prof["launches"], 1)},
        "overlap_off": None if el_off is None else {
            "tok_s": T / el_off, "s_per_chunk": el_off,
            "throughput_loss_pct": round(100.0 * (1.0 - el / el_off), 2),
            "note": "second buffer disabled: on-demand loading after each layer's routing"},
    }


def run_mxfp4(args, torch, ft, synth, HostPool):
    """MXFP4 experts at the 43-layer d=4096 shape: 2 x 8192-token prefill chunks, then
    batch-1 decode over a trace with a resize at a safe point."""
    wl, wd = synth.WORKLOADS["mxfp4-prefill8k-L43-d4096-E256-top6"], synth.WORKLOADS["mxfp4-decode-L43-d4096-E256-top6"]
    s = wl.shape
    S = s.record_bytes
    T = wl.T
    L_phys = s.L if args.mx_l_phys <= 0 else min(args.mx_l_phys, s.L)
    log(f"mxfp4 workload {wl.name}: pool {L_phys * s.E} records x {S / 1e6:.2f} MB = {L_phys * s.E * S / 1e9:.1f} GB")
    t = time.time()
    pool = HostPool(L_phys * s.E, S, s.pool_dtype)
    try:
        synth.fill_mxfp4_records_torch(pool.view, s.d, s.d_ff, wl.seed_key, seed=args.seed)
        log(f"pool allocated and filled in {time.time() - t:.1f} s")
        fshape = ft.make_shape(s.L, s.E, s.d, s.d_ff, s.k, ft.FT_W_MXFP4)
        scratch = torch.empty(64 * S, dtype=torch.uint8, device="cuda")
        B_P, B_H = ft.ft_bench_bw(fshape, pool.ptr, 64, scratch, 0)
        bwp = bw_profile(ft, fshape, pool, scratch, B_P, B_H)
        del scratch
        fq = ft.ft_frac_q16(B_P, B_H) if args.frac_q16 < 0 else args.frac_q16
        log(f"mxfp4 B_P {B_P / 1e9:.1f} GB/s, B_H {B_H / 1e9:.1f} GB/s, frac_q16 {fq}")
        N, N2 = wl.n_slots, wl.n_slots // 2
        cfg = ft.make_config(frac_q16=fq, min_fill=args.min_fill, max_fetch=-1, cpu_threads=args.cpu_threads,
                             prefill_overlap=1, T_max=T, L_phys=L_phys)
        slots = torch.empty(N * S, dtype=torch.uint8, device="cuda")
        wsb = ft.ft_workspace_bytes(fshape, T)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        wr = [torch.from_numpy(synth.router_weights(wl, l, seed=args.seed).view(np.int16)).cuda() for l in range(s.L)]
        n_chunks = 2
        xs = [[synth.tokens_torch(wl.seed_key, c, l, T, s.d, seed=args.seed) for l in range(s.L)]
              for c in range(n_chunks)]
        y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
        steps = args.mx_steps
        tr = synth.trace_for(wd, seed=args.seed, steps=steps)
        allowed = np.zeros((steps, s.L, 1, s.E), dtype=np.uint8)
        st_i, l_i = np.meshgrid(np.arange(steps), np.arange(s.L), indexing="ij")
        for j in range(s.k):
            allowed[st_i, l_i, 0, tr[:, :, 0, j].astype(np.int64)] = 1
        allowed_d = torch.from_numpy(allowed).cuda()
        xh = np.stack([np.stack([synth.tokens(wd, st, l, T=1, seed=args.seed) for l in range(s.L)])
                       for st in range(steps)])
        xd = torch.from_numpy(xh.view(np.int16)).cuda()
        yd = torch.empty((s.L, 1, s.d), dtype=torch.float32, device="cuda")
        ctx = ft.ft_create(fshape, cfg, pool.ptr, pool.nbytes, slots, N, ws, wsb)
        compute = torch.cuda.current_stream()
        copy = torch.cuda.Stream()
        try:
            ft.ft_moe_prefill_begin(ctx, copy)  # warm-up: two layers of one chunk
            for l in range(2):
                ft.ft_moe_prefill_layer(ctx, l, xs[0][l], T, wr[l], y, compute, copy)
            ft.ft_moe_prefill_end(ctx)
            torch.cuda.synchronize()
            ft.ft_profile_enable(ctx, True)
            t0 = time.perf_counter()
            for c in range(n_chunks):
                ft.ft_moe_prefill_begin(ctx, copy)
                for l in range(s.L):
                    ft.ft_moe_prefill_layer(ctx, l, xs[c][l], T, wr[l], y, compute, copy)
                ft.ft_moe_prefill_end(ctx)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            pprof = ft.ft_profile_read(ctx)
            ft.ft_profile_enable(ctx, False)
            del xs
            ft.ft_reset_stats(ctx)
            st_call = ft.ft_step_stats()
            seg = []
            for half in range(2):
                if half == 1:
                    torch.cuda.synchronize()
                    tr0 = time.perf_counter()
                    rc = ft.ft_expert_cache_resize(ctx, slots, N2)  # same buffer, half the slots
                    t_resize = time.perf_counter() - tr0
                    assert rc == ft.FT_OK, rc
                ft.ft_profile_enable(ctx, True)
                ta = time.perf_counter()
                for st in range(half * steps // 2, (half + 1) * steps // 2):
                    for l in range(s.L):
                        ft.ft_moe_decode_layer(ctx, l, xd[st, l], 1, wr[l], allowed_d[st, l], yd[l], compute,
                                               None, st_call)
                torch.cuda.synchronize()
                tb = time.perf_counter()
                seg.append((tb - ta, ft.ft_get_stats(ctx), ft.ft_profile_read(ctx)))
                ft.ft_profile_enable(ctx, False)
        finally:
            ft.ft_destroy(ctx)
    finally:
        pool.free()
    el_pf = t1 - t0
    ms_pf = pprof["ms_gateup"] + pprof["ms_down"]
    fl_pf = pprof["flops_gateup"] + pprof["flops_down"]
    tf_gu = pprof["flops_gateup"] / (pprof["ms_gateup"] * 1e-3) / 1e12 if pprof["ms_gateup"] > 0 else 0.0
    tf_dn = pprof["flops_down"] / (pprof["ms_down"] * 1e-3) / 1e12 if pprof["ms_down"] > 0 else 0.0
    tf = fl_pf / (ms_pf * 1e-3) / 1e12 if ms_pf > 0 else 0.0
    dec_el = seg[0][0] + seg[1][0]
    dprof = {k: seg[0][2][k] + seg[1][2][k] for k in seg[0][2]}
    gu_gbs = dprof["bytes_gateup"] / (dprof["ms_gateup"] * 1e-3) / 1e9 if dprof["ms_gateup"] > 0 else 0.0

    def seg_info(i, n_slots):
        el, st, _ = seg[i]
        reads = max(st["reads"], 1)
        return {"n_slots": n_slots, "steps": steps // 2, "tok_s": (steps // 2) / el, "ms_per_step": el / (steps // 2) * 1e3,
                "miss_rate_reads": 1.0 - st["read_hits"] / reads, "fills_per_step": st["fills"] / (steps // 2),
                "cpu_experts_per_step": st["cpu_experts"] / (steps // 2)}

    return {
        "workload": wl.name, "record_MB": S / 1e6, "L": s.L, "L_phys": L_phys, "B_P_GBs": B_P / 1e9,
        "B_H_GBs": B_H / 1e9, "frac_q16": fq, "bw_profile": bwp,
        "prefill": {"tokens": n_chunks * T, "chunks": n_chunks, "tok_s": n_chunks * T / el_pf,
                    "s_per_chunk": el_pf / n_chunks, "h2d_GB": n_chunks * s.L * s.E * S / 1e9,
                    "h2d_GBs_effective": n_chunks * s.L * s.E * S / el_pf / 1e9,
                    "ffn_ms_per_layer": ms_pf / max(pprof["launches"], 1),
                    "mx_mfma": {"TFLOPs": round(tf, 1), "gateup_TFLOPs": round(tf_gu, 1),
                                "down_TFLOPs": round(tf_dn, 1), "peak_TFLOPs": MFMA_FP8_PEAK_TFLOPS,
                                "frac": round(tf / MFMA_FP8_PEAK_TFLOPS, 4),
                                "note": "E4M3 x E2M1 scaled MFMA; times exclude the MXFP8 conversion kernels"}},
        "decode": {"steps": steps, "tok_s": steps / dec_el, "ms_per_step": dec_el / steps * 1e3,
                   "resize_at_step": steps // 2, "resize_ms": t_resize * 1e3,
                   "before_resize": seg_info(0, N), "after_resize": seg_info(1, N2),
                   "mx_gateup_rows": {"GBs": round(gu_gbs, 1), "frac_of_hbm_peak": round(gu_gbs / HBM_PEAK_GBS, 4),
                                      "avg_us": dprof["ms_gateup"] / max(dprof["launches"], 1) * 1e3},
                   "mx_down_rows": {"GBs": round(dprof["bytes_down"] / (dprof["ms_down"] * 1e-3) / 1e9, 1)
                                    if dprof["ms_down"] > 0 else 0.0,
                                    "avg_us": dprof["ms_down"] / max(dprof["launches"], 1) * 1e3}},
    }


def host_info():
    """CPU model, logical CPUs, physical cores (distinct (package, core) pairs) and the
    CPUs this process may run on."""
    model, cores, cur = None, set(), {}
    with open("/proc/cpuinfo") as f:
        for line in list(f) + [""]:
            if ":" not in line:
                if "physical id" in cur and "core id" in cur:
                    cores.add((cur["physical id"], cur["core id"]))
                cur = {}
                continue
            k, v = (t.strip() for t in line.split(":", 1))
            cur[k] = v
            if k == "model name" and model is None:
                model = v
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "physical_cores": len(cores) or None,
            "cpus_available": len(os.sched_getaffinity(0))}


def cpu_baseline(args, pool, wl, tr, fq, L_phys, budget_s, one_thread_budget_s):
    """The oracle as it stands, timed on the host cores over the first (step, layer)
    calls of the same trace and inputs: a bounded sample, scaled to tok/s through the
    time per layer call.  Once with BLAS on every CPU of the run, once on one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from moe_expert_offload_amd import synth
    from oracle.cache import SlotTable
    from oracle.ffn import moe_layer
    from oracle.router import route

    s = wl.shape
    T = wl.T
    wr = [synth.router_weights(wl, l, seed=args.seed) for l in range(s.L)]

    def timed(budget):
        cache = SlotTable(wl.n_slots, s.L, s.E)
        calls = 0
        t0 = time.perf_counter()
        while calls < tr.shape[0] * s.L:
            st, l = divmod(calls, s.L)
            x = synth.tokens(wl, st, l, T=T, seed=args.seed)
            allowed = synth.allowed_mask(tr[st, l], s.E)
            idx, g, _ = route(x, wr[l], s.k, allowed)
            cache.lookup(l, idx, fq, args.min_fill, -1)
            moe_layer(x, idx, g, lambda e: pool.view[(l % L_phys) * s.E + e], s.d, s.d_ff)
            calls += 1
            if time.perf_counter() - t0 > budget:
                break
        el = time.perf_counter() - t0
        step_s = el / calls * s.L
        return T / step_s, calls, el

    n_all = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=n_all):
        v_all, c_all, e_all = timed(budget_s)
        blas = [{k: p.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")}
                for p in threadpool_info()]
    with threadpool_limits(limits=1):
        v_one, c_one, e_one = timed(one_thread_budget_s)
    what = (f"{{n}} layer calls (first steps of the same trace and inputs, {s.L} layers per step) of the fp64 "
            f"NumPy oracle: router, cache decisions, exact layer output; {{el:.1f}} s, scaled to tok/s by "
            f"the time per layer call")
    return {"value": round(v_all, 5), "unit": "tok/s", "cores": n_all, "kind": "oracle",
            "sample": what.format(n=c_all, el=e_all),
            "one_thread": {"value": round(v_one, 5), "unit": "tok/s", "cores": 1,
                           "sample": what.format(n=c_one, el=e_one)},
            "host": host_info(), "blas": blas}


PAGES_FIG4B = {  # [FT] §5.3 "Expert locality": decode-read miss rates at the RTX 5090 serving capacity
    "37%": {"lru": 0.16, "hotset": 0.41, "static": 0.62, "model": "Qwen3.6-35B-A3B traces"},
    "11%": {"lru": 0.39, "hotset": 0.59, "static": 0.89, "model": "DeepSeek-V4-Flash traces"},
}


def run_placement(args, ft, synth):
    """Fig. 4b replay on synthetic traces (host only): decode-read miss rate of the
    engine's global LRU, a prefill-chosen hot set and a routing-blind static split,
    per cache capacity, for the 40-layer and 43-layer shapes; and the batch-dedup
    study (distinct experts per layer and step against batch size)."""
    out = {"requests": args.replay_requests, "prompt": args.replay_prompt, "decode": args.replay_decode,
           "trace": "Zipf(1.1) popularity per layer, 0.6 token-to-token reuse, one stream per request",
           "pages_fig4b": PAGES_FIG4B, "shapes": {}}
    pols = {"lru": ft.FT_PLACE_LRU, "hotset": ft.FT_PLACE_HOTSET, "static": ft.FT_PLACE_STATIC}
    t0 = time.perf_counter()
    for name in ("decode-L40-d2048-E128-top8", "decode-L43-d4096-E256-top6"):
        wl = synth.WORKLOADS[name]
        s = wl.shape
        steps = args.replay_prompt + args.replay_decode
        tr = synth.zipf_reuse_trace(s.L, s.E, s.k, args.replay_requests, steps, wl.zipf_alpha, wl.reuse,
                                    synth.generator(wl.seed_key, synth.STREAM_TRACE, 1, seed=args.seed))
        ids = np.ascontiguousarray(np.transpose(tr, (2, 0, 1, 3)).astype(np.int32))
        fshape = ft.make_shape(s.L, s.E, s.d, s.d_ff, s.k)
        rows = {}
        for cap in (0.05, 0.11, 0.20, 0.37, 0.60, 1.00):
            N = int(cap * s.L * s.E)
            row = {"n_slots": N}
            for pname, pol in pols.items():
                reads, misses = ft.ft_replay_placement(pol, fshape, N, ids, args.replay_prompt)
                row[pname] = round(misses / max(reads, 1), 4)
            rows[f"{round(cap * 100)}%"] = row
        # batch dedup: distinct experts per (step, layer) for B concurrent streams
        dedup = {}
        for B in (1, 4, 8):
            tb = synth.zipf_reuse_trace(s.L, s.E, s.k, B, 64, wl.zipf_alpha, wl.reuse,
                                        synth.generator(wl.seed_key, synth.STREAM_TRACE, 2, B, seed=args.seed))
            uniq = np.mean([len(np.unique(tb[st, l])) for st in range(tb.shape[0]) for l in range(s.L)])
            uni = s.E * (1.0 - (1.0 - s.k / s.E) ** B)
            dedup[f"B={B}"] = {"distinct_zipf": round(float(uniq), 3), "gain_zipf": round(B * s.k / uniq, 4),
                               "distinct_uniform_closed_form": round(uni, 3), "gain_uniform": round(B * s.k / uni, 4)}
        out["shapes"][name] = {"L": s.L, "E": s.E, "k": s.k, "miss_rate_by_capacity": rows, "batch_dedup": dedup}
    out["seconds"] = round(time.perf_counter() - t0, 2)
    return out


def counter_calibration(torch, mib=1024):
    """A plain device copy of a known size, three times: run under rocprofv3 --pmc
    FETCH_SIZE (or WRITE_SIZE), its reading per dispatch divided into the bytes each
    copy moves is the factor that turns that counter into bytes."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"counter_calibration": "device-to-device copy", "bytes_read_per_copy": mib << 20,
            "bytes_written_per_copy": mib << 20, "copies": 3}


def run_config2(args, torch, ft, synth, HostPool):
    """The 40-layer d=2048, E=128, top-8 stack (cache 37 %) on one pool: batch 1, batch 1
    without the fill floor, batch 8; each after the fixed cache warm-up."""
    out = {}
    log(f"decode {CONFIG2}, batch 1")
    d1, r1, keep = run_decode(args, torch, ft, synth, HostPool, CONFIG2, args.c2_steps, 0)
    pool = keep[0]
    try:
        out["batch1"] = {k: d1[k] for k in ("tok_s", "ms_per_step", "workload", "n_slots", "L_phys", "cache_warmup_steps",
                                            "timed_steps", "B_P_GBs", "B_H_GBs", "frac_q16", "min_fill",
                                            "miss_rate_reads", "fills_per_step", "cpu_experts_per_step",
                                            "h2d_GB_per_step", "modelled_floor_ms_per_step", "host_call_us",
                                            "cpu_branch_GBs",
                                            "kernels")}
        out["batch1"]["roofline"] = r1
        if args.min_fill0 and args.min_fill != 0:
            # q is the Q16 split alone, so single misses go to the host cores
            log("decode with min_fill = 0")
            d0, _, _ = run_decode(args, torch, ft, synth, HostPool, CONFIG2, args.mf0_steps, 0, {"min_fill": 0}, pool)
            out["min_fill0"] = {k: d0[k] for k in ("tok_s", "ms_per_step", "min_fill", "miss_rate_reads",
                                                   "fills_per_step", "cpu_experts_per_step", "h2d_GB_per_step",
                                                   "host_cpu_branch_ms_per_step", "modelled_floor_ms_per_step",
                                                   "cache_warmup_steps", "timed_steps")}
        if args.batch8:
            log("decode batch 8")
            d8, r8, _ = run_decode(args, torch, ft, synth, HostPool, CONFIG2 + "-b8", args.b8_steps, 0, None, pool)
            out["batch8"] = {"tok_s": d8["tok_s"], "ms_per_step": d8["ms_per_step"], "roofline": r8,
                             "miss_rate_reads": d8["miss_rate_reads"], "fills_per_step": d8["fills_per_step"],
                             "cpu_experts_per_step": d8["cpu_experts_per_step"], "kernels": d8["kernels"],
                             "cache_warmup_steps": d8["cache_warmup_steps"], "timed_steps": d8["timed_steps"]}
    finally:
        pool.free()
    return out


def arg_parser() -> argparse.ArgumentParser:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=CACHE_WARMUP_STEPS,
                    help=f"untimed steps before timing (at least {CACHE_WARMUP_STEPS} run in any case: cache warm-up)")
    ap.add_argument("--workload", default=HEADLINE, choices=[HEADLINE, CONFIG2, CONFIG2 + "-b8"])
    ap.add_argument("--l-phys", type=int, default=0,
                    help="physical layers in the host pool (0 = all, 4 for the 43-layer bf16 pool)")
    ap.add_argument("--min-fill", type=int, default=1)
    ap.add_argument("--max-fetch", type=int, default=-1)
    ap.add_argument("--frac-q16", type=int, default=-1, help="override the measured fetch fraction")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-graph", dest="graph", action="store_false", default=True,
                    help="skip the headline decode replayed from the graph-resident step")
    ap.add_argument("--no-config2", dest="config2", action="store_false", default=True,
                    help="skip the 40-layer d=2048 legs (batch 1, min_fill = 0, batch 8)")
    ap.add_argument("--c2-steps", type=int, default=64)
    ap.add_argument("--prefill", dest="prefill", action="store_true", default=True)
    ap.add_argument("--no-prefill", dest="prefill", action="store_false")
    ap.add_argument("--prefill-l-phys", type=int, default=2)
    ap.add_argument("--no-prefill-ablation", dest="prefill_ablation", action="store_false", default=True,
                    help="skip the overlap-off prefill pass")
    ap.add_argument("--mxfp4", dest="mxfp4", action="store_true", default=True)
    ap.add_argument("--no-mxfp4", dest="mxfp4", action="store_false")
    ap.add_argument("--mx-l-phys", type=int, default=16,
                    help="physical layers of the MXFP4 pool (0 = all; pinned memory is capped near half of host RAM)")
    ap.add_argument("--mx-steps", type=int, default=512)
    ap.add_argument("--no-batch8", dest="batch8", action="store_false", default=True,
                    help="skip the batch-8 decode leg of the 40-layer stack")
    ap.add_argument("--b8-steps", type=int, default=64)
    ap.add_argument("--no-min-fill0", dest="min_fill0", action="store_false", default=True,
                    help="skip the decode leg without the at-least-one-fill floor")
    ap.add_argument("--mf0-steps", type=int, default=64)
    ap.add_argument("--no-replay", dest="replay", action="store_false", default=True,
                    help="skip the Fig. 4b placement replay (host only)")
    ap.add_argument("--replay-requests", type=int, default=4)
    ap.add_argument("--replay-prompt", type=int, default=512)
    ap.add_argument("--replay-decode", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", dest="peaks", action="store_false", default=True,
                    help="skip the measured HBM, GEMM and host-copy ceilings")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--cpu-budget-1t-s", type=float, default=8.0)
    ap.add_argument("--counter-calibration", action="store_true",
                    help="only a plain device copy of known size, for rocprofv3 counter scaling")
    ap.add_argument("--skip-headline", action="store_true",
                    help="profiling runs of the other legs only: the headline decode is not run and no value is reported")
    return ap


def main():
    args = arg_parser().parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.counter_calibration:
        print(json.dumps(counter_calibration(torch)), flush=True)
        return

    from moe_expert_offload_amd import ft, synth
    from moe_expert_offload_amd.pool import HostPool

    ft.lib()
    dec, roof, cpu = None, None, None
    gdec = None
    if not args.skip_headline:
        dec, roof, keep = run_decode(args, torch, ft, synth, HostPool)
        pool, wl, tr, fq, L_phys = keep
        try:
            if args.graph:
                # the same workload, pool and trace, each step replayed from one HIP graph
                log("decode through the graph-resident step")
                g, _, _ = run_decode(args, torch, ft, synth, HostPool, args.workload, args.steps, args.warmup,
                                     {"mode": "graph"}, pool)
                gdec = {k: g[k] for k in ("mode", "tok_s", "ms_per_step", "miss_rate_reads", "fills_per_step",
                                          "cpu_experts_per_step", "h2d_GB_per_step", "cache_warmup_steps",
                                          "timed_steps", "B_P_GBs", "B_H_GBs", "frac_q16")}
                gdec["eager_tok_s"] = dec["tok_s"]
            if not args.no_cpu_baseline:
                log("timing the CPU oracle on the host")
                cpu = cpu_baseline(args, pool, wl, tr, fq, L_phys, args.cpu_budget_s, args.cpu_budget_1t_s)
        finally:
            pool.free()
    c2 = run_config2(args, torch, ft, synth, HostPool) if args.config2 and args.workload == HEADLINE else None
    pre = run_prefill(args, torch, ft, synth, HostPool) if args.prefill else None
    mxr = run_mxfp4(args, torch, ft, synth, HostPool) if args.mxfp4 else None
    rep = run_placement(args, ft, synth) if args.replay else None
    peaks = measured_peaks(torch) if args.peaks else None
    if dec is None:
        print(json.dumps({"profiling_run": True, "decode_L40": c2, "prefill": pre, "mxfp4": mxr,
                          "placement_replay": rep}), flush=True)
        return
    out = {
        "metric": METRIC, "value": round(dec["tok_s"], 3), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dec["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": dec["workload"], "global_batch": dec["T"], "layers": dec["L"],
                   "cache_slots": dec["n_slots"], "cache_warmup_steps": dec["cache_warmup_steps"],
                   "pool_physical_layers": dec["L_phys"], "parallelism": "single-gpu"},
        "roofline": roof, "cpu_baseline": cpu, "decode": dec, "decode_graph": gdec, "decode_L40": c2,
        "prefill": pre, "mxfp4": mxr,
        "placement_replay": rep, "measured_peaks": peaks,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
