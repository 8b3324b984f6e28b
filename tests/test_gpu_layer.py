"""GPU parity of the layer entry points (decode with the expert cache, prefill
with full-layer double buffering) against the oracle, through the C ABI.

Per call: routed ids bit-exact; every cache decision (hits, misses, q, victims,
slot rewrite, residency) bit-exact; y within max|gpu-ref| <= 2e-2 max|ref| and
sum|gpu-ref| / sum|ref| <= 3e-3.
"""
import numpy as np
import pytest

from moe_expert_offload_amd import ft
from moe_expert_offload_amd.synth import (Shape, Workload, allowed_mask, expert_record, router_weights,
                                          tokens, zipf_reuse_trace, generator)
from oracle.cache import SlotTable
from oracle.common import within_tolerance
from oracle.layer import decode_layer, prefill_layer
from oracle.qstar import Q16
from tests.gpu_helpers import Engine, PinnedPool, dev, dev_u16, host, torch_mod

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _stack(wl: Workload):
    s = wl.shape
    pool = PinnedPool(s, s.L * s.E)
    for l in range(s.L):
        for e in range(s.E):
            pool.view[l * s.E + e] = expert_record(wl, l, e)
    wr = [router_weights(wl, l) for l in range(s.L)]
    return pool, wr


def _compare_plan(plan, ref_plan, ref_idx):
    got = ft.plan_dict(plan)
    assert got["idx"] == ref_idx.reshape(-1).tolist()
    assert got["U"] == ref_plan.U and got["H"] == ref_plan.H and got["M"] == ref_plan.M
    assert got["q"] == ref_plan.q and got["avail"] == ref_plan.avail
    assert got["F_slot"] == ref_plan.F_slots and got["G_slot"] == ref_plan.G_slots
    assert got["route_slot"] == ref_plan.route_slot.reshape(-1).tolist()


SMALL = Workload("small-decode", 11, Shape(4, 32, 256, 512, 4), 2, 0.3)


@pytest.mark.parametrize("fq,min_fill,max_fetch,T,N", [
    (Q16, 1, -1, 2, 40),      # every miss filled
    (20000, 1, -1, 2, 40),    # split: fills and CPU experts
    (20000, 0, -1, 1, 40),    # the shipped rule (no floor)
    (0, 0, 0, 3, 40),         # never fetch: everything misses to the CPU
    (30000, 1, 2, 8, 40),     # fixed fetch cap, batch 8
    (Q16, 1, -1, 4, 128),     # capacity = all pairs: only compulsory misses
    (20000, 1, -1, 17, 40),   # 68 pairs: decisions by block-wide scans (more than 64 pairs)
    (20000, 1, -1, 64, 96),   # 64 tokens, the largest decode call (256 pairs)
])
def test_decode_trace_parity(fq, min_fill, max_fetch, T, N):
    _decode_trace(SMALL, fq, min_fill, max_fetch, T, N)


# d = 200 and d_ff = 328: rows whose length is not a multiple of the 512 elements a
# wavefront reads per load; calls of 1 to 9 tokens (row-streaming kernels with 1, 8
# and 2 x 8 tokens per pass)
RAGGED = Workload("ragged-decode", 13, Shape(3, 12, 200, 328, 3), 2, 0.5)


@pytest.mark.parametrize("T", [1, 5, 8, 9])
def test_decode_ragged_shape_parity(T):
    _decode_trace(RAGGED, 20000, 1, -1, T, 14)


# The decode router computes TT tokens x TE experts per wavefront (TT = 1, 4 or 8
# by T; TE = 1, 2 or 4 by E and T): every pair of them, several token groups, E not
# a multiple of the experts per block, and d with a partial last 512-element chunk.
@pytest.mark.parametrize("E,d,k,T", [
    (64, 200, 4, 1), (64, 200, 4, 4), (64, 200, 4, 13),
    (100, 1032, 6, 1), (100, 1032, 6, 3), (100, 1032, 6, 8),
    (256, 1032, 6, 1), (256, 1032, 6, 4), (256, 1032, 6, 8),
    (600, 520, 8, 1), (600, 520, 8, 3), (600, 520, 8, 13),
    (600, 520, 8, 64),  # the largest call: 64 tokens x 8 = 512 routed pairs
])
def test_decode_router_blocking_parity(E, d, k, T):
    wl = Workload(f"decode-E{E}-d{d}-top{k}", 20 + E % 7, Shape(2, E, d, 64, k), T, 0.5)
    _decode_trace(wl, 20000, 1, -1, T, max(2 * T * k, E // 2), steps=3)


def _decode_trace(wl, fq, min_fill, max_fetch, T, N, steps=6):
    torch = torch_mod()
    _say("decode", wl.name, fq, min_fill, max_fetch, T, N)
    s = wl.shape
    pool, wr = _stack(wl)
    eng = Engine(s, pool, N, T_max=max(T, 8), frac_q16=fq, min_fill=min_fill, max_fetch=max_fetch, cpu_threads=4)
    try:
        ref_cache = SlotTable(N, s.L, s.E)
        tr = zipf_reuse_trace(s.L, s.E, s.k, T, steps, 1.1, 0.6, generator(wl.seed_key, 3, T))
        wr_dev = [dev_u16(w) for w in wr]
        plan = ft.ft_plan()
        for step in range(tr.shape[0]):
            for l in range(s.L):
                x = tokens(wl, step, l, T=T)
                allowed = allowed_mask(tr[step, l], s.E)
                y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
                ft.ft_moe_decode_layer(eng.ctx, l, dev_u16(x), T, wr_dev[l], dev(allowed), y,
                                       plan=plan)
                torch.cuda.synchronize()
                ref = decode_layer(ref_cache, l, x, wr[l], s.k, lambda e: pool.view[l * s.E + e],
                                   s.d, s.d_ff, fq, min_fill, max_fetch, allowed)
                _compare_plan(plan, ref["plan"], ref["idx"])
                ok, mx, l1 = within_tolerance(host(y), ref["y"])
                assert ok, (step, l, mx, l1)
        st = ft.ft_get_stats(eng.ctx)
        assert st["unique_misses"] == ref_cache.counters.unique_misses
        assert st["fills"] == ref_cache.counters.fills
    finally:
        eng.destroy()
        pool.free()


C1 = Workload("layer-d256-E8-top2", 1, Shape(1, 8, 256, 512, 2), 16, 1.0)


def test_single_layer_configuration_all_resident():
    """d=256, E=8, top-2, d_ff=512, 16 tokens, every expert resident after the first call."""
    torch = torch_mod()
    s = C1.shape
    pool, wr = _stack(C1)
    eng = Engine(s, pool, s.E, T_max=16, frac_q16=Q16)
    try:
        x = tokens(C1, 0, 0)
        xd, wd = dev_u16(x), dev_u16(wr[0])
        ref_cache = SlotTable(s.E, 1, s.E)
        plan = ft.ft_plan()
        for call in range(3):
            y = torch.empty((16, s.d), dtype=torch.float32, device="cuda")
            ft.ft_moe_decode_layer(eng.ctx, 0, xd, 16, wd, None, y, plan=plan)
            torch.cuda.synchronize()
            ref = decode_layer(ref_cache, 0, x, wr[0], s.k, lambda e: pool.view[e], s.d, s.d_ff, Q16)
            _compare_plan(plan, ref["plan"], ref["idx"])
            ok, mx, l1 = within_tolerance(host(y), ref["y"])
            assert ok, (call, mx, l1)
            if call > 0:
                assert plan.n_m == 0  # all hits once resident
    finally:
        eng.destroy()
        pool.free()


PF = Workload("small-prefill", 12, Shape(3, 16, 256, 512, 2), 200, 0.9)


@pytest.mark.parametrize("T", [200, 1])
def test_prefill_double_buffer_then_decode(T):
    torch = torch_mod()
    _say("prefill", T)
    s = PF.shape
    pool, wr = _stack(PF)
    N = 40
    eng = Engine(s, pool, N, T_max=max(T, 8), frac_q16=40000, prefill_overlap=1, cpu_threads=4)
    try:
        ref_cache = SlotTable(N, s.L, s.E)
        wr_dev = [dev_u16(w) for w in wr]
        plan = ft.ft_plan()
        tr = zipf_reuse_trace(s.L, s.E, s.k, 2, 6, 1.1, 0.6, generator(12, 3))

        def decode_steps(steps):
            for step in steps:
                for l in range(s.L):
                    x = tokens(PF, 100 + step, l, T=2)
                    allowed = allowed_mask(tr[step, l], s.E)
                    y = torch.empty((2, s.d), dtype=torch.float32, device="cuda")
                    ft.ft_moe_decode_layer(eng.ctx, l, dev_u16(x), 2, wr_dev[l], dev(allowed), y,
                                           plan=plan)
                    torch.cuda.synchronize()
                    ref = decode_layer(ref_cache, l, x, wr[l], s.k, lambda e: pool.view[l * s.E + e],
                                       s.d, s.d_ff, 40000, 1, -1, allowed)
                    _compare_plan(plan, ref["plan"], ref["idx"])
                    assert within_tolerance(host(y), ref["y"])[0]

        decode_steps(range(3))
        ft.ft_moe_prefill_begin(eng.ctx, eng.copy)
        bufs = ref_cache.prefill_begin()
        ys = []
        for l in range(s.L):
            for e in range(s.E):
                assert ft.ft_prefill_slot(eng.ctx, l, e) == bufs[l % 2][e]
            x = tokens(PF, 0, l, T=T)
            y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
            ft.ft_moe_prefill_layer(eng.ctx, l, dev_u16(x), T, wr_dev[l], y, copy=eng.copy)
            ys.append((x, y))
        ft.ft_moe_prefill_end(eng.ctx)
        ref_cache.prefill_end(s.L)
        torch.cuda.synchronize()
        for l, (x, y) in enumerate(ys):
            ref = prefill_layer(x, wr[l], s.k, lambda e: pool.view[l * s.E + e], s.d, s.d_ff)
            ok, mx, l1 = within_tolerance(host(y), ref["y"])
            assert ok, (l, mx, l1)
        for l in range(s.L):
            for e in range(s.E):
                assert ft.ft_expert_cache_where(eng.ctx, l, e) == ref_cache.where.get(l * s.E + e, -1)
        decode_steps(range(3, 6))  # survivors of the prefill seed decode
    finally:
        eng.destroy()
        pool.free()


@pytest.mark.parametrize("N", [5, 20, 40])
def test_prefill_on_demand_then_decode(N):
    """On-demand prefill (overlap off; below 2E slots it is the only prefill): every
    layer's output within tolerance, the residency after it equal to the oracle's
    rounds (5 slots: several rounds per layer; 20: one full layer at a time; 40:
    the serial form of the double buffer), then decode from that state."""
    torch = torch_mod()
    T = 200
    _say("prefill on demand", N)
    s = PF.shape
    pool, wr = _stack(PF)
    eng = Engine(s, pool, N, T_max=T, frac_q16=40000, prefill_overlap=0, cpu_threads=4)
    try:
        ref_cache = SlotTable(N, s.L, s.E)
        wr_dev = [dev_u16(w) for w in wr]
        plan = ft.ft_plan()
        tr = zipf_reuse_trace(s.L, s.E, s.k, 2, 4, 1.1, 0.6, generator(13, N))

        def decode_steps(steps):
            for step in steps:
                for l in range(s.L):
                    x = tokens(PF, 300 + step, l, T=2)
                    allowed = allowed_mask(tr[step, l], s.E)
                    y = torch.empty((2, s.d), dtype=torch.float32, device="cuda")
                    ft.ft_moe_decode_layer(eng.ctx, l, dev_u16(x), 2, wr_dev[l], dev(allowed), y, plan=plan)
                    torch.cuda.synchronize()
                    ref = decode_layer(ref_cache, l, x, wr[l], s.k, lambda e: pool.view[l * s.E + e],
                                       s.d, s.d_ff, 40000, 1, -1, allowed)
                    _compare_plan(plan, ref["plan"], ref["idx"])
                    assert within_tolerance(host(y), ref["y"])[0]

        decode_steps(range(2))
        ft.ft_moe_prefill_begin(eng.ctx, eng.copy)
        assert ft.ft_prefill_slot(eng.ctx, 0, 0) == -1
        for l in range(s.L):
            x = tokens(PF, 0, l, T=T)
            y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
            ft.ft_moe_prefill_layer(eng.ctx, l, dev_u16(x), T, wr_dev[l], y, copy=eng.copy)
            torch.cuda.synchronize()
            ref = prefill_layer(x, wr[l], s.k, lambda e: pool.view[l * s.E + e], s.d, s.d_ff)
            ref_cache.prefill_on_demand(l, ref["idx"])
            ok, mx, l1 = within_tolerance(host(y), ref["y"])
            assert ok, (l, mx, l1)
        ft.ft_moe_prefill_end(eng.ctx)
        for l in range(s.L):
            for e in range(s.E):
                assert ft.ft_expert_cache_where(eng.ctx, l, e) == ref_cache.where.get(l * s.E + e, -1)
        decode_steps(range(2, 4))
    finally:
        eng.destroy()
        pool.free()


def test_resize_at_safe_point_keeps_outputs():
    torch = torch_mod()
    s = SMALL.shape
    pool, wr = _stack(SMALL)
    eng = Engine(s, pool, 60, T_max=2, frac_q16=30000, cpu_threads=4)
    try:
        ref_cache = SlotTable(60, s.L, s.E)
        wr_dev = [dev_u16(w) for w in wr]
        tr = zipf_reuse_trace(s.L, s.E, s.k, 1, 8, 1.1, 0.6, generator(11, 4))
        plan = ft.ft_plan()
        small_slots = torch.empty(25 * s.record_bytes, dtype=torch.uint8, device="cuda")
        for step in range(8):
            if step == 4:
                torch.cuda.synchronize()
                assert ft.ft_expert_cache_resize(eng.ctx, small_slots, 25) == ft.FT_OK
                ref_cache.resize(25)
            for l in range(s.L):
                x = tokens(SMALL, 50 + step, l, T=1)
                allowed = allowed_mask(tr[step, l], s.E)
                y = torch.empty((1, s.d), dtype=torch.float32, device="cuda")
                ft.ft_moe_decode_layer(eng.ctx, l, dev_u16(x), 1, wr_dev[l], dev(allowed), y,
                                       plan=plan)
                torch.cuda.synchronize()
                ref = decode_layer(ref_cache, l, x, wr[l], s.k, lambda e: pool.view[l * s.E + e],
                                   s.d, s.d_ff, 30000, 1, -1, allowed)
                _compare_plan(plan, ref["plan"], ref["idx"])
                assert within_tolerance(host(y), ref["y"])[0]
        assert ft.ft_get_stats(eng.ctx)["resizes"] == 1
    finally:
        eng.destroy()
        pool.free()
