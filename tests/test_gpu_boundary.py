"""GPU tests of boundary paths through the C ABI: a prefill ended early (the
residency is what the two buffers hold, checked by decoding from it with a pool
whose layers all differ), the DMA fill entry point and its events, a resize
refused while issued work still runs, a decode call whose token allows fewer
than k experts, and the routing read-back.

Expected values come from the oracle; tolerance for y: max|gpu-ref| <=
2e-2 max|ref| and sum|gpu-ref| / sum|ref| <= 3e-3."""
import numpy as np
import pytest

from moe_expert_offload_amd import ft
from moe_expert_offload_amd.synth import (Shape, Workload, allowed_mask, expert_record, generator,
                                          router_weights, tokens, zipf_reuse_trace)
from oracle.cache import SlotTable
from oracle.common import within_tolerance
from oracle.layer import decode_layer, prefill_layer
from oracle.qstar import Q16
from tests.gpu_helpers import Engine, PinnedPool, dev, dev_u16, host, torch_mod

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _stack(wl: Workload):
    """A pool holding every layer's own records (no aliasing)."""
    s = wl.shape
    pool = PinnedPool(s, s.L * s.E)
    for l in range(s.L):
        for e in range(s.E):
            pool.view[l * s.E + e] = expert_record(wl, l, e)
    return pool, [router_weights(wl, l) for l in range(s.L)]


def _compare_plan(plan, ref_plan, ref_idx, where):
    got = ft.plan_dict(plan)
    assert got["idx"] == ref_idx.reshape(-1).tolist(), where
    assert (got["U"], got["H"], got["M"], got["q"]) == (ref_plan.U, ref_plan.H, ref_plan.M, ref_plan.q), where
    assert got["F_slot"] == ref_plan.F_slots and got["G_slot"] == ref_plan.G_slots, where
    assert got["route_slot"] == ref_plan.route_slot.reshape(-1).tolist(), where


def _busy(torch, ms_target=250):
    """Queue well-behaved GPU work on the current stream (plain matrix products) that
    takes a while to finish."""
    a = torch.randn(4096, 4096, device="cuda")
    b = torch.empty_like(a)
    for _ in range(ms_target):
        torch.mm(a, a, out=b)
    return a, b


PE = Workload("prefill-early-end", 21, Shape(6, 16, 256, 512, 2), 64, 0.5)


def test_prefill_ended_early_then_decode_unaliased():
    """Prefill of layers 0..2 of 6, then end: the buffers hold layer 2 (computed)
    and layer 3 (streamed in while 2 computed), so those stay resident and layer 1
    does not.  Decoding layers 1, 2 and 3 then matches the oracle, decisions and y,
    on a pool where every layer's records differ (a slot registered under the wrong
    layer would give another layer's weights)."""
    torch = torch_mod()
    s = PE.shape
    pool, wr = _stack(PE)
    N, fq, T = 40, 30000, PE.T
    eng = Engine(s, pool, N, T_max=T, frac_q16=fq, prefill_overlap=1, cpu_threads=4)
    try:
        ref = SlotTable(N, s.L, s.E)
        wr_dev = [dev_u16(w) for w in wr]
        ft.ft_moe_prefill_begin(eng.ctx, eng.copy)
        ref.prefill_begin()
        for l in range(3):
            x = tokens(PE, 0, l, T=T)
            y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
            ft.ft_moe_prefill_layer(eng.ctx, l, dev_u16(x), T, wr_dev[l], y, copy=eng.copy)
            torch.cuda.synchronize()
            r = prefill_layer(x, wr[l], s.k, lambda e: pool.view[l * s.E + e], s.d, s.d_ff)
            assert within_tolerance(host(y), r["y"])[0], l
        ft.ft_moe_prefill_end(eng.ctx)
        ref.prefill_end(3)
        res = ref.resident()
        assert {k // s.E for k in res} == {2, 3}
        for l in range(s.L):
            for e in range(s.E):
                assert ft.ft_expert_cache_where(eng.ctx, l, e) == res.get(l * s.E + e, -1), (l, e)
        tr = zipf_reuse_trace(s.L, s.E, s.k, 1, 3, 1.1, 0.6, generator(21, 3))
        plan = ft.ft_plan()
        hits = 0
        for step in range(3):
            for l in (1, 2, 3):
                x = tokens(PE, 10 + step, l, T=1)
                allowed = allowed_mask(tr[step, l], s.E)
                y = torch.empty((1, s.d), dtype=torch.float32, device="cuda")
                ft.ft_moe_decode_layer(eng.ctx, l, dev_u16(x), 1, wr_dev[l], dev(allowed), y, plan=plan)
                torch.cuda.synchronize()
                r = decode_layer(ref, l, x, wr[l], s.k, lambda e: pool.view[l * s.E + e], s.d, s.d_ff, fq,
                                 1, -1, allowed)
                _compare_plan(plan, r["plan"], r["idx"], (step, l))
                ok, mx, l1 = within_tolerance(host(y), r["y"])
                assert ok, (step, l, mx, l1)
                hits += plan.n_h if step == 0 and l in (2, 3) else 0
        assert hits == 2 * s.k  # step 0: layers 2 and 3 hit on every routed expert
    finally:
        eng.destroy()
        pool.free()


FILL = Workload("fill-entry", 22, Shape(2, 8, 256, 512, 2), 2, 1.0)


def test_expert_cache_fill_lands_records_after_wait_event():
    """ft_expert_cache_fill copies the plan's F records into their slots on the copy
    stream, only after wait_event (a later overwrite of every slot, queued behind a
    long computation on another stream, lands first) and signals done_event."""
    torch = torch_mod()
    s = FILL.shape
    S = s.record_bytes
    pool, _ = _stack(FILL)
    N = 8
    eng = Engine(s, pool, N, T_max=2, frac_q16=Q16, cpu_threads=2)
    try:
        ref = SlotTable(N, s.L, s.E)
        idx = np.array([[3, 5], [5, 6]], dtype=np.int32)
        plan = ft.ft_expert_cache_lookup(eng.ctx, 1, idx, 2)
        rp = ref.lookup(1, idx, Q16, 1, -1)
        assert plan.q == 3 and list(plan.F_slot[:3]) == rp.F_slots and list(plan.M[:3]) == rp.M
        side = torch.cuda.Stream()
        wait_ev, done_ev = torch.cuda.Event(), torch.cuda.Event()
        done_ev.record()  # creates the event; the library records it again on the copy stream
        before = ft.ft_get_stats(eng.ctx)["h2d_bytes"]
        with torch.cuda.stream(side):
            keep = _busy(torch)
            eng.slots.fill_(0x5A)  # lands after the long computation
            wait_ev.record(side)
        ft.ft_expert_cache_fill(eng.ctx, plan, eng.copy, wait_ev.cuda_event, done_ev.cuda_event)
        done_ev.synchronize()
        got = host(eng.slots).reshape(N, S)
        pv = pool.view.view(np.uint8).reshape(-1, S)
        for i in range(plan.q):
            assert np.array_equal(got[plan.F_slot[i]], pv[1 * s.E + plan.M[i]]), i
        others = sorted(set(range(N)) - set(plan.F_slot[:plan.q]))
        assert np.all(got[others] == 0x5A)
        assert ft.ft_get_stats(eng.ctx)["h2d_bytes"] - before == plan.q * S
        del keep
    finally:
        eng.destroy()
        pool.free()


PB = Workload("busy-resize", 23, Shape(3, 16, 256, 512, 2), 64, 0.9)


def test_resize_refused_while_issued_work_runs():
    """A resize while work the library issued is still queued behind a long
    computation returns FT_EBUSY and changes nothing; once the device is idle it
    succeeds."""
    torch = torch_mod()
    s = PB.shape
    pool, wr = _stack(PB)
    N, T = 40, PB.T
    eng = Engine(s, pool, N, T_max=T, frac_q16=Q16, prefill_overlap=1, cpu_threads=2)
    try:
        wr_dev = [dev_u16(w) for w in wr]
        xs = [dev_u16(tokens(PB, 0, l, T=T)) for l in range(s.L)]
        y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
        ft.ft_moe_prefill_begin(eng.ctx, eng.copy)
        for l in range(s.L):
            if l == s.L - 1:
                keep = _busy(torch)  # the last layer's compute queues behind this
            ft.ft_moe_prefill_layer(eng.ctx, l, xs[l], T, wr_dev[l], y, copy=eng.copy)
        ft.ft_moe_prefill_end(eng.ctx)
        where = [ft.ft_expert_cache_where(eng.ctx, l, e) for l in range(s.L) for e in range(s.E)]
        with pytest.raises(ft.FtError) as ei:
            ft.ft_expert_cache_resize(eng.ctx, eng.slots, 20)
        assert ei.value.status == ft.FT_EBUSY
        assert ft.ft_n_slots(eng.ctx) == N
        assert [ft.ft_expert_cache_where(eng.ctx, l, e) for l in range(s.L) for e in range(s.E)] == where
        torch.cuda.synchronize()
        assert ft.ft_expert_cache_resize(eng.ctx, eng.slots, 20) == ft.FT_WOVERLAP_OFF
        assert ft.ft_n_slots(eng.ctx) == 20
        del keep
    finally:
        eng.destroy()
        pool.free()


DEC = Workload("decode-errors", 24, Shape(2, 16, 256, 512, 3), 2, 0.5)


def test_decode_token_allowing_fewer_than_k_changes_nothing():
    """A token whose mask allows fewer than k experts: FT_EINVAL, the device takes no
    decisions (no fills, no groups) and residency is unchanged; the next call runs
    normally against the oracle, and the routing read-back equals the plan's ids."""
    torch = torch_mod()
    s = DEC.shape
    pool, wr = _stack(DEC)
    N, fq = 8, 30000
    eng = Engine(s, pool, N, T_max=2, frac_q16=fq, cpu_threads=2)
    try:
        ref = SlotTable(N, s.L, s.E)
        wr_dev = [dev_u16(w) for w in wr]
        plan = ft.ft_plan()
        x = tokens(DEC, 0, 0, T=2)
        good = allowed_mask(np.array([[1, 4, 9], [4, 9, 12]]), s.E)
        y = torch.empty((2, s.d), dtype=torch.float32, device="cuda")
        ft.ft_moe_decode_layer(eng.ctx, 0, dev_u16(x), 2, wr_dev[0], dev(good), y, plan=plan)
        torch.cuda.synchronize()
        r = decode_layer(ref, 0, x, wr[0], s.k, lambda e: pool.view[e], s.d, s.d_ff, fq, 1, -1, good)
        _compare_plan(plan, r["plan"], r["idx"], "first")
        ids = torch.empty((2, s.k), dtype=torch.int32, device="cuda")
        g = torch.empty((2, s.k), dtype=torch.float32, device="cuda")
        ft.ft_layer_routing(eng.ctx, ids, g, 2)
        torch.cuda.synchronize()
        assert host(ids).reshape(-1).tolist() == ft.plan_dict(plan)["idx"]
        assert np.array_equal(host(g).reshape(-1), np.array(ft.plan_dict(plan)["gates"], np.float32))
        where = [ft.ft_expert_cache_where(eng.ctx, l, e) for l in range(s.L) for e in range(s.E)]
        short = good.copy()
        short[1] = 0
        short[1, [3, 7]] = 1  # two allowed for k = 3
        with pytest.raises(ft.FtError) as ei:
            ft.ft_moe_decode_layer(eng.ctx, 0, dev_u16(x), 2, wr_dev[0], dev(short), y, plan=plan)
        assert ei.value.status == ft.FT_EINVAL
        torch.cuda.synchronize()
        assert [ft.ft_expert_cache_where(eng.ctx, l, e) for l in range(s.L) for e in range(s.E)] == where
        for step in range(2):
            for l in range(s.L):
                x = tokens(DEC, 5 + step, l, T=2)
                allowed = allowed_mask(np.array([[2, 4, 6 + step], [4, 9, 12]]), s.E)
                ft.ft_moe_decode_layer(eng.ctx, l, dev_u16(x), 2, wr_dev[l], dev(allowed), y, plan=plan)
                torch.cuda.synchronize()
                r = decode_layer(ref, l, x, wr[l], s.k, lambda e: pool.view[l * s.E + e], s.d, s.d_ff, fq, 1, -1,
                                 allowed)
                _compare_plan(plan, r["plan"], r["idx"], (step, l))
                assert within_tolerance(host(y), r["y"])[0], (step, l)
    finally:
        eng.destroy()
        pool.free()
