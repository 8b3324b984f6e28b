"""GPU parity of the graph-resident decode step (ft_decode_graph_*) against the
oracle, through the C ABI: every layer's y within max|gpu-ref| <= 2e-2 max|ref| and
sum|gpu-ref| / sum|ref| <= 3e-3, residency and counters equal to the oracle's after
every step, with eager decode calls (ft_moe_decode_layer) and synchronisations
between graph replays; bf16 and MXFP4 records; a resize between replays (the graph
is captured again); the error path (a token allowing fewer than k experts)."""
import numpy as np
import pytest

from moe_expert_offload_amd import ft
from moe_expert_offload_amd.synth import (Shape, Workload, allowed_mask, expert_record, generator,
                                          mxfp4_expert_record, router_weights, tokens, zipf_reuse_trace)
from oracle.cache import SlotTable
from oracle.common import within_tolerance
from oracle.layer import decode_layer
from tests.gpu_helpers import Engine, PinnedPool, dev, dev_u16, host, torch_mod

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _stack(wl):
    s = wl.shape
    pool = PinnedPool(s, s.L * s.E)
    rec = mxfp4_expert_record if s.mxfp4 else expert_record
    for l in range(s.L):
        for e in range(s.E):
            pool.view[l * s.E + e] = rec(wl, l, e)
    return pool, [router_weights(wl, l) for l in range(s.L)]


def _residency(ctx, s):
    return [ft.ft_expert_cache_where(ctx, l, e) for l in range(s.L) for e in range(s.E)]


def _ref_residency(ref, s):
    res = ref.resident()
    return [res.get(l * s.E + e, -1) for l in range(s.L) for e in range(s.E)]


BF = Workload("graph-bf16", 31, Shape(4, 32, 256, 512, 4), 2, 0.3)
MX = Workload("graph-mxfp4", 32, Shape(3, 16, 256, 384, 4, True), 2, 0.5)


@pytest.mark.parametrize("wl,N,fq", [(BF, 40, 20000), (MX, 20, 30000)])
def test_graph_step_matches_oracle_with_eager_calls_between(wl, N, fq):
    torch = torch_mod()
    s = wl.shape
    T = wl.T
    fmt = "mxfp4" if s.mxfp4 else "bf16"
    _say("decode graph", wl.name, N, fq)
    pool, wr = _stack(wl)
    eng = Engine(s, pool, N, T_max=T, frac_q16=fq, cpu_threads=4)
    graph = None
    try:
        ref = SlotTable(N, s.L, s.E)
        wr_dev = [dev_u16(w) for w in wr]
        xb = torch.zeros((s.L, T, s.d), dtype=torch.int16, device="cuda")
        ab = torch.zeros((s.L, T, s.E), dtype=torch.uint8, device="cuda")
        yb = torch.zeros((s.L, T, s.d), dtype=torch.float32, device="cuda")
        graph = ft.ft_decode_graph_create(eng.ctx, T, xb, wr_dev, ab, yb)
        tr = zipf_reuse_trace(s.L, s.E, s.k, T, 8, 1.1, 0.6, generator(wl.seed_key, 3))
        small = torch.empty(max(N // 2, 1) * s.record_bytes, dtype=torch.uint8, device="cuda")
        n_small = max(N // 2, 1)
        for step in range(8):
            xs = [tokens(wl, step, l, T=T) for l in range(s.L)]
            masks = [allowed_mask(tr[step, l], s.E) for l in range(s.L)]
            if step == 5:  # resize at a safe point: the next launch captures again
                torch.cuda.synchronize()
                ft.ft_expert_cache_resize(eng.ctx, small, n_small)
                ref.resize(n_small)
            if step == 3:  # eager calls between replays
                for l in range(s.L):
                    y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
                    ft.ft_moe_decode_layer(eng.ctx, l, dev_u16(xs[l]), T, wr_dev[l], dev(masks[l]), y)
                    torch.cuda.synchronize()
                    r = decode_layer(ref, l, xs[l], wr[l], s.k, lambda e: pool.view[l * s.E + e], s.d, s.d_ff, fq,
                                     1, -1, masks[l], fmt=fmt)
                    assert within_tolerance(host(y), r["y"])[0], ("eager", l)
            else:
                for l in range(s.L):
                    xb[l].copy_(dev_u16(xs[l]))
                    ab[l].copy_(dev(masks[l]))
                ft.ft_decode_graph_launch(graph)
                torch.cuda.synchronize()
                ft.ft_decode_graph_status(graph)
                got = host(yb)
                for l in range(s.L):
                    r = decode_layer(ref, l, xs[l], wr[l], s.k, lambda e: pool.view[l * s.E + e], s.d, s.d_ff, fq,
                                     1, -1, masks[l], fmt=fmt)
                    ok, mx, l1 = within_tolerance(got[l], r["y"])
                    assert ok, (step, l, mx, l1)
            assert _residency(eng.ctx, s) == _ref_residency(ref, s), step
            st = ft.ft_get_stats(eng.ctx)
            c = ref.counters
            assert (st["fills"], st["cpu_experts"], st["unique_hits"], st["read_hits"]) == \
                (c.fills, c.cpu_experts, c.unique_hits, c.read_hits), step
    finally:
        if graph:
            ft.ft_decode_graph_destroy(graph)
        eng.destroy()
        pool.free()


def test_graph_step_error_empties_cache_and_reports():
    """A token of layer 1 allows fewer than k experts: the next launch returns FT_EINVAL,
    the cache is empty, and steps after it match an oracle that starts empty."""
    torch = torch_mod()
    wl = BF
    s = wl.shape
    T, N, fq = wl.T, 40, 20000
    pool, wr = _stack(wl)
    eng = Engine(s, pool, N, T_max=T, frac_q16=fq, cpu_threads=4)
    graph = None
    try:
        wr_dev = [dev_u16(w) for w in wr]
        xb = torch.zeros((s.L, T, s.d), dtype=torch.int16, device="cuda")
        ab = torch.zeros((s.L, T, s.E), dtype=torch.uint8, device="cuda")
        yb = torch.zeros((s.L, T, s.d), dtype=torch.float32, device="cuda")
        graph = ft.ft_decode_graph_create(eng.ctx, T, xb, wr_dev, ab, yb)
        tr = zipf_reuse_trace(s.L, s.E, s.k, T, 4, 1.1, 0.6, generator(wl.seed_key, 4))

        def load(step, bad=False):
            for l in range(s.L):
                xb[l].copy_(dev_u16(tokens(wl, 20 + step, l, T=T)))
                m = allowed_mask(tr[step, l], s.E)
                if bad and l == 1:
                    m[1] = 0
                    m[1, :2] = 1  # two allowed for k = 4
                ab[l].copy_(dev(m))

        load(0)
        ft.ft_decode_graph_launch(graph)
        load(1, bad=True)
        ft.ft_decode_graph_launch(graph)
        torch.cuda.synchronize()
        with pytest.raises(ft.FtError) as ei:
            ft.ft_decode_graph_launch(graph)
        assert ei.value.status == ft.FT_EINVAL
        torch.cuda.synchronize()
        assert all(w == -1 for w in _residency(eng.ctx, s))
        ref = SlotTable(N, s.L, s.E)
        for step in (2, 3):
            load(step)
            ft.ft_decode_graph_launch(graph)
            torch.cuda.synchronize()
            got = host(yb)
            for l in range(s.L):
                x = tokens(wl, 20 + step, l, T=T)
                r = decode_layer(ref, l, x, wr[l], s.k, lambda e: pool.view[l * s.E + e], s.d, s.d_ff, fq, 1, -1,
                                 allowed_mask(tr[step, l], s.E))
                assert within_tolerance(got[l], r["y"])[0], (step, l)
            assert _residency(eng.ctx, s) == _ref_residency(ref, s), step
        ft.ft_decode_graph_status(graph)
    finally:
        if graph:
            ft.ft_decode_graph_destroy(graph)
        eng.destroy()
        pool.free()


def test_graph_step_full_size_headline_shape():
    """The graph-resident step at the 43-layer d=4096 E=256 top-6 batch-1 shape, 1210 slots,
    pool of 2 physical layers: decisions (residency and counters after every step) equal
    the oracle's on every step, y of every layer within tolerance on the last step."""
    torch = torch_mod()
    from moe_expert_offload_amd import synth
    from oracle.ffn import moe_layer
    from oracle.router import route
    wl = synth.WORKLOADS["decode-L43-d4096-E256-top6"]
    s = wl.shape
    T, L_phys, fq, steps = 1, 2, 18000, 3
    _say("decode graph full size", wl.name)
    pool = PinnedPool(s, L_phys * s.E)
    pool.fill_device_random(wl.seed_key)
    eng = Engine(s, pool, wl.n_slots, T_max=T, frac_q16=fq, L_phys=L_phys)
    graph = None
    try:
        ref = SlotTable(wl.n_slots, s.L, s.E)
        tr = synth.trace_for(wl, steps=steps)
        wr = [synth.router_weights(wl, l) for l in range(s.L)]
        wr_dev = [dev_u16(w) for w in wr]
        xb = torch.zeros((s.L, T, s.d), dtype=torch.int16, device="cuda")
        ab = torch.zeros((s.L, T, s.E), dtype=torch.uint8, device="cuda")
        yb = torch.zeros((s.L, T, s.d), dtype=torch.float32, device="cuda")
        graph = ft.ft_decode_graph_create(eng.ctx, T, xb, wr_dev, ab, yb)
        for st in range(steps):
            xs = [synth.tokens(wl, st, l, T=T) for l in range(s.L)]
            masks = [synth.allowed_mask(tr[st, l], s.E) for l in range(s.L)]
            for l in range(s.L):
                xb[l].copy_(dev_u16(xs[l]))
                ab[l].copy_(dev(masks[l]))
            ft.ft_decode_graph_launch(graph)
            torch.cuda.synchronize()
            ft.ft_decode_graph_status(graph)
            got = host(yb)
            for l in range(s.L):
                idx, g, _ = route(xs[l], wr[l], s.k, masks[l])
                ref.lookup(l, idx, fq, 1, -1)
                if st == steps - 1:
                    ref_y = moe_layer(xs[l], idx, g, lambda e: pool.view[(l % L_phys) * s.E + e], s.d, s.d_ff)
                    ok, mx, l1 = within_tolerance(got[l], ref_y)
                    assert ok, (st, l, mx, l1)
            res = ref.resident()
            for l in range(s.L):
                for e in range(0, s.E, 5):
                    assert ft.ft_expert_cache_where(eng.ctx, l, e) == res.get(l * s.E + e, -1), (st, l, e)
            stt = ft.ft_get_stats(eng.ctx)
            c = ref.counters
            assert (stt["fills"], stt["cpu_experts"], stt["read_hits"]) == (c.fills, c.cpu_experts, c.read_hits), st
    finally:
        if graph:
            ft.ft_decode_graph_destroy(graph)
        eng.destroy()
        pool.free()
