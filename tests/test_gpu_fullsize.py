"""GPU parity at full workload sizes, in the configuration bench.py times.

Decisions (routed ids, hits/misses, q, victims, slot rewrite) are compared bit for
bit on every call; layer outputs on sampled calls (decode) or sampled tokens
(prefill), which the oracle can afford at these sizes.  Tolerance:
max|gpu-ref| <= 2e-2 max|ref| and sum|gpu-ref| / sum|ref| <= 3e-3.
"""
import numpy as np
import pytest

from moe_expert_offload_amd import ft, synth
from oracle.cache import SlotTable
from oracle.common import within_tolerance
from oracle.ffn import moe_layer
from oracle.router import route
from tests.gpu_helpers import Engine, PinnedPool, dev, dev_u16, host, tile_cover_tokens, torch_mod

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _compare_plan(plan, ref_plan, ref_idx, where):
    got = ft.plan_dict(plan)
    assert got["idx"] == ref_idx.reshape(-1).tolist(), where
    assert (got["U"], got["H"], got["M"], got["q"]) == (ref_plan.U, ref_plan.H, ref_plan.M, ref_plan.q), where
    assert got["F_slot"] == ref_plan.F_slots and got["G_slot"] == ref_plan.G_slots, where
    assert got["route_slot"] == ref_plan.route_slot.reshape(-1).tolist(), where


# y is checked on every y_every-th call, and on every layer of every y_step-th step
@pytest.mark.parametrize("key,L_phys,steps,y_every,y_step,fq", [
    ("decode-L40-d2048-E128-top8", 40, 6, 4, 0, 22337),     # 40 layers d=2048 E=128 top-8, batch 1, full pool, cache 37 %
    ("decode-L40-d2048-E128-top8-b8", 40, 4, 16, 0, 22337),  # same, batch 8
    ("decode-L43-d4096-E256-top6", 2, 9, 0, 8, 18000),      # 43 layers d=4096 E=256 top-6, batch 1, cache 11 %, aliased
                                                             # pool: decisions on every call, y on every layer of steps 0, 8
])
def test_decode_full_size(key, L_phys, steps, y_every, y_step, fq):
    torch = torch_mod()
    wl = synth.WORKLOADS[key]
    s = wl.shape
    T = wl.T
    _say("decode full size", wl.name, "L_phys", L_phys)
    pool = PinnedPool(s, L_phys * s.E)
    pool.fill_device_random(wl.seed_key)
    eng = Engine(s, pool, wl.n_slots, T_max=T, frac_q16=fq, L_phys=L_phys)
    try:
        ref_cache = SlotTable(wl.n_slots, s.L, s.E)
        tr = synth.trace_for(wl, steps=steps)
        wr = [synth.router_weights(wl, l) for l in range(s.L)]
        wr_dev = [dev_u16(w) for w in wr]
        plan = ft.ft_plan()
        call = 0
        for st in range(steps):
            for l in range(s.L):
                x = synth.tokens(wl, st, l, T=T)
                allowed = synth.allowed_mask(tr[st, l], s.E)
                y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
                ft.ft_moe_decode_layer(eng.ctx, l, dev_u16(x), T, wr_dev[l], dev(allowed), y,
                                       plan=plan)
                torch.cuda.synchronize()
                idx, g, _ = route(x, wr[l], s.k, allowed)
                ref_plan = ref_cache.lookup(l, idx, fq, 1, -1)
                _compare_plan(plan, ref_plan, idx, (st, l))
                if (y_every and call % y_every == 0) or (y_step and st % y_step == 0):
                    ref_y = moe_layer(x, idx, g, lambda e: pool.view[(l % L_phys) * s.E + e], s.d, s.d_ff,
                                      workers=8)
                    ok, mx, l1 = within_tolerance(host(y), ref_y)
                    assert ok, (st, l, mx, l1)
                call += 1
        st_ = ft.ft_get_stats(eng.ctx)
        assert st_["fills"] == ref_cache.counters.fills and st_["cpu_experts"] == ref_cache.counters.cpu_experts
    finally:
        eng.destroy()
        pool.free()


def test_prefill_8k_chunk_full_size():
    """8192-token chunk through the d=4096, E=256, top-6, d_ff=2048 layer shape with
    double buffering (aliased pool of 2 physical layers), first two layers of the
    stack: the ids each layer call routed, all 8192 x 6, bit-exact; y on tokens that
    reach every one of the 256 expert groups (first row, the 32-row and 256-row tile
    edges, the last row of the largest group); residency after a pass ended early."""
    torch = torch_mod()
    wl = synth.WORKLOADS["prefill8k-L43-d4096-E256-top6"]
    s = wl.shape
    T = wl.T
    L_phys = 2
    n_layers = 2
    _say("prefill full size", wl.name)
    pool = PinnedPool(s, L_phys * s.E)
    pool.fill_device_random(wl.seed_key)
    eng = Engine(s, pool, wl.n_slots, T_max=T, frac_q16=0, min_fill=0, max_fetch=0, prefill_overlap=1,
                 L_phys=L_phys, cpu_threads=2)
    try:
        ref_cache = SlotTable(wl.n_slots, s.L, s.E)
        ft.ft_moe_prefill_begin(eng.ctx, eng.copy)
        bufs = ref_cache.prefill_begin()
        outs = []
        for l in range(n_layers):
            for e in (0, 1, s.E - 1):
                assert ft.ft_prefill_slot(eng.ctx, l, e) == bufs[l % 2][e]
            xd = synth.tokens_torch(wl.seed_key, 0, l, T, s.d)
            wr = synth.router_weights(wl, l)
            y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
            ids = torch.empty((T, s.k), dtype=torch.int32, device="cuda")
            ft.ft_moe_prefill_layer(eng.ctx, l, xd, T, dev_u16(wr), y, copy=eng.copy)
            ft.ft_layer_routing(eng.ctx, ids, None, T)  # same stream, before the next layer's router
            outs.append((l, xd, wr, y, ids))
        ft.ft_moe_prefill_end(eng.ctx)
        ref_cache.prefill_end(n_layers)
        torch.cuda.synchronize()
        for l, xd, wr, y, ids in outs:
            x = host(xd).view(np.uint16)
            _say("oracle routing of layer", l)
            idx, g, _ = route(x, wr, s.k, workers=8)
            assert np.array_equal(host(ids), idx), l
            sample, sizes = tile_cover_tokens(idx, s.E)
            assert int((sizes > 0).sum()) >= 250
            _say("oracle outputs of layer", l, "on", sample.size, "tokens")
            ref_y = moe_layer(x, idx, g, lambda e: pool.view[(l % L_phys) * s.E + e], s.d, s.d_ff, tokens=sample,
                              workers=8)
            ok, mx, l1 = within_tolerance(host(y)[sample], ref_y)
            assert ok, (l, mx, l1)
        res = ref_cache.resident()
        for l in range(n_layers + 1):
            for e in range(0, s.E, 37):
                assert ft.ft_expert_cache_where(eng.ctx, l, e) == res.get(l * s.E + e, -1)
    finally:
        eng.destroy()
        pool.free()


def test_prefill_8k_all_layers_sampled():
    """The whole 43-layer pass of an 8192-token chunk (d=4096, E=256, top-6, double
    buffered over an aliased pool of 2 physical layers): on every layer, the ids the
    layer call routed and y, for 3 seeded tokens, against the oracle; the residency the
    pass leaves."""
    torch = torch_mod()
    wl = synth.WORKLOADS["prefill8k-L43-d4096-E256-top6"]
    s = wl.shape
    T = wl.T
    L_phys = 2
    _say("prefill all layers", wl.name)
    pool = PinnedPool(s, L_phys * s.E)
    pool.fill_device_random(wl.seed_key)
    eng = Engine(s, pool, wl.n_slots, T_max=T, frac_q16=0, min_fill=0, max_fetch=0, prefill_overlap=1,
                 L_phys=L_phys, cpu_threads=2)
    try:
        ref_cache = SlotTable(wl.n_slots, s.L, s.E)
        ft.ft_moe_prefill_begin(eng.ctx, eng.copy)
        ref_cache.prefill_begin()
        rng = np.random.default_rng(43)
        outs = []
        for l in range(s.L):
            xd = synth.tokens_torch(wl.seed_key, 0, l, T, s.d)
            wr = synth.router_weights(wl, l)
            y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
            ids = torch.empty((T, s.k), dtype=torch.int32, device="cuda")
            ft.ft_moe_prefill_layer(eng.ctx, l, xd, T, dev_u16(wr), y, copy=eng.copy)
            ft.ft_layer_routing(eng.ctx, ids, None, T)
            sample = np.sort(rng.choice(T, size=3, replace=False))
            sel = torch.from_numpy(sample).cuda()
            outs.append((l, sample, xd.index_select(0, sel), wr, y.index_select(0, sel), ids.index_select(0, sel)))
        ft.ft_moe_prefill_end(eng.ctx)
        ref_cache.prefill_end(s.L)
        torch.cuda.synchronize()
        for l, sample, xs, wr, ys, ids in outs:
            x = host(xs).view(np.uint16)
            idx, g, _ = route(x, wr, s.k)
            assert np.array_equal(host(ids), idx), (l, sample)
            ref_y = moe_layer(x, idx, g, lambda e: pool.view[(l % L_phys) * s.E + e], s.d, s.d_ff, workers=8)
            ok, mx, l1 = within_tolerance(host(ys), ref_y)
            assert ok, (l, sample, mx, l1)
        res = ref_cache.resident()
        for l in (0, s.L - 3, s.L - 2, s.L - 1):
            for e in range(0, s.E, 17):
                assert ft.ft_expert_cache_where(eng.ctx, l, e) == res.get(l * s.E + e, -1)
    finally:
        eng.destroy()
        pool.free()


def test_router_and_grouping_8k_full_size():
    """Router ids bit-exact for all 8192 tokens of a chunk at d=4096, E=256, top-6, and the
    grouping of its 49152 pairs bit-exact."""
    torch = torch_mod()
    from oracle.permute import group_pairs
    from oracle.router import router_logits, topk
    wl = synth.WORKLOADS["prefill8k-L43-d4096-E256-top6"]
    s = wl.shape
    T = wl.T
    xd = synth.tokens_torch(wl.seed_key, 0, 0, T, s.d)
    wr = synth.router_weights(wl, 0)
    idx = torch.empty((T, s.k), dtype=torch.int32, device="cuda")
    g = torch.empty((T, s.k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, s.E), dtype=torch.float32, device="cuda")
    ft.ft_router_topk(xd, dev_u16(wr), None, T, s.d, s.E, s.k, idx, g, lg)
    P = T * s.k
    off = torch.empty(s.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(P, dtype=torch.int32, device="cuda")
    inv = torch.empty(P, dtype=torch.int32, device="cuda")
    wsb = ft.ft_permute_workspace_bytes(P, s.E)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    ft.ft_permute(idx, P, s.E, off, perm, inv, ws, wsb)
    torch.cuda.synchronize()
    x = host(xd).view(np.uint16)
    ref_lg = router_logits(x, wr, workers=8)
    assert np.array_equal(host(lg).view(np.uint32), ref_lg.view(np.uint32))
    ref_idx = topk(ref_lg, s.k)
    assert np.array_equal(host(idx), ref_idx)
    r_off, r_perm, r_inv = group_pairs(ref_idx, s.E)
    assert np.array_equal(host(off), r_off)
    assert np.array_equal(host(perm), r_perm)
    assert np.array_equal(host(inv), r_inv)
    assert int((np.diff(r_off) > 0).sum()) >= 250  # nearly all experts active in a prefill chunk
