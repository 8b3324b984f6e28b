"""GPU parity of the MXFP4 expert path against the oracle (through the C ABI).

MXFP8 conversions of x and h (codes and scales) are compared bit for bit with the
oracle's OCP MX conversion of the same values; FFN and layer outputs within
max|gpu-ref| <= 2e-2 max|ref| and sum|gpu-ref| / sum|ref| <= 3e-3; routing and
cache decisions bit for bit.
"""
import numpy as np
import pytest

from moe_expert_offload_amd import ft, synth
from moe_expert_offload_amd.synth import (Shape, Workload, allowed_mask, f32_to_bf16_bits, generator,
                                          mxfp4_expert_record, mxfp4_record_from_weights, router_weights, tokens,
                                          zipf_reuse_trace)
from oracle import mx
from oracle.cache import SlotTable
from oracle.common import bf16_to_f64, within_tolerance
from oracle.layer import decode_layer, prefill_layer
from oracle.qstar import Q16
from oracle.router import route
from tests.gpu_helpers import Engine, PinnedPool, dev, dev_u16, host, tile_cover_tokens, torch_mod

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _align(n):
    return (n + 255) // 256 * 256


def _records(rng, n, d, d_ff):
    return np.stack([mxfp4_record_from_weights(rng.normal(0, 0.02, (d_ff, d)), rng.normal(0, 0.02, (d_ff, d)),
                                               rng.normal(0, 0.02, (d, d_ff))) for _ in range(n)])


def _mx_ffn_case(form, d, d_ff, rows, k=2, split=None, seed=0):
    torch = torch_mod()
    _say("mx ffn", form, d, d_ff, rows, split)
    rng = generator(93, seed, d, d_ff, len(rows))
    G = len(rows)
    n_slots = G + 1
    recs = _records(rng, n_slots, d, d_ff)
    group_slot = rng.permutation(n_slots)[:G].astype(np.int32)
    total = int(sum(rows))
    T = max(1, (total + k - 1) // k)
    pair_ids = rng.permutation(T * k)[:total].astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    x = f32_to_bf16_bits(rng.normal(0, 1, (T, d)))
    x[0, :32] = 0  # an all-zero activation block
    out = torch.full((max(total, 1), d), float("nan"), dtype=torch.float32, device="cuda")
    wsb = ft.ft_grouped_ffn_mx_workspace_bytes(T, d, d_ff, total)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    args = (dev_u16(x), T, d, d_ff, k, dev(recs), dev(group_slot), dev(offsets), dev(pair_ids), G)
    ranges = [(0, G)] if split is None else [(0, split), (split, G)]
    for g0, g1 in ranges:
        ft.ft_grouped_ffn_mx(*args, g0, g1, max(rows), total, ws, wsb, out, form)
    torch.cuda.synchronize()
    got = host(out)[:total]
    x64 = bf16_to_f64(x)
    ref = np.zeros((total, d))
    ffn = mx.expert_ffn_decode if form == 1 else mx.expert_ffn_prefill
    for g in range(G):
        W = mx.split_record(recs[group_slot[g]], d, d_ff)
        r = slice(offsets[g], offsets[g + 1])
        if offsets[g + 1] > offsets[g]:
            ref[r] = ffn(W, x64[pair_ids[r] // k])
    ok, mxe, l1 = within_tolerance(got, ref)
    assert ok, (mxe, l1)
    if form == 2 and total > 0:
        # MXFP8 copies left in the workspace: x bit for bit; h (converted inside the
        # gate/up kernel from its fp32 value) against the oracle's conversion of its
        # fp64 h: equal except next to rounding boundaries.  The scaled MFMA sums its
        # 64 products with an error of about 1e-4 of their absolute sum, so h carries
        # absolute errors of that order relative to its row's size; a block's small
        # elements may then move by more than one step, hence the X/8 of slack.
        wsh = host(ws)
        o_x = _align(total * d_ff * 4)
        o_h = o_x + _align(T * d + T * d // 32)
        xq = wsh[o_x:o_x + T * d].reshape(T, d)
        xs = wsh[o_x + T * d:o_x + T * d + T * d // 32].reshape(T, d // 32)
        rc, rs = mx.quantize_act_codes(x64)
        assert np.array_equal(xq, rc) and np.array_equal(xs, rs)
        assert xs[0, 0] == 0 and not xq[0, :32].any()
        hq = wsh[o_h:o_h + total * d_ff].reshape(total, d_ff)
        hs = wsh[o_h + total * d_ff:o_h + total * d_ff + total * d_ff // 32].reshape(total, d_ff // 32)
        xdq = mx.quantize_act(x64)
        h_ref = np.zeros((total, d_ff))
        for g in range(G):
            wg, wu, _ = mx.split_record(recs[group_slot[g]], d, d_ff)
            r = slice(offsets[g], offsets[g + 1])
            xr = xdq[pair_ids[r] // k]
            h_ref[r] = mx.silu(xr @ wg.T) * (xr @ wu.T)
        rc, rs = mx.quantize_act_codes(h_ref)
        assert (hq == rc).mean() >= 0.99 and (hs == rs).mean() >= 0.99
        assert np.abs(hs.astype(int) - rs.astype(int)).max() <= 1
        got_v = mx.e8m0_value(np.repeat(hs, 32, axis=1)) * mx.e4m3_value(hq)
        ref_v = mx.e8m0_value(np.repeat(rs, 32, axis=1)) * mx.e4m3_value(rc)
        step = np.maximum(np.abs(got_v), np.abs(ref_v)) / 8 + mx.e8m0_value(np.repeat(np.maximum(hs, rs), 32, axis=1)) / 8
        bad = np.argwhere(np.abs(got_v - ref_v) > step)
        if bad.size:
            i, j = bad[0]
            b = j // 32
            pytest.fail(f"{len(bad)} h codes off by more than a step; first at row {i} col {j}: "
                        f"gpu code {hq[i, j]} scale {hs[i, b]} value {got_v[i, j]}, oracle code {rc[i, j]} "
                        f"scale {rs[i, b]} value {ref_v[i, j]}, h {h_ref[i, j]}, block amax "
                        f"{np.abs(h_ref[i, 32 * b:32 * b + 32]).max()}")


@pytest.mark.parametrize("d,d_ff,rows,split", [
    (256, 512, [1, 3, 0, 2, 8], None),
    (2048, 768, [1] * 6, 2),            # decode shape, hits then fills
    (4096, 2048, [1, 2], None),         # the MXFP4 decode shape
    (4096, 2048, [1, 1, 1], 1),         # the same at one token per group
    (384, 128, [9, 1], None),
    (256, 4096, [6, 1], None),          # d_ff = 4096: h staged in LDS 4 rows at a time
])
def test_mx_grouped_ffn_rows_form(d, d_ff, rows, split):
    _mx_ffn_case(1, d, d_ff, rows, split=split)


@pytest.mark.parametrize("d,d_ff,rows", [
    (256, 512, [40, 1, 300, 77, 0]),    # more rows than one tile, a single row, an empty group
    (512, 384, [257, 3]),
    (4096, 2048, [96, 260]),            # prefill shape
    (256, 128, [40, 300, 5]),           # one-stage down items, two-stage gate/up items
    (512, 1024, [(37 * i) % 300 for i in range(40)]),  # more blocks than compute units
    (256, 512, [1100, 3, 0, 20]),       # one expert with five passes of rows (a skewed load)
])
def test_mx_grouped_ffn_mfma_form(d, d_ff, rows):
    _mx_ffn_case(2, d, d_ff, rows)


def _mx_stack(wl: Workload):
    s = wl.shape
    pool = PinnedPool(s, s.L * s.E)
    for l in range(s.L):
        for e in range(s.E):
            pool.view[l * s.E + e] = mxfp4_expert_record(wl, l, e)
    wr = [router_weights(wl, l) for l in range(s.L)]
    return pool, wr


def _compare_plan(plan, ref_plan, ref_idx, where):
    got = ft.plan_dict(plan)
    assert got["idx"] == ref_idx.reshape(-1).tolist(), where
    assert (got["U"], got["H"], got["M"], got["q"]) == (ref_plan.U, ref_plan.H, ref_plan.M, ref_plan.q), where
    assert got["F_slot"] == ref_plan.F_slots and got["G_slot"] == ref_plan.G_slots, where
    assert got["route_slot"] == ref_plan.route_slot.reshape(-1).tolist(), where


MXS = Workload("small-mxfp4", 13, Shape(3, 16, 256, 384, 4, True), 2, 0.5)


@pytest.mark.parametrize("fq,T", [(20000, 2), (0, 1), (Q16, 4), (20000, 64)])
def test_mx_decode_trace_parity(fq, T):
    """Decode with MXFP4 experts: hits, fills and CPU-branch experts (in-kernel dequantisation)."""
    torch = torch_mod()
    _say("mx decode", fq, T)
    s = MXS.shape
    pool, wr = _mx_stack(MXS)
    N = 20
    eng = Engine(s, pool, N, T_max=max(T, 8), frac_q16=fq, min_fill=1 if fq else 0, max_fetch=-1 if fq else 0,
                 cpu_threads=4)
    try:
        ref_cache = SlotTable(N, s.L, s.E)
        tr = zipf_reuse_trace(s.L, s.E, s.k, T, 5, 1.1, 0.6, generator(13, 3, T))
        wr_dev = [dev_u16(w) for w in wr]
        plan = ft.ft_plan()
        for step in range(tr.shape[0]):
            for l in range(s.L):
                x = tokens(MXS, step, l, T=T)
                allowed = allowed_mask(tr[step, l], s.E)
                y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
                ft.ft_moe_decode_layer(eng.ctx, l, dev_u16(x), T, wr_dev[l], dev(allowed), y,
                                       plan=plan)
                torch.cuda.synchronize()
                ref = decode_layer(ref_cache, l, x, wr[l], s.k, lambda e: pool.view[l * s.E + e], s.d, s.d_ff,
                                   fq, 1 if fq else 0, -1 if fq else 0, allowed, fmt="mxfp4")
                _compare_plan(plan, ref["plan"], ref["idx"], (step, l))
                ok, mxe, l1 = within_tolerance(host(y), ref["y"])
                assert ok, (step, l, mxe, l1)
        st = ft.ft_get_stats(eng.ctx)
        assert st["fills"] == ref_cache.counters.fills
        assert st["cpu_experts"] == ref_cache.counters.cpu_experts
    finally:
        eng.destroy()
        pool.free()


@pytest.mark.parametrize("T", [300, 1])
def test_mx_prefill_double_buffer_then_resize(T):
    """Prefill with MXFP4 experts on the scaled MFMA (double-buffered), a decode step,
    then a resize at a safe point and more decode."""
    torch = torch_mod()
    _say("mx prefill", T)
    s = MXS.shape
    pool, wr = _mx_stack(MXS)
    N = 40
    eng = Engine(s, pool, N, T_max=max(T, 8), frac_q16=30000, prefill_overlap=1, cpu_threads=4)
    try:
        ref_cache = SlotTable(N, s.L, s.E)
        wr_dev = [dev_u16(w) for w in wr]
        ft.ft_moe_prefill_begin(eng.ctx, eng.copy)
        bufs = ref_cache.prefill_begin()
        ys = []
        for l in range(s.L):
            assert ft.ft_prefill_slot(eng.ctx, l, s.E - 1) == bufs[l % 2][s.E - 1]
            x = tokens(MXS, 0, l, T=T)
            y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
            ft.ft_moe_prefill_layer(eng.ctx, l, dev_u16(x), T, wr_dev[l], y, copy=eng.copy)
            ys.append((x, y))
        ft.ft_moe_prefill_end(eng.ctx)
        ref_cache.prefill_end(s.L)
        torch.cuda.synchronize()
        for l, (x, y) in enumerate(ys):
            ref = prefill_layer(x, wr[l], s.k, lambda e: pool.view[l * s.E + e], s.d, s.d_ff, fmt="mxfp4")
            ok, mxe, l1 = within_tolerance(host(y), ref["y"])
            assert ok, (l, mxe, l1)
        tr = zipf_reuse_trace(s.L, s.E, s.k, 1, 4, 1.1, 0.6, generator(13, 5))
        small = torch.empty(20 * s.record_bytes, dtype=torch.uint8, device="cuda")
        plan = ft.ft_plan()
        for step in range(4):
            if step == 2:
                torch.cuda.synchronize()
                assert ft.ft_expert_cache_resize(eng.ctx, small, 20) == ft.FT_WOVERLAP_OFF
                ref_cache.resize(20)
            for l in range(s.L):
                x = tokens(MXS, 40 + step, l, T=1)
                allowed = allowed_mask(tr[step, l], s.E)
                y = torch.empty((1, s.d), dtype=torch.float32, device="cuda")
                ft.ft_moe_decode_layer(eng.ctx, l, dev_u16(x), 1, wr_dev[l], dev(allowed), y,
                                       plan=plan)
                torch.cuda.synchronize()
                ref = decode_layer(ref_cache, l, x, wr[l], s.k, lambda e: pool.view[l * s.E + e], s.d, s.d_ff,
                                   30000, 1, -1, allowed, fmt="mxfp4")
                _compare_plan(plan, ref["plan"], ref["idx"], (step, l))
                assert within_tolerance(host(y), ref["y"])[0], (step, l)
        # with 20 < 2E slots the next prefill loads each layer's routed experts on demand
        ft.ft_moe_prefill_begin(eng.ctx, eng.copy)
        for l in range(s.L):
            x = tokens(MXS, 7, l, T=T)
            y = torch.empty((T, s.d), dtype=torch.float32, device="cuda")
            ft.ft_moe_prefill_layer(eng.ctx, l, dev_u16(x), T, wr_dev[l], y, copy=eng.copy)
            torch.cuda.synchronize()
            ref = prefill_layer(x, wr[l], s.k, lambda e: pool.view[l * s.E + e], s.d, s.d_ff, fmt="mxfp4")
            ref_cache.prefill_on_demand(l, ref["idx"])
            ok, mxe, l1 = within_tolerance(host(y), ref["y"])
            assert ok, ("on demand", l, mxe, l1)
        ft.ft_moe_prefill_end(eng.ctx)
        for l in range(s.L):
            for e in range(s.E):
                assert ft.ft_expert_cache_where(eng.ctx, l, e) == ref_cache.where.get(l * s.E + e, -1)
    finally:
        eng.destroy()
        pool.free()


def test_mx_full_size_prefill_chunk_and_decode():
    """The MXFP4 configuration at full size: d=4096, E=256, top-6, d_ff=2048; one
    8192-token chunk through two layers (double-buffered, aliased pool of two
    physical layers): every routed id bit-exact, y on tokens reaching every expert
    group and the tile edges; then 9 batch-1 decode steps over all 43 layers with the cache
    of 1210 slots, resized at a safe point to 605 slots before step 5: every decision
    bit-exact, across the resize too, and y on every layer of steps 0 and 8."""
    torch = torch_mod()
    wl = synth.WORKLOADS["mxfp4-prefill8k-L43-d4096-E256-top6"]
    s = wl.shape
    L_phys = 2
    _say("mx full size", wl.name)
    pool = PinnedPool(s, L_phys * s.E)
    pool.fill_device_random(wl.seed_key)
    eng = Engine(s, pool, wl.n_slots, T_max=wl.T, frac_q16=20000, prefill_overlap=1, L_phys=L_phys, cpu_threads=0)
    try:
        ref_cache = SlotTable(wl.n_slots, s.L, s.E)
        ft.ft_moe_prefill_begin(eng.ctx, eng.copy)
        ref_cache.prefill_begin()
        outs = []
        for l in range(2):
            xd = synth.tokens_torch(wl.seed_key, 0, l, wl.T, s.d)
            wr = synth.router_weights(wl, l)
            y = torch.empty((wl.T, s.d), dtype=torch.float32, device="cuda")
            ids = torch.empty((wl.T, s.k), dtype=torch.int32, device="cuda")
            ft.ft_moe_prefill_layer(eng.ctx, l, xd, wl.T, dev_u16(wr), y, copy=eng.copy)
            ft.ft_layer_routing(eng.ctx, ids, None, wl.T)
            outs.append((l, xd, wr, y, ids))
        ft.ft_moe_prefill_end(eng.ctx)
        ref_cache.prefill_end(2)
        torch.cuda.synchronize()
        for l, xd, wr, y, ids in outs:
            x = host(xd).view(np.uint16)
            _say("oracle routing of layer", l)
            idx, g, _ = route(x, wr, s.k, workers=8)
            assert np.array_equal(host(ids), idx), l  # every id the prefill layer routed
            sample, sizes = tile_cover_tokens(idx, s.E)
            _say("oracle outputs of layer", l, "on", sample.size, "tokens")
            ref_y = mx.moe_layer(x, idx, g, lambda e: pool.view[(l % L_phys) * s.E + e], s.d, s.d_ff,
                                 form="prefill", tokens=sample, workers=8)
            ok, mxe, l1 = within_tolerance(host(y)[sample], ref_y)
            assert ok, (l, mxe, l1)
        wd = synth.WORKLOADS["mxfp4-decode-L43-d4096-E256-top6"]
        tr = synth.trace_for(wd, steps=9)
        plan = ft.ft_plan()
        small = None
        for st in range(9):  # decisions on every call; outputs on every layer of steps 0 and 8
            if st == 5:
                torch.cuda.synchronize()
                small = torch.empty(605 * s.record_bytes, dtype=torch.uint8, device="cuda")
                assert ft.ft_expert_cache_resize(eng.ctx, small, 605) == ft.FT_OK
                ref_cache.resize(605)
            for l in range(s.L):
                x = synth.tokens(wd, st, l, T=1)
                wr = synth.router_weights(wd, l)
                allowed = allowed_mask(tr[st, l], s.E)
                y = torch.empty((1, s.d), dtype=torch.float32, device="cuda")
                ft.ft_moe_decode_layer(eng.ctx, l, dev_u16(x), 1, dev_u16(wr), dev(allowed), y,
                                       plan=plan)
                torch.cuda.synchronize()
                idx, g, _ = route(x, wr, s.k, allowed)
                ref_plan = ref_cache.lookup(l, idx, 20000, 1, -1)
                _compare_plan(plan, ref_plan, idx, (st, l))
                if st % 8:
                    continue
                ref_y = mx.moe_layer(x, idx, g, lambda e: pool.view[(l % L_phys) * s.E + e], s.d, s.d_ff,
                                     workers=8)
                ok, mxe, l1 = within_tolerance(host(y), ref_y)
                assert ok, (st, l, mxe, l1)
    finally:
        eng.destroy()
        pool.free()


def test_mx_prefill_8k_all_layers_sampled():
    """The whole 43-layer pass of an 8192-token chunk with MXFP4 experts (scaled MFMA on
    MXFP8 activations, double buffered over an aliased pool of 2 physical layers): on every
    layer, the ids the layer call routed and y, for 3 seeded tokens, against the oracle's
    prefill form; the residency the pass leaves."""
    torch = torch_mod()
    wl = synth.WORKLOADS["mxfp4-prefill8k-L43-d4096-E256-top6"]
    s = wl.shape
    T = wl.T
    L_phys = 2
    _say("mx prefill all layers", wl.name)
    pool = PinnedPool(s, L_phys * s.E)
    pool.fill_device_random(wl.seed_key)
    eng = Engine(s, pool, wl.n_slots, T_max=T, frac_q16=20000, prefill_overlap=1, L_phys=L_phys, cpu_threads=0)
    try:
        ref_cache = SlotTable(wl.n_slots, s.L, s.E)
        ft.ft_moe_prefill_begin(eng.ctx, eng.copy)
        ref_cache.prefill_begin()
        rng = np.random.default_rng(53)
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
            ref_y = mx.moe_layer(x, idx, g, lambda e: pool.view[(l % L_phys) * s.E + e], s.d, s.d_ff,
                                 form="prefill", workers=8)
            ok, mxe, l1 = within_tolerance(host(ys), ref_y)
            assert ok, (l, sample, mxe, l1)
        res = ref_cache.resident()
        for l in (0, s.L - 3, s.L - 2, s.L - 1):
            for e in range(0, s.E, 17):
                assert ft.ft_expert_cache_where(eng.ctx, l, e) == res.get(l * s.E + e, -1)
    finally:
        eng.destroy()
        pool.free()
