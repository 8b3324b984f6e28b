"""CPU-only tests of libft: it loads, exports every symbol the header declares,
and its host-side decisions (fetch split, cache residency, prefill buffers,
resize) are bit-exact with the oracle.  No call here touches a GPU."""
import ctypes as C
import json
import os
import re

import numpy as np
import pytest

from moe_expert_offload_amd import ft
from moe_expert_offload_amd.synth import zipf_reuse_trace
from oracle.cache import SlotTable
from oracle.qstar import Q16, frac_q16, q_split

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "ft.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ft_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = ft.lib()
    declared = _header_functions()
    assert len(declared) >= 25
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(ft.EXPORTED) == declared


def test_frac_q16_bit_exact():
    rng = np.random.default_rng(0)
    pairs = [(52.7, 77.3), (25.1, 63.2), (11.8, 47.5), (0.0, 5.0), (9.0, 9.0), (10.0, 2.0)]
    pairs += [(float(a), float(b)) for a, b in rng.uniform(0.01, 300, size=(2000, 2))]
    # exact ties at half a Q16 unit
    pairs += [((i + 0.5) / Q16, 1.0) for i in range(0, 65536, 4099)]
    for bp, bh in pairs:
        assert ft.ft_frac_q16(bp, bh) == frac_q16(bp, bh), (bp, bh)


def test_qstar_split_bit_exact():
    rng = np.random.default_rng(1)
    fqs = list(range(0, Q16 + 1, 997)) + [Q16, 1, Q16 - 1, 16384, 27197]
    for fq in fqs:
        for m in range(0, 65):
            for min_fill, max_fetch, avail in ((1, -1, 10 ** 6), (0, -1, 10 ** 6), (2, 3, 7), (1, 0, 100)):
                assert ft.ft_qstar_split(m, fq, min_fill, max_fetch, avail) == q_split(m, fq, min_fill, max_fetch, avail)
    assert ft.lib().ft_qstar_split(-1, 0, 1, -1, 5) == ft.FT_EINVAL
    assert ft.lib().ft_qstar_split(3, Q16 + 1, 1, -1, 5) == ft.FT_EINVAL


def _ctx(L, E, d, d_ff, k, N, fq, min_fill=1, max_fetch=-1, overlap=0):
    shape = ft.make_shape(L, E, d, d_ff, k)
    cfg = ft.make_config(frac_q16=fq, min_fill=min_fill, max_fetch=max_fetch, prefill_overlap=overlap, T_max=8)
    return ft.ft_create(shape, cfg, n_slots=N)


def _compare(plan, ref):
    got = ft.plan_dict(plan)
    assert got["U"] == ref.U and got["H"] == ref.H and got["M"] == ref.M
    assert got["q"] == ref.q and got["n_c"] == len(ref.C) and got["avail"] == ref.avail
    assert got["F_slot"] == ref.F_slots and got["G_slot"] == ref.G_slots
    assert got["route_slot"] == ref.route_slot.reshape(-1).tolist()
    assert got["pair_group"] == ref.pair_group.reshape(-1).tolist()


@pytest.mark.parametrize("N,fq,min_fill,max_fetch,B", [
    (40, 30000, 1, -1, 1), (40, 30000, 0, -1, 4), (13, Q16, 1, -1, 2), (200, 8000, 1, 2, 3),
    (0, 30000, 1, -1, 2), (500, Q16, 1, -1, 8), (64, 0, 0, -1, 2)])
def test_controller_matches_oracle_over_trace(N, fq, min_fill, max_fetch, B):
    L, E, k, steps = 5, 32, 4, 60
    rng = np.random.default_rng(N + B)
    tr = zipf_reuse_trace(L, E, k, B, steps, 1.1, 0.6, rng)
    ctx = _ctx(L, E, 64, 64, k, N, fq, min_fill, max_fetch)
    try:
        ref = SlotTable(N, L, E)
        plan = ft.ft_plan()
        for s in range(steps):
            for layer in range(L):
                idx = np.ascontiguousarray(np.stack([rng.permutation(r) for r in tr[s, layer]]).astype(np.int32))
                ft.ft_expert_cache_lookup(ctx, layer, idx, B, plan)
                _compare(plan, ref.lookup(layer, idx, fq, min_fill, max_fetch))
        st = ft.ft_get_stats(ctx)
        rc = ref.counters
        assert (st["calls"], st["unique_hits"], st["unique_misses"], st["fills"], st["cpu_experts"]) == \
            (rc.calls, rc.unique_hits, rc.unique_misses, rc.fills, rc.cpu_experts)
        assert (st["reads"], st["read_hits"], st["read_fills"], st["read_cpu"]) == \
            (rc.reads, rc.read_hits, rc.read_fills, rc.read_cpu)
        for layer in range(L):
            for e in range(E):
                assert ft.ft_expert_cache_where(ctx, layer, e) == ref.where.get(layer * E + e, -1)
    finally:
        ft.ft_destroy(ctx)


def test_prefill_residency_and_resize_match_oracle():
    L, E, k, B = 6, 16, 3, 2
    rng = np.random.default_rng(3)
    tr = zipf_reuse_trace(L, E, k, B, 40, 1.1, 0.6, rng)
    ctx = _ctx(L, E, 64, 64, k, 40, 40000, overlap=1)
    try:
        ref = SlotTable(40, L, E)
        plan = ft.ft_plan()
        for s in range(40):
            if s == 12:
                ft.ft_moe_prefill_begin(ctx, 0)
                bufs = ref.prefill_begin()
                for layer in range(L):
                    for e in range(E):
                        assert ft.ft_prefill_slot(ctx, layer, e) == bufs[layer % 2][e]
                # decisions are refused while a prefill is open
                with pytest.raises(ft.FtError):
                    ft.ft_expert_cache_lookup(ctx, 0, np.zeros((1, k), np.int32), 1, plan)
                with pytest.raises(ft.FtError) as ei:
                    ft.ft_expert_cache_resize(ctx, None, 40)
                assert ei.value.status == ft.FT_EBUSY
                ft.ft_moe_prefill_end(ctx)
                ref.prefill_end(L)
            if s == 25:
                assert ft.ft_expert_cache_resize(ctx, None, 33) == ft.FT_OK
                ref.resize(33)
                assert ft.ft_get_stats(ctx)["calls"] == 0
            for layer in range(L):
                idx = np.ascontiguousarray(tr[s, layer].astype(np.int32))
                ft.ft_expert_cache_lookup(ctx, layer, idx, B, plan)
                _compare(plan, ref.lookup(layer, idx, 40000))
        # shrinking below 2E disables the prefill overlap with a warning code; prefill then
        # falls back to on-demand loading
        assert ft.ft_expert_cache_resize(ctx, None, 2 * E - 1) == ft.FT_WOVERLAP_OFF
        ref.resize(2 * E - 1)
        assert ft.ft_get_config(ctx).prefill_overlap == 0
        ft.ft_moe_prefill_begin(ctx, 0)
        assert ft.ft_prefill_slot(ctx, 0, 0) == -1
        for layer in range(L):
            idx = np.ascontiguousarray(np.stack([rng.choice(E, size=k, replace=False) for _ in range(20)]).astype(np.int32))
            groups, n_h, rounds = ft.ft_expert_cache_prefill_on_demand(ctx, layer, idx, 20)
            U, H, M, ref_rounds = ref.prefill_on_demand(layer, idx)
            assert rounds == ref_rounds and n_h == len(H) and [e for e, _ in groups] == H + M
        ft.ft_moe_prefill_end(ctx)
        for layer in range(L):
            for e in range(E):
                assert ft.ft_expert_cache_where(ctx, layer, e) == ref.where.get(layer * E + e, -1)
    finally:
        ft.ft_destroy(ctx)


@pytest.mark.parametrize("N,T", [(5, 16), (12, 40), (40, 64), (1, 4), (33, 200)])
def test_on_demand_prefill_decisions_bit_exact(N, T):
    """The C++ controller's on-demand prefill rounds and residency against the oracle,
    interleaved with decode lookups, over pools smaller than one layer's experts and
    larger than two."""
    L, E, k = 4, 16, 3
    rng = np.random.default_rng(N * 13 + T)
    tr = zipf_reuse_trace(L, E, k, 1, 8, 1.1, 0.6, rng)
    ctx = _ctx(L, E, 64, 200, k, N, 40000, overlap=0)
    try:
        ref = SlotTable(N, L, E)
        plan = ft.ft_plan()
        for s in range(8):
            for layer in range(L):
                idx = np.ascontiguousarray(tr[s, layer].astype(np.int32))
                ft.ft_expert_cache_lookup(ctx, layer, idx, 1, plan)
                _compare(plan, ref.lookup(layer, idx, 40000))
            if s % 3 == 1:
                ft.ft_moe_prefill_begin(ctx, 0)
                for layer in range(L):
                    idx = np.ascontiguousarray(
                        np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32))
                    groups, n_h, rounds = ft.ft_expert_cache_prefill_on_demand(ctx, layer, idx, T)
                    U, H, M, ref_rounds = ref.prefill_on_demand(layer, idx)
                    assert rounds == ref_rounds and n_h == len(H)
                ft.ft_moe_prefill_end(ctx)
        for layer in range(L):
            for e in range(E):
                assert ft.ft_expert_cache_where(ctx, layer, e) == ref.where.get(layer * E + e, -1)
    finally:
        ft.ft_destroy(ctx)


def test_error_codes():
    shape = ft.make_shape(4, 16, 64, 64, 2)
    with pytest.raises(ft.FtError) as ei:  # overlap needs 2E slots at construction
        ft.ft_create(shape, ft.make_config(prefill_overlap=1), n_slots=31)
    assert ei.value.status == ft.FT_ECAP
    with pytest.raises(ft.FtError) as ei:
        ft.ft_create(ft.make_shape(4, 16, 60, 64, 2), ft.make_config(), n_slots=8)
    assert ei.value.status == ft.FT_EINVAL
    with pytest.raises(ft.FtError) as ei:  # MXFP4 needs d and d_ff multiples of 128
        ft.ft_create(ft.make_shape(4, 16, 64, 128, 2, ft.FT_W_MXFP4), ft.make_config(), n_slots=8)
    assert ei.value.status == ft.FT_EINVAL
    with pytest.raises(ft.FtError) as ei:
        ft.ft_create(ft.make_shape(4, 16, 64, 64, 2, 7), ft.make_config(), n_slots=8)
    assert ei.value.status == ft.FT_EUNSUPPORTED
    mxs = ft.make_shape(4, 16, 256, 384, 2, ft.FT_W_MXFP4)
    assert ft.ft_record_bytes(mxs) == 3 * 256 * 384 // 2 + 3 * 256 * 384 // 32
    ft.ft_destroy(ft.ft_create(mxs, ft.make_config(), n_slots=8))
    ctx = ft.ft_create(shape, ft.make_config(), n_slots=8)
    try:
        with pytest.raises(ft.FtError):  # routed id out of range
            ft.ft_expert_cache_lookup(ctx, 0, np.array([[0, 99]], np.int32), 1)
        with pytest.raises(ft.FtError):  # T*k over the plan capacity
            ft.ft_expert_cache_lookup(ctx, 0, np.zeros((300, 2), np.int32), 300)
        with pytest.raises(ft.FtError):  # no device path in a decisions-only context
            ft.ft_moe_decode_layer(ctx, 0, 16, 1, 16, None, 16, compute=0)
    finally:
        ft.ft_destroy(ctx)
    assert ft.ft_record_bytes(shape) == 6 * 64 * 64
    assert ft.ft_workspace_bytes(shape, 8) > 0


def test_argument_checks_before_any_device_call():
    """Entry points refuse bad arguments with FT_EINVAL before touching a device: the
    routing read-back and the decode graph need a context with a device path and a
    matching T; the no-alloc permutation refuses sizes beyond its fixed scratch array.
    Addresses passed here are never dereferenced."""
    shape = ft.make_shape(4, 16, 64, 64, 2)
    ctx = ft.ft_create(shape, ft.make_config(), n_slots=8)
    fake = 1 << 20
    try:
        for call in (lambda: ft.ft_layer_routing(ctx, fake, fake, 1, stream=0),
                     lambda: ft.ft_decode_graph_create(ctx, 1, fake, [fake] * 4, None, fake)):
            with pytest.raises(ft.FtError) as ei:
                call()
            assert ei.value.status == ft.FT_EINVAL
            assert "device path" in str(ei.value)
    finally:
        ft.ft_destroy(ctx)
    for g in (None, 0):
        with pytest.raises(ft.FtError) as ei:
            ft.ft_decode_graph_launch(g, stream=0)
        assert ei.value.status == ft.FT_EINVAL
        with pytest.raises(ft.FtError) as ei:
            ft.ft_decode_graph_status(g)
        assert ei.value.status == ft.FT_EINVAL
        ft.ft_decode_graph_destroy(g)  # destroying nothing is not an error
    cap = ft.ft_permute_noalloc_max_scratch_bytes()
    assert cap == 1 << 20
    # largest P the array holds at 1024 groups fits; one past the byte bound does not
    P_fit = max(p for p in range(0, 1 << 18, 256) if ft.ft_permute_workspace_bytes(p, 1024) <= cap)
    assert P_fit >= 65536
    for P_, n_groups in ((16 * P_fit, 1024), (-1, 8), (16, 0), (16, 1025)):
        with pytest.raises(ft.FtError) as ei:
            ft.ft_permute_noalloc(fake, P_, n_groups, fake, fake, fake, stream=0)
        assert ei.value.status == ft.FT_EINVAL
    with pytest.raises(ft.FtError) as ei:  # null key with pairs to group
        ft.ft_permute_noalloc(None, 16, 8, fake, fake, fake, stream=0)
    assert ei.value.status == ft.FT_EINVAL


@pytest.mark.parametrize("T,d,d_ff,uses,threads", [
    (1, 256, 512, [[0], [0]], 3),
    (8, 520, 136, [[0, 3, 7], [2], [1, 2, 3, 4, 5, 6, 7, 0]], 4),
    (2, 2048, 768, [[0, 1]], 0),
])
def test_host_expert_kernel_matches_oracle(T, d, d_ff, uses, threads):
    """The CPU branch: gate-weighted partials of experts run on the host, against the fp64 oracle."""
    from moe_expert_offload_amd.synth import f32_to_bf16_bits, generator
    from oracle.common import bf16_to_f64, within_tolerance
    from oracle.ffn import expert_ffn, split_record
    rng = generator(50, T, d, d_ff)
    n_exp = len(uses)
    recs = [np.ascontiguousarray(f32_to_bf16_bits(rng.normal(0, 0.02, 3 * d * d_ff))) for _ in range(n_exp)]
    x = f32_to_bf16_bits(rng.normal(0, 1, (T, d)))
    use_off = np.cumsum([0] + [len(u) for u in uses]).astype(np.int32)
    use_t = np.array([t for u in uses for t in u], np.int32)
    use_g = rng.random(use_t.size).astype(np.float32)
    partial = np.full((T, d), np.nan, np.float32)
    ft.ft_host_experts(x, T, d, d_ff, recs, use_off, use_t, use_g, n_exp, threads, partial)
    ref = np.zeros((T, d))
    x64 = bf16_to_f64(x)
    for i in range(n_exp):
        W = split_record(recs[i], d, d_ff)
        for u in range(use_off[i], use_off[i + 1]):
            ref[use_t[u]] += float(use_g[u]) * expert_ffn(W, x64[use_t[u]:use_t[u] + 1])[0]
    ok, mx, l1 = within_tolerance(partial, ref, 1e-4, 1e-5)
    assert ok, (mx, l1)


@pytest.mark.parametrize("T,d,d_ff,uses,threads", [
    (1, 256, 512, [[0], [0]], 3),
    (8, 384, 128, [[0, 3, 7], [2], [1, 2, 3, 4, 5, 6, 7, 0]], 4),
    (2, 2048, 768, [[0, 1]], 0),
])
def test_host_expert_kernel_mxfp4_matches_oracle(T, d, d_ff, uses, threads):
    """The CPU branch over MXFP4 records (in-kernel dequantisation) against the oracle's
    exact dequantisation with bf16 activations."""
    from moe_expert_offload_amd.synth import f32_to_bf16_bits, generator, mxfp4_record_from_weights
    from oracle import mx
    from oracle.common import bf16_to_f64, within_tolerance
    rng = generator(51, T, d, d_ff)
    n_exp = len(uses)
    recs = [mxfp4_record_from_weights(rng.normal(0, 0.02, (d_ff, d)), rng.normal(0, 0.02, (d_ff, d)),
                                      rng.normal(0, 0.02, (d, d_ff))) for _ in range(n_exp)]
    x = f32_to_bf16_bits(rng.normal(0, 1, (T, d)))
    use_off = np.cumsum([0] + [len(u) for u in uses]).astype(np.int32)
    use_t = np.array([t for u in uses for t in u], np.int32)
    use_g = rng.random(use_t.size).astype(np.float32)
    partial = np.full((T, d), np.nan, np.float32)
    ft.ft_host_experts(x, T, d, d_ff, recs, use_off, use_t, use_g, n_exp, threads, partial, fmt=ft.FT_W_MXFP4)
    ref = np.zeros((T, d))
    x64 = bf16_to_f64(x)
    for i in range(n_exp):
        W = mx.split_record(recs[i], d, d_ff)
        for u in range(use_off[i], use_off[i + 1]):
            ref[use_t[u]] += float(use_g[u]) * mx.expert_ffn_decode(W, x64[use_t[u]:use_t[u] + 1])[0]
    ok, mxe, l1 = within_tolerance(partial, ref, 1e-4, 1e-5)
    assert ok, (mxe, l1)


# ---- the bandwidth profile: contended fraction, hybrid gate, profile files --------

def test_contended_fraction_bit_exact():
    from oracle.qstar import fetch_fraction_q16, frac_q16_contended
    rng = np.random.default_rng(7)
    pairs = [(52.7, 24.6), (25.1, 38.1), (0.0, 5.0), (5.0, 0.0), (1.0, 131071.0), (3.0, 131069.0)]
    pairs += [(float(a), float(b)) for a, b in rng.uniform(0.01, 300, size=(2000, 2))]
    for po, co in pairs:
        assert ft.ft_frac_q16_contended(po, co) == frac_q16_contended(po, co), (po, co)
    for bp, bh, po, co in rng.uniform(0.0, 300, size=(500, 4)):
        for pair in ((po, co), (0.0, co), (po, 0.0)):
            prof = ft.ft_bw_profile(float(bp), float(bh), float(pair[0]), float(pair[1]), ft.FT_W_BF16)
            assert ft.ft_fetch_fraction_q16(prof) == fetch_fraction_q16(bp, bh, *pair)


def test_hybrid_recommendation_matches_oracle():
    from oracle.qstar import recommend_hybrid
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "qstar_pages.json")))
    t1 = [(r["B_P"], r["B_H"]) for r in gold["table1"]["rows"]]
    rng = np.random.default_rng(8)
    cases = [t1, t1[1:3], [t1[1], t1[2], t1[4], t1[5]], [t1[0]], [t1[3]], [], [(10.0, 20.0)], [(10.0, 20.01)]]
    cases += [[tuple(p) for p in rng.uniform(1, 100, size=(int(rng.integers(1, 5)), 2))] for _ in range(300)]
    for c in cases:
        for thr in (2.0, 1.5):
            got = ft.ft_recommend_hybrid([p for p, _ in c], [h for _, h in c], thr)
            assert got == recommend_hybrid(c, thr), (c, thr)
    with pytest.raises(ft.FtError):
        ft.ft_recommend_hybrid([1.0], [3.0], 0.0)


def test_bandwidth_profile_file_round_trip(tmp_path):
    path = str(tmp_path / "prof_bf16.txt")
    prof = ft.ft_bw_profile(55.1e9, 163.3e9, 50.2e9, 101.7e9, ft.FT_W_BF16)
    ft.ft_bw_profile_save(path, prof)
    back = ft.ft_bw_profile_load(path, ft.FT_W_BF16)
    assert (back.B_P, back.B_H, back.pcie_ov, back.cpu_ov, back.fmt) == (55.1e9, 163.3e9, 50.2e9, 101.7e9, 0)
    # a profile says nothing about another expert format, and a missing file is no profile
    assert ft.ft_bw_profile_load(path, ft.FT_W_MXFP4) is None
    assert ft.ft_bw_profile_load(str(tmp_path / "absent.txt"), ft.FT_W_BF16) is None
    # a profile without the contended pair falls back to Eq. (4)
    path2 = str(tmp_path / "prof_mx.txt")
    ft.ft_bw_profile_save(path2, ft.ft_bw_profile(55.8e9, 156.0e9, 0.0, 0.0, ft.FT_W_MXFP4))
    p2 = ft.ft_bw_profile_load(path2, ft.FT_W_MXFP4)
    assert ft.ft_fetch_fraction_q16(p2) == ft.ft_frac_q16(55.8e9, 156.0e9)
    # incomplete files are refused
    (tmp_path / "bad.txt").write_text("format: bf16\nB_P: 1e9\n")
    assert ft.ft_bw_profile_load(str(tmp_path / "bad.txt"), ft.FT_W_BF16) is None
    with pytest.raises(ft.FtError):
        ft.ft_bw_profile_save(path, ft.ft_bw_profile(0.0, 1.0, 0.0, 0.0, ft.FT_W_BF16))


@pytest.mark.parametrize("L,E,k,R,prompt,decode,key", [
    (4, 16, 2, 3, 12, 30, 21),     # small pool: on-demand prefill below 2E slots
    (6, 32, 4, 2, 40, 25, 22),
    (5, 128, 8, 2, 64, 20, 23),    # the 40-layer shape's experts per layer and top-k
])
def test_placement_replay_matches_oracle(L, E, k, R, prompt, decode, key):
    """Fig. 4b replay: decode reads and misses of every policy, bit-exact with the
    oracle at capacities below and above 2E (or an error in both)."""
    from oracle.placement import replay
    from moe_expert_offload_amd.synth import generator
    tr = zipf_reuse_trace(L, E, k, R, prompt + decode, 1.1, 0.6, generator(key, 3))
    ids = np.ascontiguousarray(np.transpose(tr, (2, 0, 1, 3)).astype(np.int32))
    shape = ft.make_shape(L, E, 64, 64, k)
    pols = {"lru": ft.FT_PLACE_LRU, "hotset": ft.FT_PLACE_HOTSET, "static": ft.FT_PLACE_STATIC}
    for N in sorted({0, k, E - 1, E + 3, 2 * E - 1, 2 * E, 2 * E + 5, L * E // 3, L * E // 2, L * E, L * E + 7}):
        for name, pol in pols.items():
            try:
                want = replay(name, ids, L, E, N, prompt)
            except ValueError:
                with pytest.raises(ft.FtError) as ei:
                    ft.ft_replay_placement(pol, shape, N, ids, prompt)
                assert ei.value.status == ft.FT_ECAP and name == "lru"
                continue
            assert ft.ft_replay_placement(pol, shape, N, ids, prompt) == want, (name, N)


def test_placement_replay_rejects_bad_input():
    shape = ft.make_shape(2, 8, 64, 64, 2)
    ids = np.zeros((1, 3, 2, 2), dtype=np.int32)
    with pytest.raises(ft.FtError):
        ft.ft_replay_placement(7, shape, 4, ids, 1)
    ids[0, 2, 1, 0] = 8
    with pytest.raises(ft.FtError):
        ft.ft_replay_placement(ft.FT_PLACE_STATIC, shape, 4, ids, 1)
