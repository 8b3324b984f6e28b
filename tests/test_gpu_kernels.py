"""GPU parity of each kernel entry point against the oracle (through the C ABI).

Router logits, ids and the permutation are compared bit for bit; gates within
fp32 rounding; FFN outputs within the layer-output tolerance
(max|gpu-ref| <= 2e-2 max|ref|, sum|gpu-ref| / sum|ref| <= 3e-3).
"""
import numpy as np
import pytest

from moe_expert_offload_amd import ft
from moe_expert_offload_amd.synth import f32_to_bf16_bits, generator
from oracle.common import bf16_to_f64, within_tolerance
from oracle.ffn import expert_ffn, split_record
from oracle.permute import group_pairs
from oracle.router import gates as oracle_gates
from oracle.router import router_logits, topk
from tests.gpu_helpers import dev, dev_u16, host, torch_mod

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.mark.parametrize("T,d,E,k,use_allowed,zero_x", [
    (16, 256, 8, 2, False, False),      # single-layer configuration
    (1, 2048, 128, 8, True, False),     # decode, trace-driven
    (8, 2048, 128, 8, True, False),
    (37, 4096, 256, 6, False, False),
    (300, 4096, 256, 6, False, False),  # tile path for many tokens
    (70, 520, 33, 3, False, False),     # ragged d and E
    (5, 256, 16, 4, False, True),       # all-equal logits: ties go to the lower index
    (3, 256, 1024, 8, False, False),    # the largest expert count (16 experts per lane)
    (1, 2048, 600, 8, True, False),     # 600 experts, trace-driven
    (2, 64, 1, 1, False, False),        # one expert: top-1 of 1, gate 1
])
def test_router_bit_exact(T, d, E, k, use_allowed, zero_x):
    torch = torch_mod()
    _say("router", T, d, E, k, use_allowed, zero_x)
    rng = generator(90, 0, T, d, E)
    x = f32_to_bf16_bits(np.zeros((T, d)) if zero_x else rng.normal(0, 1, (T, d)))
    w = f32_to_bf16_bits(rng.normal(0, 0.02, (E, d)))
    allowed = None
    if use_allowed:
        allowed = np.zeros((T, E), np.uint8)
        for t in range(T):
            allowed[t, rng.choice(E, k, replace=False)] = 1
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    g = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ft.ft_router_topk(dev_u16(x), dev_u16(w), dev(allowed) if allowed is not None else None,
                      T, d, E, k, idx, g, lg)
    torch.cuda.synchronize()
    ref_lg = router_logits(x, w)
    assert np.array_equal(host(lg).view(np.uint32), ref_lg.view(np.uint32))
    ref_idx = topk(ref_lg, k, allowed)
    assert np.array_equal(host(idx), ref_idx)
    assert np.allclose(host(g), oracle_gates(ref_lg, ref_idx), rtol=2e-6, atol=1e-7)
    if zero_x:
        assert np.all(host(idx) == np.arange(k)[None, :])


@pytest.mark.parametrize("P,G", [(0, 3), (1, 1), (64, 8), (300, 17), (1000, 256), (512, 512),
                                 (5000, 1024), (49152, 256)])
def test_permute_bit_exact(P, G):
    torch = torch_mod()
    _say("permute", P, G)
    rng = generator(91, 0, P, G)
    key = rng.integers(-1, G, size=P).astype(np.int32)
    off = torch.empty(G + 1, dtype=torch.int32, device="cuda")
    perm = torch.full((max(P, 1),), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((max(P, 1),), -7, dtype=torch.int32, device="cuda")
    wsb = ft.ft_permute_workspace_bytes(P, G)
    ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device="cuda")
    dkey = dev(key) if P > 0 else torch.empty(1, dtype=torch.int32, device="cuda")
    ft.ft_permute(dkey, P, G, off, perm, inv, ws, wsb)
    torch.cuda.synchronize()
    r_off, r_perm, r_inv = group_pairs(key, G)
    assert np.array_equal(host(off), r_off)
    n = int(r_off[-1])
    assert np.array_equal(host(perm)[:n], r_perm)
    if P > 0:
        assert np.array_equal(host(inv)[:P], r_inv)


def _ffn_case(form, d, d_ff, rows, k=2, split=None, seed=0, max_rows=None):
    torch = torch_mod()
    _say("ffn", form, d, d_ff, rows, split)
    rng = generator(92, seed, d, d_ff, len(rows))
    G = len(rows)
    n_slots = G + 2
    recs = f32_to_bf16_bits(rng.normal(0, 0.02, (n_slots, 3 * d * d_ff)))
    group_slot = rng.permutation(n_slots)[:G].astype(np.int32)
    total = int(sum(rows))
    T = max(1, (total + k - 1) // k)
    pair_ids = rng.permutation(T * k)[:total].astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    x = f32_to_bf16_bits(rng.normal(0, 1, (T, d)))
    out = torch.full((max(total, 1), d), float("nan"), dtype=torch.float32, device="cuda")
    h = torch.empty(max(total, 1) * d_ff * 4, dtype=torch.uint8, device="cuda")
    args = (dev_u16(x), T, d, d_ff, k, dev_u16(recs), dev(group_slot), dev(offsets), dev(pair_ids), G)
    ranges = [(0, G)] if split is None else [(0, split), (split, G)]
    for g0, g1 in ranges:
        ft.ft_grouped_ffn(*args, g0, g1, max(rows) if max_rows is None else max_rows, h, out, form)
    torch.cuda.synchronize()
    got = host(out)[:total]
    x64 = bf16_to_f64(x)
    ref = np.zeros((total, d))
    for g in range(G):
        W = split_record(recs[group_slot[g]], d, d_ff)
        r = slice(offsets[g], offsets[g + 1])
        if offsets[g + 1] > offsets[g]:
            ref[r] = expert_ffn(W, x64[pair_ids[r] // k])
    ok, mx, l1 = within_tolerance(got, ref)
    assert ok, (mx, l1)
    return mx, l1


@pytest.mark.parametrize("d,d_ff,rows,split", [
    (256, 512, [1, 3, 0, 2, 8], None),
    (2048, 768, [1] * 8, 3),            # decode shape, hits then fills
    (2048, 768, [8, 5, 1, 2], None),
    (4096, 2048, [1, 2, 4], None),
    (520, 136, [2, 9], None),           # ragged sizes
    (256, 4096, [6, 1], None),          # d_ff = 4096: h staged in LDS 4 rows at a time
])
def test_grouped_ffn_rows_form(d, d_ff, rows, split):
    _ffn_case(1, d, d_ff, rows, split=split)


# One token (T = 1: every pair is token 0) takes the form that stages the token row in
# LDS once per block; groups of one row, and groups of more rows than the stated bound of
# rows per group (the form then takes them one after another).
@pytest.mark.parametrize("d,d_ff,rows,max_rows", [
    (4096, 2048, [1, 1, 1, 1], 1),
    (4096, 2048, [1, 3], 1),
    (2048, 768, [2, 1, 1], 1),
    (4096, 2048, [3, 1], 2),            # batched form, a group above the bound
])
def test_grouped_ffn_rows_form_one_token(d, d_ff, rows, max_rows):
    assert sum(rows) == 4
    _ffn_case(1, d, d_ff, rows, k=4, max_rows=max_rows)


@pytest.mark.parametrize("d,d_ff,rows", [
    (256, 512, [40, 1, 300, 77, 0]),    # more rows than one tile, a single row, an empty group
    (4096, 2048, [192, 250, 5]),        # prefill shape
    (2048, 768, [64, 130]),
    (256, 512, [1100, 3, 0, 20]),       # one expert with five passes of rows (a skewed load)
])
def test_grouped_ffn_mfma_form(d, d_ff, rows):
    _ffn_case(2, d, d_ff, rows)


@pytest.mark.parametrize("split", [None, 150])
def test_grouped_ffn_mfma_form_more_tiles_than_blocks(split):
    """300 groups of one tile each: more tiles than compute units, so every block of the
    persistent MFMA kernels runs several (and empty groups are skipped in between)."""
    _ffn_case(2, 256, 128, [(i * 37) % 70 for i in range(300)], split=split)


@pytest.mark.parametrize("with_cpu,k", [(False, 3), (True, 3), (True, 8)])
def test_combine(with_cpu, k):
    torch = torch_mod()
    _say("combine", with_cpu, k)
    rng = generator(93, int(with_cpu), k)
    T, d = 5, 256
    inv = np.arange(T * k, dtype=np.int32)
    inv[[1, 7, 14]] = -1
    out = rng.normal(size=(T * k, d)).astype(np.float32)
    gates = rng.random((T, k)).astype(np.float32)
    cpu = rng.normal(size=(T, d)).astype(np.float32) if with_cpu else None
    y = torch.empty((T, d), dtype=torch.float32, device="cuda")
    ft.ft_combine(dev(out), dev(inv), dev(gates), dev(cpu) if with_cpu else None, T, k, d, y)
    torch.cuda.synchronize()
    ref = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            if inv[t * k + j] >= 0:
                ref[t] += float(gates[t, j]) * out[inv[t * k + j]].astype(np.float64)
        if with_cpu:
            ref[t] += cpu[t]
    assert np.allclose(host(y), ref, rtol=1e-5, atol=1e-5)


def test_contended_bandwidth_pair_and_profile_file(tmp_path):
    """The contended pair at the 40-layer d=2048 shape: each rate is positive and
    finite (the rates next to the uncontended B_P and B_H are printed, not compared:
    separate measurements on a shared host spread by more than any fixed margin);
    the profile file keyed by this GPU's UUID round-trips and gives the contended
    fraction."""
    from moe_expert_offload_amd.synth import Shape
    from tests.gpu_helpers import PinnedPool
    torch = torch_mod()
    s = Shape(40, 128, 2048, 768, 8)
    pool = PinnedPool(s, 16)
    pool.fill_device_random(2)
    shape = ft.make_shape(s.L, s.E, s.d, s.d_ff, s.k)
    scratch = torch.empty(8 * s.record_bytes, dtype=torch.uint8, device="cuda")
    _say("bench_bw and bench_bw_contended, 16 records")
    B_P, B_H = ft.ft_bench_bw(shape, pool.ptr, 8, scratch, 0)
    po, co = ft.ft_bench_bw_contended(shape, pool.ptr, 16, scratch, 0)
    _say(f"B_P {B_P / 1e9:.1f} B_H {B_H / 1e9:.1f} pcie_ov {po / 1e9:.1f} cpu_ov {co / 1e9:.1f} GB/s")
    assert 0.0 < po < float("inf") and 0.0 < co < float("inf")
    assert 0.0 < B_P < float("inf") and 0.0 < B_H < float("inf")
    path = ft.ft_bw_profile_path(torch.cuda.current_device(), ft.FT_W_BF16, str(tmp_path))
    assert path.startswith(str(tmp_path) + "/ft_bw_") and path.endswith("_bf16.txt") and len(path) > len(str(tmp_path)) + 40
    ft.ft_bw_profile_save(path, ft.ft_bw_profile(B_P, B_H, po, co, ft.FT_W_BF16))
    prof = ft.ft_bw_profile_load(path, ft.FT_W_BF16)
    assert ft.ft_fetch_fraction_q16(prof) == ft.ft_frac_q16_contended(po, co)
    assert ft.ft_bw_profile_load(path, ft.FT_W_MXFP4) is None
