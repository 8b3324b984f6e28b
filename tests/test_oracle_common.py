"""Pins of the oracle's helpers and of the exact merge.

* within_tolerance, the checker behind every float parity assertion: passes just
  inside each bound, fails just outside each one (one at a time), and treats an
  all-zero reference as needing an exact match.  Each pin is a function of the
  checker under test, and plausible slips of it (``or`` for ``and``, the l1 ratio
  over the max, a bound compared with ``<`` against its own edge) are shown to
  fail at least one pin.
* bf16_to_f64 / bf16_to_f32 against words whose values follow from the binary32
  layout by hand: sign, exponent and the top 7 mantissa bits.
* the exact merge ([FT] §3.2: the GPU and CPU partial sums merge into the exact
  MoE output, with no algorithmic approximation; §8 C10): for every forced split
  q in [0, m] the GPU partial plus the CPU partial equals the layer output to
  1e-12, every pair lands in exactly one partial, and a pair of C contributes
  nothing to the GPU partial.
* the read counters and pair groups of both cache simulators on a hand-worked
  three-call case.
"""
import math

import numpy as np
import pytest

from moe_expert_offload_amd.synth import Shape, Workload, expert_record, router_weights, tokens
from oracle.cache import OrderedLRU, SlotTable
from oracle.common import bf16_to_f32, bf16_to_f64, within_tolerance
from oracle.layer import decode_layer
from oracle.qstar import Q16


# ---- within_tolerance ------------------------------------------------------------

def _pins_within_tolerance(check):
    """The pins as a list of failures (empty when `check` behaves as the tolerance
    max|d| <= 2e-2 max|ref| and sum|d| / sum|ref| <= 3e-3 says)."""
    bad = []
    ref = np.zeros(1000)
    ref[0] = 10.0       # max|ref| = 10, sum|ref| = 10 + 999 * 1 = 1009
    ref[1:] = 1.0
    tiny = 1e-9

    def expect(got, want, what):
        ok = check(got, ref)[0]
        if bool(ok) != want:
            bad.append(what)

    # max bound alone: one entry off by just under / just over 2e-2 * 10 = 0.2
    # (0.2 / 1009 is far below the l1 bound)
    g = ref.copy(); g[5] += 0.2 - tiny
    expect(g, True, "max just inside")
    g = ref.copy(); g[5] += 0.2 + tiny
    expect(g, False, "max just outside")
    # l1 bound alone: spread 3e-3 * 1009 = 3.027 over 999 entries (each 0.00303, far
    # below the max bound)
    spread = 3e-3 * 1009.0
    g = ref.copy(); g[1:] += (spread - 1e-6) / 999
    expect(g, True, "l1 just inside")
    g = ref.copy(); g[1:] += (spread + 1e-6) / 999
    expect(g, False, "l1 just outside")
    # both outside, and a sign flip of the whole output
    expect(ref + 0.5, False, "both outside")
    expect(-ref, False, "sign flip")
    # ratios reported
    g = ref.copy(); g[5] += 0.1
    ok, mx, l1 = check(g, ref)
    if not (abs(mx - 0.01) < 1e-12 and abs(l1 - 0.1 / 1009.0) < 1e-12):
        bad.append("ratios")
    # an all-zero reference needs an exact match
    z = np.zeros(8)
    if not check(z, z)[0]:
        bad.append("zero reference, exact")
    if check(z + 1e-3, z)[0]:
        bad.append("zero reference, off")
    return bad


def test_within_tolerance_pins():
    assert _pins_within_tolerance(within_tolerance) == []


def _broken_or(got, ref, max_rel=2e-2, l1_rel=3e-3):
    d = np.abs(np.asarray(got, float) - ref)
    mx, l1 = d.max() / np.abs(ref).max(), d.sum() / np.abs(ref).sum()
    return (mx <= max_rel or l1 <= l1_rel), mx, l1


def _broken_l1_over_max(got, ref, max_rel=2e-2, l1_rel=3e-3):
    d = np.abs(np.asarray(got, float) - ref)
    mx, l1 = d.max() / np.abs(ref).max(), d.sum() / np.abs(ref).max()
    return (mx <= max_rel and l1 <= l1_rel), mx, l1


def _broken_mean_abs(got, ref, max_rel=2e-2, l1_rel=3e-3):
    d = np.abs(np.asarray(got, float) - ref)
    mx, l1 = d.max() / np.abs(ref).max(), d.mean()
    return (mx <= max_rel and l1 <= l1_rel), mx, l1


def _broken_signed(got, ref, max_rel=2e-2, l1_rel=3e-3):
    d = np.asarray(got, float) - ref
    mx, l1 = d.max() / np.abs(ref).max(), d.sum() / np.abs(ref).sum()
    return (mx <= max_rel and l1 <= l1_rel), mx, l1


@pytest.mark.parametrize("broken", [_broken_or, _broken_l1_over_max, _broken_mean_abs, _broken_signed])
def test_within_tolerance_pins_catch_plausible_slips(broken):
    with np.errstate(all="ignore"):
        assert _pins_within_tolerance(broken) != []


# ---- bf16 decoding -------------------------------------------------------------------

BF16_WORDS = [
    (0x3F80, 1.0),                 # sign 0, exponent 127, mantissa 0
    (0xC020, -2.5),                # sign 1, exponent 128, mantissa 0.25
    (0x4049, 3.140625),            # exponent 128, mantissa 0x49 / 128 = 0.5703125
    (0x0001, 2.0 ** -133),         # smallest bf16 subnormal: 2^-126 * 2^-7
    (0x0080, 2.0 ** -126),         # smallest normal
    (0x7F7F, (2 - 2 ** -7) * 2.0 ** 127),  # largest finite
    (0x8000, -0.0),
    (0x7F80, math.inf),
    (0xFF80, -math.inf),
]


@pytest.mark.parametrize("fn", [bf16_to_f64, bf16_to_f32])
def test_bf16_known_words(fn):
    got = fn(np.array([w for w, _ in BF16_WORDS], dtype=np.uint16))
    for (w, v), g in zip(BF16_WORDS, got.tolist()):
        assert g == v and math.copysign(1.0, g) == math.copysign(1.0, v), hex(w)
    assert math.isnan(float(fn(np.array([0x7FC0], np.uint16))[0]))


def _bf16_pins_fail(fn):
    try:
        test_bf16_known_words(fn)
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("broken", [
    lambda b: np.asarray(b, np.uint16).view(np.float16).astype(np.float64),            # read as fp16
    lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 15).view(np.float32).astype(np.float64),  # shift
    lambda b: (np.asarray(b, np.uint16).astype(np.uint32)).view(np.float32).astype(np.float64),  # low half
])
def test_bf16_pins_catch_plausible_slips(broken):
    with np.errstate(all="ignore"):
        assert _bf16_pins_fail(broken)


# ---- the exact merge (split invariance) ---------------------------------------------

@pytest.mark.parametrize("T", [1, 5])
def test_gpu_plus_cpu_partial_is_the_layer_output_for_every_split(T):
    wl = Workload("merge-pin", 11, Shape(1, 8, 64, 96, 3), T, 1.0)
    s = wl.shape
    recs = [expert_record(wl, 0, e) for e in range(s.E)]
    x = tokens(wl, 0, 0, T=T)
    wr = router_weights(wl, 0)
    seen_q = set()
    m_ref = None
    for forced in range(0, 3 * T + 2):
        cache = SlotTable(64, 1, s.E)  # cold: every routed expert misses, m = |U|
        # fq = 2^16 gives q = m; max_fetch then forces q = min(m, forced)
        r = decode_layer(cache, 0, x, wr, s.k, lambda e: recs[e], s.d, s.d_ff, Q16, min_fill=0,
                         max_fetch=forced)
        plan = r["plan"]
        m = len(plan.M)
        m_ref = m if m_ref is None else m_ref
        assert m == m_ref and plan.q == min(forced, m)
        seen_q.add(plan.q)
        y, yg, yc = r["y"], r["y_gpu"], r["y_cpu"]
        assert np.max(np.abs(yg + yc - y)) <= 1e-12 * np.max(np.abs(y))
        on_gpu = plan.pair_group >= 0
        assert on_gpu.sum() + (~on_gpu).sum() == T * s.k
        if plan.q == 0:
            assert np.all(yg == 0.0) and np.array_equal(yc, y)
        if plan.q == m:
            assert np.all(yc == 0.0) and np.array_equal(yg, y)
        for t in range(T):  # a token with no CPU pair has no CPU partial, and vice versa
            if on_gpu[t].all():
                assert np.all(yc[t] == 0.0)
            if not on_gpu[t].any():
                assert np.all(yg[t] == 0.0)
    assert seen_q == set(range(m_ref + 1))


# ---- plans and read counters on a hand-worked case ------------------------------------

@pytest.mark.parametrize("Sim", [SlotTable, OrderedLRU])
def test_plan_and_counters_hand_worked(Sim):
    # N = 3 slots, one layer of 6 experts, top-2, two tokens per call
    c = Sim(3, 1, 6)
    # call 1, cold, q = m: U = [3, 1, 4], all fill the empty slots 0, 1, 2 in order
    p = c.lookup(0, np.array([[3, 1], [1, 4]]), Q16, 1, -1)
    assert (p.U, p.H, p.M, p.q, p.F_slots) == ([3, 1, 4], [], [3, 1, 4], 3, [0, 1, 2])
    assert p.route_slot.tolist() == [[0, 1], [1, 2]] and p.pair_group.tolist() == [[0, 1], [1, 2]]
    k = c.counters
    assert (k.reads, k.read_hits, k.read_fills, k.read_cpu) == (4, 0, 4, 0)
    # call 2, no fetch: 1 and 3 hit, 5 runs on the host; G = H = [1, 3]
    p = c.lookup(0, np.array([[1, 5], [5, 3]]), 0, 0, -1)
    assert (p.U, p.H, p.M, p.q, p.C) == ([1, 5, 3], [1, 3], [5], 0, [5])
    assert p.route_slot.tolist() == [[1, -1], [-1, 0]] and p.pair_group.tolist() == [[0, -1], [-1, 1]]
    assert (k.reads, k.read_hits, k.read_fills, k.read_cpu) == (8, 2, 4, 2)
    assert (k.calls, k.unique_hits, k.unique_misses, k.fills, k.cpu_experts) == (2, 2, 4, 3, 1)
    # call 3: stamps are slot 2 (expert 4) < slot 1 (expert 1) < slot 0 (expert 3), so
    # the two fills evict 4 then 1
    p = c.lookup(0, np.array([[2, 0]]), Q16, 1, -1)
    assert (p.M, p.q, p.F_slots) == ([2, 0], 2, [2, 1])
    assert p.route_slot.tolist() == [[2, 1]] and p.pair_group.tolist() == [[0, 1]]
    assert (k.reads, k.read_hits, k.read_fills, k.read_cpu) == (10, 2, 6, 2)
    assert c.resident() == {2: 2, 0: 1, 3: 0}
