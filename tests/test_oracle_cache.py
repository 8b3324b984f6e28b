"""Pins of the oracle's residency simulators: the two independent simulators
agree on every decision; textbook LRU (stack distance) for one expert per call;
compulsory-miss, zero-capacity and no-fetch special cases; invariants; prefill
residency; the batch-dedup closed form."""
import json
import os

import numpy as np
import pytest

from moe_expert_offload_amd.synth import zipf_reuse_trace
from oracle.cache import OrderedLRU, SlotTable
from oracle.qstar import Q16

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "qstar_pages.json")))


def _same_plan(a, b):
    assert a.U == b.U and a.H == b.H and a.M == b.M
    assert a.q == b.q and a.F == b.F and a.C == b.C
    assert a.F_slots == b.F_slots and a.avail == b.avail
    assert np.array_equal(a.route_slot, b.route_slot)
    assert a.G == b.G and a.G_slots == b.G_slots
    assert np.array_equal(a.pair_group, b.pair_group)


def _check_invariants(sim_a, N):
    keys = [k for k in sim_a.slot_key if k >= 0]
    assert len(keys) == len(set(keys)) <= N
    for kk, s in sim_a.where.items():
        assert sim_a.slot_key[s] == kk


@pytest.mark.parametrize("N,fq,min_fill,max_fetch,B", [
    (40, 30000, 1, -1, 1), (40, 30000, 0, -1, 4), (13, Q16, 1, -1, 2), (200, 8000, 1, 2, 3),
    (7, 50000, 1, -1, 8), (0, 30000, 1, -1, 2), (64, 0, 0, -1, 2), (500, Q16, 1, -1, 2)])
def test_two_simulators_agree(N, fq, min_fill, max_fetch, B):
    L, E, k, steps = 5, 32, 4, 60
    rng = np.random.default_rng(N * 7 + B)
    tr = zipf_reuse_trace(L, E, k, B, steps, 1.1, 0.6, rng)
    a, b = SlotTable(N, L, E), OrderedLRU(N, L, E)
    for s in range(steps):
        for layer in range(L):
            idx = tr[s, layer]
            # random rank order inside each token row, as the router would give
            idx = np.stack([rng.permutation(r) for r in idx])
            pa = a.lookup(layer, idx, fq, min_fill, max_fetch)
            pb = b.lookup(layer, idx, fq, min_fill, max_fetch)
            _same_plan(pa, pb)
            _check_invariants(a, N)
            for t in range(idx.shape[0]):
                for j in range(k):
                    e = int(idx[t, j])
                    if e in pa.C:
                        assert pa.route_slot[t, j] == -1
                    else:
                        assert a.slot_key[pa.route_slot[t, j]] == layer * E + e
    assert a.resident() == b.resident()
    assert a.counters == b.counters


def test_resize_and_prefill_sequences_agree():
    L, E, k = 6, 16, 3
    rng = np.random.default_rng(5)
    tr = zipf_reuse_trace(L, E, k, 2, 40, 1.1, 0.6, rng)
    a, b = SlotTable(40, L, E), OrderedLRU(40, L, E)
    for s in range(40):
        if s == 15:
            ba, bb = a.prefill_begin(), b.prefill_begin()
            assert ba == bb
            a.prefill_end(L), b.prefill_end(L)
            assert a.resident() == b.resident()
            res = a.resident()
            assert sorted(res) == sorted(set(res))
            for layer in (L - 2, L - 1):
                for e in range(E):
                    assert layer * E + e in res
        if s == 25:
            a.resize(33), b.resize(33)
            assert a.counters.calls == 0 and a.resident() == {}
        for layer in range(L):
            _same_plan(a.lookup(layer, tr[s, layer], 40000), b.lookup(layer, tr[s, layer], 40000))
    assert a.resident() == b.resident() and a.counters == b.counters


def test_textbook_lru_stack_distance():
    """One routed expert per call and q = m: a call misses iff fewer than N distinct
    other keys separate it from the previous access of the same key (Mattson)."""
    rng = np.random.default_rng(7)
    L, E, N = 3, 10, 6
    seq = [(int(rng.integers(L)), int(rng.integers(E))) for _ in range(3000)]
    sim = SlotTable(N, L, E)
    for i, (layer, e) in enumerate(seq):
        plan = sim.lookup(layer, np.array([[e]]), Q16, 1, -1)
        prev = max((j for j in range(i) if seq[j] == (layer, e)), default=None)
        if prev is None:
            expect_miss = True
        else:
            expect_miss = len(set(seq[prev + 1:i])) >= N
        assert (plan.m == 1) == expect_miss, i


def test_special_cases():
    L, E, k = 4, 16, 4
    rng = np.random.default_rng(8)
    tr = zipf_reuse_trace(L, E, k, 2, 50, 1.1, 0.6, rng)
    # capacity >= all pairs: only compulsory misses
    big = SlotTable(L * E, L, E)
    for s in range(50):
        for layer in range(L):
            big.lookup(layer, tr[s, layer], Q16)
    distinct = {(layer, int(e)) for layer in range(L) for e in np.unique(tr[:, layer])}
    assert big.counters.unique_misses == len(distinct)
    # zero capacity: every routed expert runs on the CPU
    z = SlotTable(0, L, E)
    for s in range(10):
        p = z.lookup(0, tr[s, 0], Q16)
        assert p.q == 0 and p.H == [] and np.all(p.route_slot == -1)
    # never fetch: residency never changes
    nf = SlotTable(20, L, E)
    for s in range(10):
        p = nf.lookup(1, tr[s, 1], 0, min_fill=0)
        assert p.q == 0 and nf.resident() == {}
    # a hit is never evicted by a fill of the same call
    h = SlotTable(3, 1, 8)
    h.lookup(0, np.array([[0, 1, 2]]), Q16)
    p = h.lookup(0, np.array([[0, 5, 6]]), Q16)
    assert p.H == [0] and p.avail == 2 and p.q == 2
    assert h.resident()[0] == 0


def test_dedup_closed_form_uniform():
    g = GOLD["dedup"]
    E, k, B = g["E"], g["k"], g["B"]
    rng = np.random.default_rng(9)
    trials = 4000
    u = []
    for _ in range(trials):
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(B)])
        u.append(len(SlotTable(0, 1, E).lookup(0, idx, 0, 0).U))
    mean = float(np.mean(u))
    closed = E * (1 - (1 - k / E) ** B)
    se = float(np.std(u)) / np.sqrt(trials)
    assert abs(mean - closed) < 4 * se + 1e-9
    # the page prints its own Monte Carlo estimate of the gain to 3 decimals
    assert abs(B * k / closed - g["gain_uniform"]) < 2e-3
    assert abs(B * k / mean - g["gain_uniform"]) < 4e-3


# ---- on-demand prefill ------------------------------------------------------------

def _prefill_idx(rng, T, E, k):
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])


@pytest.mark.parametrize("N,T", [(5, 16), (20, 40), (31, 64), (64, 8), (100, 200), (1, 6), (33, 300)])
def test_on_demand_prefill_simulators_agree(N, T):
    """The two independent simulators give the same rounds and residency over decode
    steps interleaved with on-demand prefill layers, at pools smaller and larger than
    one layer's expert set."""
    L, E, k = 4, 32, 4
    rng = np.random.default_rng(N * 31 + T)
    a, b = SlotTable(N, L, E), OrderedLRU(N, L, E)
    tr = zipf_reuse_trace(L, E, k, 1, 6, 1.1, 0.6, rng)
    for s in range(6):
        for layer in range(L):
            _same_plan(a.lookup(layer, tr[s, layer], 30000), b.lookup(layer, tr[s, layer], 30000))
        for layer in range(L):
            idx = _prefill_idx(rng, T, E, k)
            ra, rb = a.prefill_on_demand(layer, idx), b.prefill_on_demand(layer, idx)
            assert ra == rb
            _check_invariants(a, N)
            U, H, M, rounds = ra
            # every routed expert is computed exactly once; hits are never evicted in the layer
            computed = [e for rd in rounds for e, _ in rd["compute"]]
            assert sorted(computed) == sorted(U) and len(computed) == len(set(computed))
            hit_slots = {sl for e, sl in rounds[0]["compute"] if e in H}
            avail = N - len(H)
            for i, rd in enumerate(rounds):
                slots = [sl for _, sl in rd["fill"]]
                assert len(slots) == len(set(slots)) and not (set(slots) & hit_slots)
                assert len(rd["fill"]) == (avail if i < len(rounds) - 1 else len(M) - avail * (len(rounds) - 1))
            assert len(rounds) == max(1, -(-len(M) // avail)) if M else len(rounds) == 1
    assert a.resident() == b.resident()


def test_on_demand_prefill_special_cases():
    L, E, k = 2, 16, 2
    idx = np.array([[3, 1], [1, 7], [9, 3], [0, 7]])  # U = 3, 1, 7, 9, 0
    # cold cache with room: one round, misses into the empty slots in ascending order, U order
    a = SlotTable(40, L, E)
    U, H, M, rounds = a.prefill_on_demand(0, idx)
    assert U == [3, 1, 7, 9, 0] and H == [] and M == U
    assert rounds == [{"fill": [(3, 0), (1, 1), (7, 2), (9, 3), (0, 4)],
                       "compute": [(3, 0), (1, 1), (7, 2), (9, 3), (0, 4)]}]
    assert [a.slot_stamp[s] for s in range(5)] == [1, 2, 3, 4, 5]
    # the same layer again: all hits, one round, nothing loaded, touched in U order
    U, H, M, rounds = a.prefill_on_demand(0, idx)
    assert H == U and rounds == [{"fill": [], "compute": [(3, 0), (1, 1), (7, 2), (9, 3), (0, 4)]}]
    assert [a.slot_stamp[s] for s in range(5)] == [6, 7, 8, 9, 10]
    # a single slot: one expert per round, each evicting the previous; the last stays
    b = SlotTable(1, L, E)
    U, H, M, rounds = b.prefill_on_demand(1, idx)
    assert [rd["fill"] for rd in rounds] == [[(3, 0)], [(1, 0)], [(7, 0)], [(9, 0)], [(0, 0)]]
    assert b.resident() == {1 * E + 0: 0}
    # two slots, one of them a hit of this layer: the misses cycle through the other
    c = SlotTable(2, L, E)
    c.prefill_on_demand(0, np.array([[5, 6]]))     # 5 -> slot 0, 6 -> slot 1
    U, H, M, rounds = c.prefill_on_demand(0, np.array([[6, 2], [4, 6]]))
    assert H == [6] and M == [2, 4]
    assert rounds[0] == {"fill": [(2, 0)], "compute": [(6, 1), (2, 0)]}
    assert rounds[1] == {"fill": [(4, 0)], "compute": [(4, 0)]}
    # no slot for a miss: 4 holds the only slot and is a hit, 5 has nowhere to go
    for sim in (SlotTable(1, L, E), OrderedLRU(1, L, E)):
        sim.prefill_on_demand(0, np.array([[4, 4]]))
        with pytest.raises(ValueError):
            sim.prefill_on_demand(0, np.array([[4, 5]]))


@pytest.mark.parametrize("n_done", [0, 1, 2, 3, 5, 6])
def test_prefill_ended_early_keeps_what_the_buffers_hold(n_done):
    """[FT] §3.1: layer l+1 streams into the other buffer while layer l computes, so
    after n_done < L layers the buffers hold layers n_done-1 and n_done (never
    n_done-2, whose buffer the prefetch of n_done overwrote); after the whole pass
    L-2 and L-1.  Both simulators, and the slots are exactly the buffer slots."""
    L, E = 6, 4
    a, b = SlotTable(20, L, E), OrderedLRU(20, L, E)
    bufs = a.prefill_begin()
    assert b.prefill_begin() == bufs
    a.prefill_end(n_done), b.prefill_end(n_done)
    held = [n_done - 1, n_done] if n_done < L else [L - 2, L - 1]
    want = {l * E + e: bufs[l % 2][e] for l in held if l >= 0 for e in range(E)}
    assert a.resident() == want and b.resident() == want
