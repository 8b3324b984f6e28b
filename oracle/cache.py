"""GPU expert-cache residency: classify, split, LRU update, slot rewrite, prefill, resize.

Test infrastructure (see the package docstring).  Two simulators, written
apart (each its own dedup, victim order, plan and counters; both take q from
the pinned split rule of oracle.qstar), so each can be checked against the
other.

Pages:
  [FT] §3 one elastic cache shared by all MoE layers, keyed on logical
       (layer, expert); a slot holds every tensor of one pair.
  [FT] §3.2 hits H run on the GPU; the m unique misses split into F (filled,
       stay resident) and C (run on the CPU, residency unchanged); a hit
       refreshes recency, a fill admits, eviction removes the least recently
       demanded entry.
  [FT] §4.1 "Device-side cache control": per layer, dedup the routed experts,
       classify against the residency table, derive q, pick victims (the K least
       recently used, of which the first q are consumed), rewrite routed ids to
       slot ids or a CPU flag.  [AIN] "Decode residency": the CPU flag is -1.
  [FT] §3.1 two full-layer prefill buffers come out of the same slot pool and
       entries that survive prefill seed decode.
  [FT] §3.3 the cache can be rebuilt for a new budget at a safe point;
       [AIN] "How to run it in production": a rebuild resets hit/miss counters.

Readings of this build (the pages leave these open):
  * "unique" is per (step, layer); U lists distinct routed experts in first
    occurrence order over (t, j) flattened t-major; H and M keep U order.
  * eligible victims are the slots not holding a hit of this call, ordered by
    (recency stamp before the call, slot index), empty slots (stamp -1) first;
    avail = N - |H|; F = M[:q] takes victims in that order; C = M[q:].
  * one access clock: each expert of H and F is touched once, in U order.
  * the cache starts cold; a resize empties it (cold rebuild), resets the
    counters and keeps the clock.
  * prefill: at begin, the first 2E slots in victim order (no hits to protect)
    become buffers B0 = first E, B1 = next E and lose their keys; layer l uses
    B[l % 2] with expert e in B[l % 2][e].  Layer 0 loads at begin and layer l+1
    streams into the other buffer while layer l computes ([FT] §3.1), so after
    n of the L layers the buffers hold layers n-1 and n (n < L), or L-2 and L-1
    after the whole pass.  At end the layers the buffers hold are registered
    (ascending layer, e ascending), each touching the clock; a copy of the same
    key elsewhere is emptied; buffer slots left unregistered become empty.
  * on-demand prefill ([FT] §3.1: the fallback when the pool cannot spare two
    full layers, and the serial loading left when the second buffer is off):
    per layer, after routing, U (first occurrence over the chunk's (t, j)) splits
    into resident H and missing M; M is loaded in rounds of at most avail =
    (slots not holding a hit) experts, each round taking victims like a decode
    fill (victim order before the round, M order) and computing its experts
    once their loads land; round 0 also computes H.  Touches: round 0 touches
    H and its batch in U order, each later round its batch in order.  Hit slots
    are never victims within the layer; a round may evict what an earlier round
    of the same layer loaded (after that round computed).  No slot at all for a
    miss is an error.  Decode counters are untouched.
"""
from __future__ import annotations

import heapq
from collections import OrderedDict
from dataclasses import dataclass, field

import numpy as np

from .qstar import q_split

EMPTY = -1
RESERVED = -2


@dataclass
class Plan:
    layer: int
    U: list
    H: list
    M: list
    q: int
    F: list
    C: list
    F_slots: list
    avail: int
    route_slot: np.ndarray  # int32 [T, k]: slot of the pair's expert, -1 for C
    G: list = field(default_factory=list)        # GPU experts: H then F
    G_slots: list = field(default_factory=list)
    pair_group: np.ndarray = None  # int32 [T, k]: index into G, -1 for C

    @property
    def m(self):
        return len(self.M)


@dataclass
class Counters:
    calls: int = 0
    unique_hits: int = 0
    unique_misses: int = 0
    fills: int = 0
    cpu_experts: int = 0
    reads: int = 0
    read_hits: int = 0
    read_fills: int = 0
    read_cpu: int = 0


def _first_occurrence(idx):  # simulator A
    seen, out = set(), []
    for e in np.asarray(idx).reshape(-1).tolist():
        if e not in seen:
            seen.add(e)
            out.append(e)
    return out


def _finish_plan(layer, idx, U, H, M, q, F_slots, avail, slot_of, counters):  # simulator A
    idx = np.asarray(idx)
    F = M[:q]
    C = M[q:]
    G = H + F
    G_slots = [slot_of(e) for e in G]
    gpos = {e: i for i, e in enumerate(G)}
    route = np.full(idx.shape, -1, np.int32)
    group = np.full(idx.shape, -1, np.int32)
    Hs, Fs = set(H), set(F)
    for t in range(idx.shape[0]):
        for j in range(idx.shape[1]):
            e = int(idx[t, j])
            if e in gpos:
                route[t, j] = G_slots[gpos[e]]
                group[t, j] = gpos[e]
            counters.reads += 1
            if e in Hs:
                counters.read_hits += 1
            elif e in Fs:
                counters.read_fills += 1
            else:
                counters.read_cpu += 1
    counters.calls += 1
    counters.unique_hits += len(H)
    counters.unique_misses += len(M)
    counters.fills += len(F)
    counters.cpu_experts += len(C)
    return Plan(layer, U, H, M, q, F, C, list(F_slots), avail, route, G, G_slots, group)


class SlotTable:
    """Simulator A: explicit per-slot key and stamp arrays plus a key->slot table."""

    def __init__(self, N, L, E):
        self.L, self.E = L, E
        self.clock = 0
        self._reset(N)

    def _reset(self, N):
        self.N = N
        self.slot_key = [EMPTY] * N
        self.slot_stamp = [-1] * N
        self.where = {}
        self.counters = Counters()
        self.buffers = None

    def key(self, layer, e):
        return layer * self.E + e

    def _victim_order(self, protected):
        cand = [s for s in range(self.N) if s not in protected and self.slot_key[s] != RESERVED]
        return sorted(cand, key=lambda s: (self.slot_stamp[s], s))

    def lookup(self, layer, idx, fq, min_fill=1, max_fetch=-1):
        U = _first_occurrence(idx)
        H = [e for e in U if self.key(layer, e) in self.where]
        M = [e for e in U if self.key(layer, e) not in self.where]
        hit_slots = {self.where[self.key(layer, e)] for e in H}
        V = self._victim_order(hit_slots)
        avail = len(V)
        q = q_split(len(M), fq, min_fill, max_fetch, avail)
        F_slots = []
        for i in range(q):
            s = V[i]
            old = self.slot_key[s]
            if old >= 0:
                del self.where[old]
            kk = self.key(layer, M[i])
            self.slot_key[s] = kk
            self.where[kk] = s
            F_slots.append(s)
        gpu = set(H) | set(M[:q])
        for e in U:
            if e in gpu:
                self.clock += 1
                self.slot_stamp[self.where[self.key(layer, e)]] = self.clock
        return _finish_plan(layer, idx, U, H, M, q, F_slots, avail,
                            lambda e: self.where[self.key(layer, e)], self.counters)

    def prefill_begin(self):
        E = self.E
        if self.N < 2 * E:
            raise ValueError("prefill double buffering needs N >= 2E")
        V = self._victim_order(set())
        b0, b1 = V[:E], V[E:2 * E]
        for s in b0 + b1:
            old = self.slot_key[s]
            if old >= 0:
                del self.where[old]
            self.slot_key[s] = RESERVED
            self.slot_stamp[s] = -1
        self.buffers = (b0, b1)
        return [list(b0), list(b1)]

    def prefill_slot(self, layer, e):
        return self.buffers[layer % 2][e]

    def prefill_end(self, n_done):
        """End a double-buffered prefill after n_done of the L layers were computed
        (n_done = L for a whole pass)."""
        used = set()
        if n_done < self.L:
            held = [n_done - 1, n_done]
        else:
            held = [self.L - 2, self.L - 1]
        for layer in held:
            if layer < 0:
                continue
            buf = self.buffers[layer % 2]
            for e in range(self.E):
                s = buf[e]
                kk = self.key(layer, e)
                if kk in self.where:
                    s_old = self.where[kk]
                    self.slot_key[s_old] = EMPTY
                    self.slot_stamp[s_old] = -1
                self.slot_key[s] = kk
                self.where[kk] = s
                self.clock += 1
                self.slot_stamp[s] = self.clock
                used.add(s)
        for buf in self.buffers:
            for s in buf:
                if s not in used:
                    self.slot_key[s] = EMPTY
                    self.slot_stamp[s] = -1
        self.buffers = None

    def prefill_on_demand(self, layer, idx):
        """Rounds of one on-demand prefill layer: a list of {"fill": [(e, slot)],
        "compute": [(e, slot)]}; returns (U, H, M, rounds)."""
        U = _first_occurrence(idx)
        H = [e for e in U if self.key(layer, e) in self.where]
        M = [e for e in U if self.key(layer, e) not in self.where]
        hit_slots = {self.where[self.key(layer, e)] for e in H}
        rounds, done, r = [], 0, 0
        while r == 0 or done < len(M):
            V = self._victim_order(hit_slots)
            n = min(len(V), len(M) - done)
            if n == 0 and done < len(M):
                raise ValueError("on-demand prefill: no slot to load a miss into")
            batch = M[done:done + n]
            fills = []
            for i, e in enumerate(batch):
                s = V[i]
                old = self.slot_key[s]
                if old >= 0:
                    del self.where[old]
                kk = self.key(layer, e)
                self.slot_key[s] = kk
                self.where[kk] = s
                fills.append((e, s))
            touched = [e for e in U if e in set(H) | set(batch)] if r == 0 else batch
            for e in touched:
                self.clock += 1
                self.slot_stamp[self.where[self.key(layer, e)]] = self.clock
            hits = [(e, self.where[self.key(layer, e)]) for e in H] if r == 0 else []
            rounds.append({"fill": fills, "compute": hits + fills})
            done += n
            r += 1
        return U, H, M, rounds

    def resize(self, N_new):
        self._reset(N_new)

    def resident(self):
        return {k: s for k, s in self.where.items()}


class OrderedLRU:
    """Simulator B: an ordered map key->slot (least recent first) plus a min-heap of free slots."""

    def __init__(self, N, L, E):
        self.L, self.E = L, E
        self.N = N
        self.od = OrderedDict()
        self.free = list(range(N))
        heapq.heapify(self.free)
        self.counters = Counters()
        self.buffers = None

    def lookup(self, layer, idx, fq, min_fill=1, max_fetch=-1):
        idx = np.asarray(idx)
        U = list(dict.fromkeys(int(e) for e in idx.reshape(-1)))  # insertion order = first occurrence
        tag = lambda e: (layer, e)
        H = [e for e in U if tag(e) in self.od]
        M = [e for e in U if tag(e) not in self.od]
        avail = self.N - len(H)
        q = q_split(len(M), fq, min_fill, max_fetch, avail)
        hit_tags = {tag(e) for e in H}
        victims = []  # (slot, evicted tag or None)
        free_taken = []
        while len(victims) < q and self.free:
            s = heapq.heappop(self.free)
            free_taken.append(s)
            victims.append((s, None))
        if len(victims) < q:
            for t_old, s in self.od.items():  # least recent first, state before this call
                if t_old in hit_tags:
                    continue
                victims.append((s, t_old))
                if len(victims) == q:
                    break
        F_slots = []
        for i, (s, t_old) in enumerate(victims):
            if t_old is not None:
                del self.od[t_old]
            self.od[tag(M[i])] = s
            F_slots.append(s)
        gpu = set(H) | set(M[:q])
        for e in U:
            if e in gpu:
                self.od.move_to_end(tag(e))
        return self._plan(layer, idx, U, H, M, q, F_slots, avail)

    def _plan(self, layer, idx, U, H, M, q, F_slots, avail):
        """The plan and the counters of one call, from the ordered map (written apart
        from simulator A's: slots looked up in the map, read counts by set membership
        over the whole id array)."""
        F, C = M[:q], M[q:]
        G = H + F
        G_slots = [self.od[(layer, e)] for e in G]
        flat = idx.reshape(-1)
        route = np.array([self.od[(layer, int(e))] if int(e) in G else -1 for e in flat], np.int32)
        group = np.array([G.index(int(e)) if int(e) in G else -1 for e in flat], np.int32)
        c = self.counters
        c.calls += 1
        c.unique_hits += len(H)
        c.unique_misses += len(M)
        c.fills += len(F)
        c.cpu_experts += len(C)
        c.reads += flat.size
        c.read_hits += int(np.isin(flat, np.array(H, dtype=flat.dtype)).sum())
        c.read_fills += int(np.isin(flat, np.array(F, dtype=flat.dtype)).sum())
        c.read_cpu += int(np.isin(flat, np.array(C, dtype=flat.dtype)).sum())
        return Plan(layer, U, H, M, q, F, C, list(F_slots), avail, route.reshape(idx.shape), G, G_slots,
                    group.reshape(idx.shape))

    def _all_in_victim_order(self):
        return sorted(self.free) + list(self.od.values())

    def prefill_begin(self):
        E = self.E
        if self.N < 2 * E:
            raise ValueError("prefill double buffering needs N >= 2E")
        order = self._all_in_victim_order()[:2 * E]
        taken = set(order)
        self.free = [s for s in self.free if s not in taken]
        heapq.heapify(self.free)
        for t_old in [t for t, s in self.od.items() if s in taken]:
            del self.od[t_old]
        self.buffers = (order[:E], order[E:2 * E])
        return [list(self.buffers[0]), list(self.buffers[1])]

    def prefill_slot(self, layer, e):
        return self.buffers[layer % 2][e]

    def prefill_end(self, n_done):
        # the buffers hold the last layer computed and the one streamed in during its
        # compute; after the whole pass, the last two layers
        last = min(n_done, self.L - 1)
        used = set()
        for layer in (last - 1, last):
            if layer < 0:
                continue
            buf = self.buffers[layer % 2]
            for e in range(self.E):
                if (layer, e) in self.od:
                    heapq.heappush(self.free, self.od.pop((layer, e)))
                self.od[(layer, e)] = buf[e]
                used.add(buf[e])
        for buf in self.buffers:
            for s in buf:
                if s not in used:
                    heapq.heappush(self.free, s)
        self.buffers = None

    def prefill_on_demand(self, layer, idx):
        U = list(dict.fromkeys(int(e) for e in np.asarray(idx).reshape(-1)))
        tag = lambda e: (layer, e)
        H = [e for e in U if tag(e) in self.od]
        M = [e for e in U if tag(e) not in self.od]
        hit_tags = {tag(e) for e in H}
        rounds, done, r = [], 0, 0
        while r == 0 or done < len(M):
            want = len(M) - done
            victims = []  # (slot, evicted tag or None), in victim order before this round
            while len(victims) < want and self.free:
                victims.append((heapq.heappop(self.free), None))
            if len(victims) < want:
                for t_old, s in self.od.items():  # least recent first
                    if t_old in hit_tags:
                        continue
                    victims.append((s, t_old))
                    if len(victims) == want:
                        break
            if not victims and want > 0:
                raise ValueError("on-demand prefill: no slot to load a miss into")
            batch = M[done:done + len(victims)]
            fills = []
            for e, (s, t_old) in zip(batch, victims):
                if t_old is not None:
                    del self.od[t_old]
                self.od[tag(e)] = s
                fills.append((e, s))
            in_round = set(H) | set(batch) if r == 0 else set(batch)
            for e in (U if r == 0 else batch):
                if e in in_round:
                    self.od.move_to_end(tag(e))
            hits = [(e, self.od[tag(e)]) for e in H] if r == 0 else []
            rounds.append({"fill": fills, "compute": hits + fills})
            done += len(batch)
            r += 1
        return U, H, M, rounds

    def resize(self, N_new):
        self.N = N_new
        self.od = OrderedDict()
        self.free = list(range(N_new))
        heapq.heapify(self.free)
        self.counters = Counters()

    def resident(self):
        return {layer * self.E + e: s for (layer, e), s in self.od.items()}
