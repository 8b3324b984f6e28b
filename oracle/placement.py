"""Expert-placement replay: decode-time miss rate of a routing trace under three
placement policies at one cache capacity.

Test infrastructure (see the package docstring).

Pages:
  [FT] §5.3 "Expert locality" and Fig. 4b: identical routing traces are replayed
       against three placement policies at equal cache capacity, and the share of
       decode-time expert reads that miss the GPU is reported per capacity:
         * FreeToken's global LRU, updated on every miss;
         * a placement chosen from what each prefill routed, held through decode
           (the KTransformers policy, as the pages describe it in one line);
         * a routing-blind static split of the pool (the llama.cpp policy, as
           the pages describe it in one line).
  [FT] §3.1 prefill streams every layer through two full-layer buffers whose
       survivors seed decode (the LRU engine's prefill, `cache.SlotTable`).

Readings of this build (the pages give one sentence per policy):
  * A trace is R requests served one after another at batch 1: `prompt` prefill
    tokens, then `decode` decode steps; ids[r, s, l, :] are the k experts token
    s of request r routes to in layer l.  Only decode reads are counted: k per
    (step, layer).
  * LRU: the engine's own residency rule (`cache.SlotTable`) with every miss
    filled (q = m, the per-miss LRU of the pages).  Each request's prefill is the
    engine's: two full-layer buffers when N >= 2E (begin, then the last two
    layers registered at the end), else on-demand loading of each layer's routed
    experts.  The cache persists across requests.
  * Hot set: after each prefill the resident set becomes the N (layer, expert)
    pairs routed most often by that prefill's tokens, ties to the lower l*E + e
    (pairs never routed fill the rest in that order); it does not change during
    decode.
  * Static split: the GPU holds the last N pairs in l*E + e order (whole layers
    from the top, as when the experts of the first layers are kept on the CPU),
    whatever the routing.
"""
from __future__ import annotations

import numpy as np

from .cache import OrderedLRU, SlotTable
from .qstar import Q16


def _check(ids, L, E):
    ids = np.asarray(ids)
    if ids.ndim != 4 or ids.shape[2] != L:
        raise ValueError("ids must be [requests, steps, L, k]")
    if ids.size and (ids.min() < 0 or ids.max() >= E):
        raise ValueError("expert id out of range")
    return ids


def replay_lru(ids, L, E, N, prompt, sim=SlotTable):
    """(decode reads, decode misses) under the engine's global LRU."""
    ids = _check(ids, L, E)
    k = ids.shape[3]
    cache = sim(N, L, E)
    reads = misses = 0
    for r in range(ids.shape[0]):
        if prompt > 0:
            if N >= 2 * E:
                cache.prefill_begin()
                cache.prefill_end(L)
            else:
                for layer in range(L):
                    cache.prefill_on_demand(layer, ids[r, :prompt, layer, :])
        for s in range(prompt, ids.shape[1]):
            for layer in range(L):
                plan = cache.lookup(layer, ids[r, s:s + 1, layer, :], Q16)
                reads += k
                misses += len(plan.M)
    return reads, misses


def hot_set(prompt_ids, L, E, N):
    """The N pairs (l*E + e) a prefill routed most often, ties to the lower index."""
    counts = {}
    for s in range(prompt_ids.shape[0]):
        for layer in range(L):
            for e in prompt_ids[s, layer]:
                key = layer * E + int(e)
                counts[key] = counts.get(key, 0) + 1
    order = sorted(range(L * E), key=lambda key: (-counts.get(key, 0), key))
    return set(order[:max(0, min(N, L * E))])


def replay_hotset(ids, L, E, N, prompt):
    """(decode reads, decode misses) with the resident set chosen at each prefill."""
    ids = _check(ids, L, E)
    k = ids.shape[3]
    reads = misses = 0
    for r in range(ids.shape[0]):
        resident = hot_set(ids[r, :prompt], L, E, N)
        for s in range(prompt, ids.shape[1]):
            for layer in range(L):
                for e in ids[r, s, layer]:
                    reads += 1
                    misses += (layer * E + int(e)) not in resident
    assert reads == ids.shape[0] * (ids.shape[1] - prompt) * L * k
    return reads, misses


def replay_static(ids, L, E, N, prompt):
    """(decode reads, decode misses) with the last N pairs resident."""
    ids = _check(ids, L, E)
    first = L * E - max(0, min(N, L * E))
    reads = misses = 0
    for r in range(ids.shape[0]):
        for s in range(prompt, ids.shape[1]):
            for layer in range(L):
                for e in ids[r, s, layer]:
                    reads += 1
                    misses += (layer * E + int(e)) < first
    return reads, misses


POLICIES = {"lru": replay_lru, "hotset": replay_hotset, "static": replay_static}


def replay(policy, ids, L, E, N, prompt):
    return POLICIES[policy](ids, L, E, N, prompt)


def replay_lru_ordered(ids, L, E, N, prompt):
    """The LRU replay on the second, independently written simulator."""
    return replay_lru(ids, L, E, N, prompt, sim=OrderedLRU)
