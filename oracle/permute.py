"""Grouping of (token, rank) pairs by expert before the grouped expert FFN.

Test infrastructure (see the package docstring).

The pages do not describe this step (the grouped evaluation of the GPU set
needs the pairs of each expert together).  This build defines it as a stable
counting sort of the flattened pair ids p = t*k + j by their group key, pairs
with key -1 being left out:

  counts[g]  = #{p : key[p] = g}
  offsets    = exclusive prefix sum of counts (length n_groups + 1)
  perm       = pair ids ordered by (key, p)
  inv[p]     = position of p in perm, or -1 for a left-out pair
"""
import numpy as np


def group_pairs(key, n_groups):
    key = np.asarray(key).reshape(-1)
    counts = [0] * n_groups
    for g in key.tolist():
        if g >= 0:
            counts[g] += 1
    offsets = [0] * (n_groups + 1)
    for g in range(n_groups):
        offsets[g + 1] = offsets[g] + counts[g]
    cursor = offsets[:-1].copy()
    perm = [0] * offsets[-1]
    inv = [-1] * key.size
    for p, g in enumerate(key.tolist()):
        if g < 0:
            continue
        perm[cursor[g]] = p
        inv[p] = cursor[g]
        cursor[g] += 1
    return (np.asarray(offsets, np.int32), np.asarray(perm, np.int32), np.asarray(inv, np.int32))
