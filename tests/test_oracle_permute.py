"""Pins of the oracle's pair grouping against library routines (stable argsort, bincount)."""
import numpy as np

from oracle.permute import group_pairs


def test_group_pairs_against_stable_argsort():
    rng = np.random.default_rng(20)
    for P, G in [(0, 4), (1, 1), (64, 8), (1000, 37), (49152 // 16, 256)]:
        key = rng.integers(-1, G, size=P).astype(np.int32)
        off, perm, inv = group_pairs(key, G)
        inc = np.flatnonzero(key >= 0)
        ref_perm = inc[np.argsort(key[inc], kind="stable")]
        assert np.array_equal(perm, ref_perm)
        counts = np.bincount(key[inc], minlength=G)
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(counts)]))
        ref_inv = np.full(P, -1)
        ref_inv[ref_perm] = np.arange(ref_perm.size)
        assert np.array_equal(inv, ref_inv)
