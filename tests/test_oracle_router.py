"""Pins of the oracle's router: fp32 logits against the exact dot product within
the rounding-error bound of the documented order, top-k against a brute-force
sort, gates against the softmax-then-renormalise form."""
import math

import numpy as np

from moe_expert_offload_amd.synth import f32_to_bf16_bits
from oracle.common import bf16_to_f64
from oracle.router import gates, route, router_logits, topk


def _bits(rng, shape, std):
    return f32_to_bf16_bits(rng.normal(0, std, size=shape))


def test_logits_within_error_bound_of_exact_dot():
    rng = np.random.default_rng(1)
    for d in (8, 256, 520, 2048, 4096):
        x = _bits(rng, (5, d), 1.0)
        w = _bits(rng, (7, d), 0.02)
        lg = router_logits(x, w).astype(np.float64)
        xe, we = bf16_to_f64(x), bf16_to_f64(w)
        exact = xe @ we.T   # every bf16 product is exact in fp64 and the fp64 sum error is tiny
        absdot = np.abs(xe) @ np.abs(we).T
        n_round = 8 * math.ceil(d / 512) + 6  # longest chain of fp32 roundings in the order
        u = 2.0 ** -24
        bound = n_round * u / (1 - n_round * u) * absdot + 1e-12 * absdot
        assert np.all(np.abs(lg - exact) <= bound), d


def test_dropped_term_is_detected_by_the_bound():
    # a plausible slip (skipping the last element of each 8-wide group) breaks the bound
    rng = np.random.default_rng(2)
    d = 512
    x = _bits(rng, (3, d), 1.0)
    w = _bits(rng, (4, d), 0.02)
    xe, we = bf16_to_f64(x), bf16_to_f64(w)
    x2 = x.copy()
    x2[:, 7::8] = 0
    slip = router_logits(x2, w).astype(np.float64)
    exact = xe @ we.T
    absdot = np.abs(xe) @ np.abs(we).T
    bound = 14 * 2.0 ** -24 * absdot * 1.01
    assert np.any(np.abs(slip - exact) > bound)


def test_order_scalar_reference_tiny():
    """Scalar float32 evaluation of the documented order on a tiny input."""
    rng = np.random.default_rng(3)
    d = 1040  # two full chunks and a partial third
    x = _bits(rng, (2, d), 1.0)
    w = _bits(rng, (3, d), 0.5)
    xf = bf16_to_f64(x).astype(np.float32)
    wf = bf16_to_f64(w).astype(np.float32)
    got = router_logits(x, w)
    for t in range(2):
        for e in range(3):
            lanes = []
            for lane in range(64):
                acc = np.float32(0.0)
                for j in range(3):
                    for r in range(8):
                        i = 512 * j + 8 * lane + r
                        p = np.float32(xf[t, i] * wf[e, i]) if i < d else np.float32(0.0)
                        acc = np.float32(acc + p)
                lanes.append(acc)
            for o in (32, 16, 8, 4, 2, 1):
                lanes = [np.float32(lanes[l] + lanes[l ^ o]) for l in range(64)]
            assert lanes[0].view(np.uint32) == got[t, e].view(np.uint32)


def test_topk_brute_force_and_ties():
    rng = np.random.default_rng(4)
    lg = rng.integers(-3, 4, size=(50, 16)).astype(np.float32)  # many ties
    idx = topk(lg, 5)
    for t in range(50):
        ref = sorted(range(16), key=lambda e: (-float(lg[t, e]), e))[:5]
        assert idx[t].tolist() == ref
    assert topk(np.zeros((1, 8), np.float32), 3)[0].tolist() == [0, 1, 2]
    g = gates(np.zeros((1, 8), np.float32), np.array([[0, 1, 2]]))
    assert np.allclose(g, 1.0 / 3.0, rtol=0, atol=1e-15)


def test_gates_equal_softmax_over_all_renormalised():
    rng = np.random.default_rng(5)
    lg = rng.normal(0, 2, size=(20, 32)).astype(np.float32)
    idx = topk(lg, 6)
    g = gates(lg, idx)
    full = np.exp(lg.astype(np.float64) - lg.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, idx.astype(np.int64), axis=1)
    assert np.allclose(g, sel / sel.sum(axis=1, keepdims=True), rtol=1e-12, atol=0)
    assert np.allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(g, axis=1) <= 1e-15)  # rank order = descending gates


def test_allowed_mask_restricts_choice():
    rng = np.random.default_rng(6)
    x = _bits(rng, (4, 256), 1.0)
    w = _bits(rng, (16, 256), 0.02)
    allowed = np.zeros((4, 16), np.uint8)
    for t in range(4):
        allowed[t, rng.choice(16, 3, replace=False)] = 1
    idx, g, lg = route(x, w, 3, allowed)
    for t in range(4):
        assert set(idx[t].tolist()) == set(np.flatnonzero(allowed[t]).tolist())
        assert [float(lg[t, e]) for e in idx[t]] == sorted([float(lg[t, e]) for e in idx[t]], reverse=True)
