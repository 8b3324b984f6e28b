"""Router of one MoE layer: logits, top-k experts per token, renormalised gates.

Test infrastructure (see the package docstring).

[FT] §3.2 (decode: "the router and cache lookup run on the GPU", each token
goes to k experts) and [AIN] "Architecture" (the router picks the top-k for
each token).  The pages do not fix the gate function, the tie rule or the
precision; this build reads them as: softmax gating, top-k renormalised, ties
to the lower expert index.

Logit summation order (a definition of this build, since routing must be
bit-exact and the pages are silent): logits are fp32.  A 64-lane accumulator
array is used; element i of the dot product belongs to lane (i mod 512) // 8,
and lane l adds its products in increasing i, i.e. chunk j = 0, 1, ... and
inside a chunk r = 0..7 for i = 512 j + 8 l + r.  Positions past d are padded
with zeros (adding +0.0 products).  The 64 partial sums are then combined by
the butterfly a_l <- a_l + a_(l xor o) for o = 32, 16, 8, 4, 2, 1 and the result
is a_0.  A product of two bf16 values is exact in fp32, so a fused or unfused
multiply-add gives the same bits.
"""
import numpy as np

from .common import bf16_to_f32
from .ffn import _map

LANES = 64
VEC = 8
CHUNK = LANES * VEC  # 512


def router_logits(x_bits, w_bits, workers=1) -> np.ndarray:
    """fp32 logits [T, E] of x [T, d] against W_r [E, d] (bf16 words), in the order above
    (``workers`` > 1: blocks of tokens on that many threads, arithmetic unchanged)."""
    x = bf16_to_f32(x_bits)
    w = bf16_to_f32(w_bits)
    T, d = x.shape
    E = w.shape[0]
    J = (d + CHUNK - 1) // CHUNK
    xp = np.zeros((T, J * CHUNK), np.float32)
    wp = np.zeros((E, J * CHUNK), np.float32)
    xp[:, :d] = x
    wp[:, :d] = w
    xp = xp.reshape(T, J, LANES, VEC)
    wp = wp.reshape(E, J, LANES, VEC)
    out = np.empty((T, E), np.float32)
    tb = max(1, 4096 // max(E, 1))
    lanes = np.arange(LANES)

    def block(t0):
        t1 = min(T, t0 + tb)
        acc = np.zeros((t1 - t0, E, LANES), np.float32)
        for j in range(J):
            for r in range(VEC):
                prod = xp[t0:t1, None, j, :, r] * wp[None, :, j, :, r]  # exact in fp32
                acc = acc + prod
        for o in (32, 16, 8, 4, 2, 1):
            acc = acc + acc[:, :, lanes ^ o]
        out[t0:t1] = acc[:, :, 0]

    list(_map(block, range(0, T, tb), workers))
    return out


def topk(logits, k, allowed=None):
    """Top-k expert ids per token, ordered by (logit descending, index ascending).

    With ``allowed`` (uint8 [T, E]) only allowed experts are ranked; each row must
    allow at least k experts."""
    logits = np.asarray(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    for t in range(T):
        cand = np.arange(E) if allowed is None else np.flatnonzero(np.asarray(allowed[t]) != 0)
        if cand.size < k:
            raise ValueError("fewer than k allowed experts")
        # lexsort: last key is primary -> (-logit asc, index asc)
        order = np.lexsort((cand, -logits[t, cand].astype(np.float64)))
        idx[t] = cand[order[:k]]
    return idx


def gates(logits, idx) -> np.ndarray:
    """Softmax over the k selected logits (fp64) == softmax over all E renormalised to the top-k."""
    sel = np.take_along_axis(np.asarray(logits, np.float64), np.asarray(idx, np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def route(x_bits, w_bits, k, allowed=None, workers=1):
    """(idx int32 [T,k], gates fp64 [T,k], logits fp32 [T,E])."""
    lg = router_logits(x_bits, w_bits, workers)
    idx = topk(lg, k, allowed)
    return idx, gates(lg, idx), lg
