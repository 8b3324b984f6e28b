"""SwiGLU expert FFN and the routed layer output, in fp64.

Test infrastructure (see the package docstring).

[FT] §3 (a cache slot holds every tensor of one layer-expert pair) and §3.2
(the CPU and GPU partial sums merge into the exact MoE output, with no
approximation).  The pages do not spell out the expert function; this build
uses SwiGLU without biases:

    FFN_e(x) = W_down,e ( silu(W_gate,e x) * (W_up,e x) ),   silu(z) = z / (1 + e^-z)

and the layer output  y[t] = sum_j g[t,j] * FFN_{idx[t,j]}(x[t])  (j in rank order).

Expert records are bf16 words laid out [W_gate (d_ff x d) | W_up (d_ff x d) |
W_down (d x d_ff)], row-major.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .common import bf16_to_f64


def _map(fn, items, workers):
    if workers <= 1:
        return map(fn, items)
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, items))


def split_record(record_bits, d, d_ff):
    """(W_gate [d_ff,d], W_up [d_ff,d], W_down [d,d_ff]) as float64 from one record."""
    r = np.asarray(record_bits, dtype=np.uint16).reshape(-1)
    n = d * d_ff
    if r.size != 3 * n:
        raise ValueError("record size does not match (d, d_ff)")
    wg = bf16_to_f64(r[0:n]).reshape(d_ff, d)
    wu = bf16_to_f64(r[n:2 * n]).reshape(d_ff, d)
    wd = bf16_to_f64(r[2 * n:3 * n]).reshape(d, d_ff)
    return wg, wu, wd


def silu(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def expert_ffn(weights, x):
    """FFN_e for a batch of rows x [n, d] (float64) -> [n, d]."""
    wg, wu, wd = weights
    x = np.atleast_2d(np.asarray(x, np.float64))
    zg = x @ wg.T
    zu = x @ wu.T
    h = silu(zg) * zu
    return h @ wd.T


def moe_layer(x_bits, idx, g, record_of, d, d_ff, tokens=None, workers=1):
    """Sparse layer output y [T or len(tokens), d] (float64).

    record_of(e) returns the bf16 record of expert e of this layer.  ``tokens``
    restricts the computation to a sample of token rows (for large inputs).
    The k gate-weighted expert outputs of a token are summed in rank order j.
    ``workers`` > 1 evaluates the experts on that many threads (each expert's
    arithmetic is unchanged; only its wall time is shared)."""
    x = bf16_to_f64(x_bits)
    idx = np.asarray(idx)
    g = np.asarray(g, np.float64)
    rows = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    k = idx.shape[1]
    sub = idx[rows]
    contrib = np.zeros((rows.size, k, d))

    def one(e):
        w = split_record(record_of(int(e)), d, d_ff)
        sel_t, sel_j = np.nonzero(sub == e)
        return sel_t, sel_j, expert_ffn(w, x[rows[sel_t]])

    for sel_t, sel_j, out in _map(one, np.unique(sub), workers):
        contrib[sel_t, sel_j] = g[rows[sel_t], sel_j][:, None] * out
    y = np.zeros((rows.size, d))
    for j in range(k):
        y = y + contrib[:, j]
    return y


def moe_layer_dense(x_bits, idx, g, record_of, E, d, d_ff):
    """Brute force: evaluate every expert on every token, then mask by the gates."""
    x = bf16_to_f64(x_bits)
    T = x.shape[0]
    gate_dense = np.zeros((T, E))
    for t in range(T):
        for j in range(idx.shape[1]):
            gate_dense[t, idx[t, j]] += g[t, j]
    y = np.zeros((T, d))
    for e in range(E):
        out = expert_ffn(split_record(record_of(e), d, d_ff), x)
        y += gate_dense[:, e:e + 1] * out
    return y
