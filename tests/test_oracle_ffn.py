"""Pins of the oracle's SwiGLU expert FFN and layer output: explicit loops with
math.exp on tiny inputs, the record layout, the branch that carries silu, the
dense evaluate-every-expert brute force, and linearity in the gates."""
import math

import numpy as np

from moe_expert_offload_amd.synth import f32_to_bf16_bits
from oracle.common import bf16_to_f64
from oracle.ffn import expert_ffn, moe_layer, moe_layer_dense, split_record
from oracle.router import route


def _record(rng, d, d_ff, std=0.5):
    return f32_to_bf16_bits(rng.normal(0, std, size=3 * d * d_ff))


def test_expert_ffn_explicit_loops():
    rng = np.random.default_rng(10)
    d, d_ff = 5, 3
    rec = _record(rng, d, d_ff)
    v = bf16_to_f64(rec)
    x = rng.normal(size=d)
    # record layout written out by index: gate rows, then up rows, then down rows
    def Wg(r, i): return v[r * d + i]
    def Wu(r, i): return v[d * d_ff + r * d + i]
    def Wd(c, r): return v[2 * d * d_ff + c * d_ff + r]
    ref = []
    for c in range(d):
        s = 0.0
        for r in range(d_ff):
            zg = sum(Wg(r, i) * x[i] for i in range(d))
            zu = sum(Wu(r, i) * x[i] for i in range(d))
            s += Wd(c, r) * (zg / (1.0 + math.exp(-zg))) * zu
        ref.append(s)
    got = expert_ffn(split_record(rec, d, d_ff), x[None, :])[0]
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_silu_is_on_the_gate_branch():
    d, d_ff = 2, 1
    # gate row picks x0, up row picks x1, down maps h to both outputs
    wg = np.array([[1.0, 0.0]]); wu = np.array([[0.0, 1.0]]); wd = np.array([[1.0], [2.0]])
    x = np.array([[-4.0, 3.0]])
    out = expert_ffn((wg, wu, wd), x)[0]
    silu_m4 = -4.0 / (1.0 + math.exp(4.0))
    assert np.allclose(out, [silu_m4 * 3.0, 2 * silu_m4 * 3.0], rtol=1e-14)
    swapped = (3.0 / (1.0 + math.exp(-3.0))) * -4.0
    assert not np.isclose(out[0], swapped)
    assert np.allclose(expert_ffn((wg, np.zeros_like(wu), wd), x), 0.0)


def test_dense_brute_force_matches_sparse():
    rng = np.random.default_rng(11)
    T, d, d_ff, E, k = 7, 16, 8, 5, 2
    recs = [_record(rng, d, d_ff, 0.3) for _ in range(E)]
    x = f32_to_bf16_bits(rng.normal(size=(T, d)))
    wr = f32_to_bf16_bits(rng.normal(0, 0.5, size=(E, d)))
    idx, g, _ = route(x, wr, k)
    y = moe_layer(x, idx, g, lambda e: recs[e], d, d_ff)
    yd = moe_layer_dense(x, idx, g, lambda e: recs[e], E, d, d_ff)
    assert np.allclose(y, yd, rtol=1e-12, atol=1e-14)
    # sampled rows give the same rows
    ys = moe_layer(x, idx, g, lambda e: recs[e], d, d_ff, tokens=[1, 4])
    assert np.allclose(ys, y[[1, 4]], rtol=1e-13, atol=1e-15)


def test_linear_in_gates_and_zero_gate_drops_expert():
    rng = np.random.default_rng(12)
    T, d, d_ff, E, k = 4, 8, 4, 3, 2
    recs = [_record(rng, d, d_ff, 0.3) for _ in range(E)]
    x = f32_to_bf16_bits(rng.normal(size=(T, d)))
    idx = np.array([[0, 1], [1, 2], [2, 0], [0, 2]])
    g = rng.random((T, k))
    y1 = moe_layer(x, idx, g, lambda e: recs[e], d, d_ff)
    y2 = moe_layer(x, idx, 2 * g, lambda e: recs[e], d, d_ff)
    assert np.allclose(y2, 2 * y1, rtol=1e-13)
    g0 = g.copy(); g0[:, 1] = 0
    y0 = moe_layer(x, idx, g0, lambda e: recs[e], d, d_ff)
    x64 = bf16_to_f64(x)
    ref = np.stack([g[t, 0] * expert_ffn(split_record(recs[idx[t, 0]], d, d_ff), x64[t:t + 1])[0] for t in range(T)])
    assert np.allclose(y0, ref, rtol=1e-13)
