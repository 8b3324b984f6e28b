"""Composition of one routed MoE layer call, decode and prefill.

Test infrastructure (see the package docstring).

Decode ([FT] §3.2): route, then classify / split / update the cache, then
y = sum_j g[t,j] FFN_idx[t,j](x[t]).  The merge of the GPU partial (pairs whose
expert is in G = H u F) and the CPU partial (pairs in C) is exact, so y does
not depend on the split; the oracle computes y once from its definition and
also returns the two partials for the split form.

Prefill ([FT] §3.1, §5.3 "Pipelined prefill"): all experts of the layer are
served from the prefill buffer, so y is the plain routed layer output.

fmt "mxfp4": expert records in MXFP4 (oracle.mx); decode applies the exactly
dequantised weights to the bf16 activations (on the GPU and on the CPU alike),
prefill quantises x and h to MXFP8 before each contraction.
"""
import numpy as np

from . import mx
from .ffn import moe_layer
from .router import route


def _layer_fn(fmt, form):
    if fmt == "bf16":
        return moe_layer
    if fmt == "mxfp4":
        return lambda *a, **kw: mx.moe_layer(*a, form=form, **kw)
    raise ValueError(f"unknown record format {fmt}")


def decode_layer(cache, layer, x_bits, w_r_bits, k, record_of, d, d_ff, fq,
                 min_fill=1, max_fetch=-1, allowed=None, fmt="bf16"):
    layer_fn = _layer_fn(fmt, "decode")
    idx, g, logits = route(x_bits, w_r_bits, k, allowed)
    plan = cache.lookup(layer, idx, fq, min_fill, max_fetch)
    y = layer_fn(x_bits, idx, g, record_of, d, d_ff)
    on_gpu = plan.pair_group >= 0
    y_gpu = layer_fn(x_bits, idx, g * on_gpu, record_of, d, d_ff)
    y_cpu = layer_fn(x_bits, idx, g * (~on_gpu), record_of, d, d_ff)
    return {"idx": idx, "gates": g, "logits": logits, "plan": plan, "y": y,
            "y_gpu": y_gpu, "y_cpu": y_cpu}


def prefill_layer(x_bits, w_r_bits, k, record_of, d, d_ff, tokens=None, fmt="bf16"):
    idx, g, logits = route(x_bits, w_r_bits, k)
    y = _layer_fn(fmt, "prefill")(x_bits, idx, g, record_of, d, d_ff, tokens=tokens)
    return {"idx": idx, "gates": g, "logits": logits, "y": y}
