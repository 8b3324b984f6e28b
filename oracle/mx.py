"""MXFP4 experts and MXFP8 activations: decoding, quantisation and the FFN forms.

Test infrastructure (see the package docstring).

[FT] §5.1 "Models": DeepSeek-V4-Flash is served from its official checkpoint
whose routed experts are natively MXFP4-quantised, and [FT] §4.1 "Graph-resident
CPU execution": the CPU workers dequantise inside their kernels.  The pages do
not define the format beyond its name; this build follows the OCP Microscaling
(MX) Formats specification v1.0:

  * an MX block is k = 32 elements sharing one E8M0 scale X = 2^(E - 127)
    (E = 255 is NaN and never produced), element value = X * decode(code);
  * FP4 E2M1 element codes: sign bit 3, magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6};
  * FP8 E4M3 element codes: sign bit 7, exponent bias 7, 3 mantissa bits,
    subnormals at exponent field 0, max normal 448, S.1111.111 is NaN;
  * conversion of a block (OCP MX v1.0, §6.3): shared exponent
    floor(log2(max|v|)) - emax_elem (emax = 2 for E2M1, 8 for E4M3), elements
    v / X rounded to nearest even and clamped to the largest normal.

Readings of this build:
  * weights: blocks of 32 consecutive elements along the reduction axis of each
    matrix (d for W_gate/W_up, d_ff for W_down); two E2M1 codes per byte, the
    lower-index element in the low nibble;
  * activations (only where the prefill uses the scaled MFMA): MXFP8 E4M3 with
    blocks of 32 consecutive elements along the reduction axis, like the
    weights; a block whose values are all zero gets E = 0 and zero codes;
  * decode (few tokens per expert) uses the weights alone: FFN with exactly
    dequantised weights and the bf16 activations as given;
  * prefill with MXFP4 experts quantises x and h = silu(W_gate x) * (W_up x) to
    MXFP8 before each contraction; h is quantised from its fp64 value here, so
    codes may differ from a fp32 computation only at rounding boundaries.

Record layout (bytes): [gate codes d_ff x d/2 | up codes d_ff x d/2 |
down codes d x d_ff/2 | gate scales d_ff x d/32 | up scales d_ff x d/32 |
down scales d x d_ff/32], all row-major.
"""
import numpy as np

from .common import bf16_to_f64
from .ffn import _map

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_EMAX = 2
E4M3_EMAX = 8
E4M3_MAX = 448.0


# the 16 code values: bit 3 is the sign, bits 0-2 index the magnitude (code 8 is -0)
_E2M1_SIGNED = np.concatenate([E2M1_MAG, -E2M1_MAG])


def e2m1_value(codes):
    c = np.asarray(codes, np.uint8) & 0xF
    return np.take(_E2M1_SIGNED, c)


def e4m3_value(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    if np.any((e == 15) & (m == 7)):
        raise ValueError("E4M3 NaN code")
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where(s == 1, -mag, mag)


def e8m0_value(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    if np.any(c == 255):
        raise ValueError("E8M0 NaN scale")
    return np.exp2(c - 127.0)


def _sorted_grid(vals, codes):
    order = np.argsort(vals, kind="stable")
    gv, gc = vals[order], codes[order]
    keep = np.ones(gv.size, bool)  # +0 and -0: keep +0
    zeros = np.flatnonzero(gv == 0)
    if zeros.size > 1:
        keep[zeros] = False
        keep[zeros[np.argmin(gc[zeros])]] = True
    return gv[keep], gc[keep]


def _e2m1_grid():
    codes = np.arange(16, dtype=np.uint8)
    return _sorted_grid(e2m1_value(codes), codes)


def _e4m3_grid():
    codes = np.arange(256, dtype=np.uint8)
    ok = (((codes >> 3) & 0xF) != 15) | ((codes & 7) != 7)
    return _sorted_grid(e4m3_value(codes[ok]), codes[ok])


_GRID = {"e2m1": _e2m1_grid() + (E2M1_EMAX, 6.0), "e4m3": _e4m3_grid() + (E4M3_EMAX, E4M3_MAX)}


def _round_to_grid(v, gv, gc):
    """Nearest grid value, ties to the code with an even mantissa bit (round half to
    even); v within the grid's range."""
    i = np.clip(np.searchsorted(gv, v), 1, gv.size - 1)
    lo, hi = gv[i - 1], gv[i]
    dlo, dhi = v - lo, hi - v
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((gc[i] & 1) == 0))
    return np.where(pick_hi, gc[i], gc[i - 1])


def quantize_blocks(v, fmt):
    """OCP MX conversion of blocks v [..., 32] (fp64): (E8M0 codes [...], element codes [..., 32])."""
    v = np.asarray(v, np.float64)
    gv, gc, emax, vmax = _GRID[fmt]
    amax = np.max(np.abs(v), axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))).astype(np.int64) - emax
    e = np.clip(e, -127, 127)
    scaled = np.clip(v / np.exp2(e)[..., None], -vmax, vmax)
    codes = _round_to_grid(scaled, gv, gc).astype(np.uint8)
    zero = amax == 0
    codes[zero] = 0
    return np.where(zero, 0, e + 127).astype(np.uint8), codes


def quantize_block(v, fmt):
    """One block: (E8M0 code, element codes)."""
    s, c = quantize_blocks(np.asarray(v, np.float64)[None, :], fmt)
    return int(s[0]), c[0]


def act_block_index(n):
    """For a reduction axis of length n (multiple of 32): an int array [n // 32, 32]
    listing the element indices of each activation block (32 consecutive elements)."""
    if n % 32:
        raise ValueError("activation MX blocks need a multiple of 32 elements")
    return np.arange(n).reshape(n // 32, 32)


def quantize_act_codes(v):
    """MXFP8 E4M3 conversion of activation rows v [rows, n]: (element codes uint8
    [rows, n], E8M0 scale codes uint8 [rows, n // 32])."""
    v = np.atleast_2d(np.asarray(v, np.float64))
    blocks = act_block_index(v.shape[1])
    s, c = quantize_blocks(v[:, blocks], "e4m3")
    codes = np.empty(v.shape, np.uint8)
    codes[:, blocks] = c
    return codes, s


def quantize_act(v):
    """MXFP8 E4M3 quantisation of activation rows v [rows, n] -> dequantised fp64 values."""
    v = np.atleast_2d(np.asarray(v, np.float64))
    blocks = act_block_index(v.shape[1])
    c, s = quantize_act_codes(v)
    out = np.empty_like(v)
    out[:, blocks] = e8m0_value(s)[..., None] * e4m3_value(c[:, blocks])
    return out


def record_bytes(d, d_ff):
    return 3 * d * d_ff // 2 + 3 * d * d_ff // 32


def _unpack_codes(b, rows, cols):
    b = np.asarray(b, np.uint8).reshape(rows, cols // 2)
    out = np.empty((rows, cols), np.uint8)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return out


def split_record(rec, d, d_ff):
    """(W_gate, W_up, W_down) as exactly dequantised float64 from one MXFP4 record."""
    r = np.asarray(rec, np.uint8).reshape(-1)
    if r.size != record_bytes(d, d_ff):
        raise ValueError("record size does not match (d, d_ff)")
    n2 = d * d_ff // 2
    n32 = d * d_ff // 32
    cg, cu, cd = r[0:n2], r[n2:2 * n2], r[2 * n2:3 * n2]
    sg, su, sd = r[3 * n2:3 * n2 + n32], r[3 * n2 + n32:3 * n2 + 2 * n32], r[3 * n2 + 2 * n32:3 * n2 + 3 * n32]

    def deq(codes, scales, rows, cols):
        v = e2m1_value(_unpack_codes(codes, rows, cols))
        x = e8m0_value(np.asarray(scales, np.uint8).reshape(rows, cols // 32))
        return v * np.repeat(x, 32, axis=1)

    return deq(cg, sg, d_ff, d), deq(cu, su, d_ff, d), deq(cd, sd, d, d_ff)


def silu(z):
    return z / (1.0 + np.exp(-z))


def expert_ffn_decode(W, x):
    """Decode form: dequantised weights, activations as given (fp64)."""
    wg, wu, wd = W
    x = np.atleast_2d(np.asarray(x, np.float64))
    h = silu(x @ wg.T) * (x @ wu.T)
    return h @ wd.T


def expert_ffn_prefill(W, x):
    """Prefill form on the scaled MFMA: x and h quantised to MXFP8 before each contraction."""
    wg, wu, wd = W
    xq = quantize_act(np.atleast_2d(np.asarray(x, np.float64)))
    h = silu(xq @ wg.T) * (xq @ wu.T)
    return quantize_act(h) @ wd.T


def moe_layer(x_bits, idx, g, record_of, d, d_ff, form="decode", tokens=None, workers=1):
    """y [rows, d] = sum_j g[t,j] FFN_idx[t,j](x[t]) in rank order, with MXFP4 experts
    (``workers`` > 1: experts evaluated on that many threads, arithmetic unchanged)."""
    x = bf16_to_f64(x_bits)
    idx = np.asarray(idx)
    g = np.asarray(g, np.float64)
    rows = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    sub = idx[rows]
    k = idx.shape[1]
    ffn = expert_ffn_decode if form == "decode" else expert_ffn_prefill
    contrib = np.zeros((rows.size, k, d))

    def one(e):
        W = split_record(record_of(int(e)), d, d_ff)
        sel_t, sel_j = np.nonzero(sub == e)
        return sel_t, sel_j, ffn(W, x[rows[sel_t]])

    for sel_t, sel_j, out in _map(one, np.unique(sub), workers):
        contrib[sel_t, sel_j] = g[rows[sel_t], sel_j][:, None] * out
    y = np.zeros((rows.size, d))
    for j in range(k):
        y = y + contrib[:, j]
    return y
