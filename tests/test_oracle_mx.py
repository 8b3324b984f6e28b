"""Pins of the oracle's MXFP4 / MXFP8 handling against the OCP Microscaling
Formats v1.0 definitions: element code tables, the block conversion (brute-force
nearest representable value with ties to even, saturation, shared-exponent
rule), the activation block partition, and the record layout."""
import numpy as np
import pytest

from moe_expert_offload_amd.synth import mxfp4_record_from_weights
from oracle import mx


def test_e2m1_table():
    # OCP MX v1.0 FP4 E2M1: exponent bias 1, one mantissa bit, subnormal 0.5
    want = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert mx.e2m1_value(np.arange(8)).tolist() == want
    assert mx.e2m1_value(np.arange(8, 16)).tolist() == [-v for v in want]


def test_e4m3_table_points():
    v = mx.e4m3_value(np.array([0x7E, 0x08, 0x07, 0x01, 0x38, 0xB8, 0x00], np.uint8)).tolist()
    assert v == [448.0, 2.0 ** -6, 0.875 * 2.0 ** -6, 2.0 ** -9, 1.0, -1.0, 0.0]
    with pytest.raises(ValueError):
        mx.e4m3_value(np.array([0x7F], np.uint8))
    assert mx.e8m0_value(np.array([127, 0, 254], np.uint8)).tolist() == [1.0, 2.0 ** -127, 2.0 ** 127]


def _brute(v, fmt):
    """Nearest representable scaled value by exhaustive search, ties to the even code."""
    if fmt == "e2m1":
        codes = np.arange(16, dtype=np.uint8)
        vals = mx.e2m1_value(codes)
        emax, vmax = 2, 6.0
    else:
        codes = np.array([c for c in range(256) if not (((c >> 3) & 15) == 15 and (c & 7) == 7)], np.uint8)
        vals = mx.e4m3_value(codes)
        emax, vmax = 8, 448.0
    amax = np.max(np.abs(v))
    e = int(np.floor(np.log2(amax))) - emax
    out = []
    for x in v:
        s = min(max(x / 2.0 ** e, -vmax), vmax)
        best = None
        for c, val in zip(codes.tolist(), vals.tolist()):
            dist = abs(s - val)
            key = (dist, c & 1, c)  # smaller distance, then even mantissa bit
            if best is None or key < best[0]:
                best = (key, val)
        out.append(best[1] * 2.0 ** e)
    return np.array(out)


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_block_conversion_matches_brute_force(fmt):
    rng = np.random.default_rng(1)
    for trial in range(40):
        v = rng.normal(0, 0.02, 32) * (10.0 ** rng.integers(-3, 3))
        if trial % 5 == 0:  # exact ties and boundaries
            v[:8] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.5]) * 2.0 ** -3
        s, c = mx.quantize_block(v, fmt)
        val = mx.e8m0_value(s) * (mx.e2m1_value(c) if fmt == "e2m1" else mx.e4m3_value(c))
        assert np.array_equal(val, _brute(v, fmt)), trial


def test_scale_rule_and_saturation():
    v = np.zeros(32)
    v[0] = 7.9  # top binade [4, 8) at scale 2^0 for E2M1: clamps to 6
    s, c = mx.quantize_block(v, "e2m1")
    assert s == 127 and mx.e2m1_value(c)[0] == 6.0
    v[0] = 500.0 * 2 ** -5  # E4M3 at scale 2^(floor(log2)) - 8
    s, c = mx.quantize_block(v, "e4m3")
    assert s == 127 + int(np.floor(np.log2(v[0]))) - 8
    assert mx.e4m3_value(c)[0] * mx.e8m0_value(s) == 448.0 * mx.e8m0_value(s)
    s, c = mx.quantize_block(np.zeros(32), "e4m3")
    assert s == 0 and not c.any()


def test_representable_values_round_trip_and_idempotence():
    rng = np.random.default_rng(2)
    x = rng.normal(0, 1, (5, 128))
    q = mx.quantize_act(x)
    assert np.array_equal(mx.quantize_act(q), q)
    blocks = mx.act_block_index(128)
    for r in range(5):
        for b in blocks:
            xb = x[r, b]
            X = 2.0 ** (np.floor(np.log2(np.abs(xb).max())) - 8)  # the block's scale
            a = np.abs(xb)
            # half an E4M3 ulp of each element's own binade (subnormals: X 2^-10), or the
            # clamp to 448 X in the top binade
            half_ulp = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(a, 1e-300))) - 4), X * 2.0 ** -10)
            bound = np.where(a > 448 * X, a - 448 * X, half_ulp)
            assert np.all(np.abs(q[r, b] - xb) <= bound * (1 + 1e-12))


def test_activation_blocks_partition_the_axis():
    b = mx.act_block_index(256)
    assert b.shape == (8, 32)
    assert b.reshape(-1).tolist() == list(range(256))
    assert b[1].tolist() == list(range(32, 64))
    with pytest.raises(ValueError):
        mx.act_block_index(80)


def test_record_layout_from_known_codes():
    """Weights chosen exactly representable: the record must decode to them."""
    d, d_ff = 64, 32
    rng = np.random.default_rng(3)
    def rep(rows, cols):
        codes = rng.integers(0, 16, (rows, cols))
        codes[:, ::32] = 7  # every block reaches +6 so its scale is exactly the chosen one
        scale_e = rng.integers(-9, -3, (rows, cols // 32))
        return mx.e2m1_value(codes) * np.repeat(2.0 ** scale_e, 32, axis=1)
    wg, wu, wd = rep(d_ff, d), rep(d_ff, d), rep(d, d_ff)
    rec = mxfp4_record_from_weights(wg, wu, wd)
    g, u, dd = mx.split_record(rec, d, d_ff)
    assert np.array_equal(g, wg) and np.array_equal(u, wu) and np.array_equal(dd, wd)
    # byte-level: first byte = codes of elements 0 (low nibble) and 1 (high nibble) of W_gate row 0
    c0 = int(mx.e2m1_value(np.arange(16)).tolist().index(wg[0, 0] / 2.0 ** np.floor(np.log2(np.abs(wg[0, :32]).max()) - 2)))
    assert rec[0] & 0xF == c0
    assert rec.size == mx.record_bytes(d, d_ff)


def test_prefill_form_reduces_to_decode_form_on_representable_inputs():
    """When x and h are already MXFP8 values the two forms agree exactly in fp64."""
    d, d_ff = 64, 64
    W = (np.eye(d_ff, d) * 0.5, np.eye(d_ff, d) * 2.0, np.eye(d, d_ff))
    x = mx.quantize_act(np.full((1, d), 1.0))
    # h = silu(0.5) * 2 is not representable in general; compare against explicit quantisation
    y_pre = mx.expert_ffn_prefill(W, x)
    h = mx.silu(0.5 * x) * (2.0 * x)
    assert np.allclose(y_pre, mx.quantize_act(h) @ W[2].T, rtol=0, atol=0)
