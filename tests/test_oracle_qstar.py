"""Pins of the oracle's fetch split q against the pages' printed values and the
brute-force makespan optimum."""
import json
import os

import numpy as np
import pytest

from oracle.qstar import (Q16, fetch_fraction_q16, frac_q16, frac_q16_contended, hybrid_gate, phased_step_time,
                          q_rule, q_split, recommend_hybrid)

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "qstar_pages.json")))


def test_table1_q_at_m4():
    rows = GOLD["table1"]["rows"]
    got = [q_rule(4, frac_q16(r["B_P"], r["B_H"])) for r in rows]
    assert got == GOLD["q_m4_table1"]["values"]


def test_phi_0415_ceiling_regression():
    fq = round(GOLD["phi_0415"]["phi"] * Q16)
    for m, q in GOLD["phi_0415"]["cases"]:
        assert q_rule(m, fq) == q
    assert int(np.ceil(0.415 * 3)) == 2  # the rule is not a ceiling


def test_5090_m12_and_phased_cost():
    g = GOLD["rtx5090_m12"]
    fq = frac_q16(g["B_P"], g["B_H"])
    assert q_rule(g["m"], fq) == g["q"]
    bp, bh, S, m = g["B_P"] * 1e9, g["B_H"] * 1e9, g["S_bytes"], g["m"]
    t = [phased_step_time(m, q, S, bp, bh) for q in range(m + 1)]
    for q in range(g["q"] + 1):
        assert round(t[q] * 1e3, 3) == g["phased_ms_le_qstar"]
    assert round(t[m] * 1e3, 3) == g["phased_ms_q_eq_m"]
    assert all(b > a for a, b in zip(t[g["q"]:], t[g["q"] + 1:]))
    # Eq. (3) makespan with the residual CPU bandwidth has its integer argmin at q*
    eq3 = [max(q * S / bp, (m - q) * S / (bh - bp)) for q in range(m + 1)]
    assert int(np.argmin(eq3)) == g["q"]


def test_laptop_returns_zero_without_floor_and_one_with():
    g = GOLD["laptop_small_m"]
    fq = frac_q16(g["B_P"], g["B_H"])
    for m, q in g["cases"]:
        assert q_rule(m, fq) == q
        assert q_split(m, fq, min_fill=0) == 0
        assert q_split(m, fq, min_fill=1) == 1  # the paper's "at least one fill"


def test_figure2_example():
    g = GOLD["figure2"]
    assert q_rule(g["m"], round(g["phi"] * Q16)) == g["q"]


def test_endpoints():
    g = GOLD["endpoints"]
    for bp, bh in g["pairs_full_fill"]:
        assert frac_q16(bp, bh) == Q16
        assert q_rule(g["m"], frac_q16(bp, bh)) == g["m"]
    assert frac_q16(0.0, 77.3) == 0
    for m in range(0, 65):
        assert q_rule(m, 0) == 0
        assert q_rule(m, Q16) == m
    d = GOLD["degraded_cpu"]
    assert q_rule(d["m"], frac_q16(d["B_P"], d["B_H"])) == d["q"]


def test_within_one_expert_of_eq4():
    for phi in GOLD["phi_set"]["values"]:
        fq = round(phi * Q16)
        for m in range(65):
            q = q_rule(m, fq)
            assert 0 <= q <= m
            assert abs(q - phi * m) <= 1.0


def test_rule_is_lowest_integer_argmin_exhaustive():
    """For every fq in [0, 2^16] and m <= 64 the two-candidate pick equals the
    lowest-index argmin over all f in [0, m] of the Eq. (3) makespan (scaled)."""
    fq = np.arange(Q16 + 1, dtype=np.int64)
    for m in range(0, 65):
        f = np.arange(m + 1, dtype=np.int64)[:, None]
        cost = np.maximum(f * (Q16 - fq)[None, :], (m - f) * fq[None, :])
        best = np.argmin(cost, axis=0)  # first minimum = lowest index
        got = np.array([q_rule(m, int(v)) for v in fq[:: 97]] + [q_rule(m, Q16)])
        assert np.array_equal(got, np.concatenate([best[:: 97], best[-1:]])), m
    # a denser sweep at small m, where ties are most frequent
    for m in range(1, 9):
        f = np.arange(m + 1, dtype=np.int64)[:, None]
        cost = np.maximum(f * (Q16 - fq)[None, :], (m - f) * fq[None, :])
        best = np.argmin(cost, axis=0)
        got = np.array([q_rule(m, int(v)) for v in fq])
        assert np.array_equal(got, best), m


def test_rule_matches_eq3_with_table1_bandwidths():
    """Against the physical Eq. (3) makespan max(qS/B_P, (m-q)S/(B_H-B_P)) in floating point."""
    for r in GOLD["table1"]["rows"]:
        bp, bh = r["B_P"], r["B_H"]
        fq = frac_q16(bp, bh)
        for m in range(1, 65):
            c = [max(q / bp, (m - q) / (bh - bp)) for q in range(m + 1)]
            best = min(range(m + 1), key=lambda q: (c[q], q))
            assert q_rule(m, fq) == best, (r["system"], m)


def test_caps_and_floor_order():
    fq = frac_q16(11.8, 47.5)
    assert q_split(3, fq, min_fill=1, max_fetch=0) == 0       # 0 never fetches
    assert q_split(12, Q16, min_fill=1, max_fetch=2) == 2     # fixed cap
    assert q_split(12, Q16, min_fill=1, max_fetch=-1, avail=5) == 5
    assert q_split(0, Q16) == 0
    assert q_split(5, 0, min_fill=3) == 3
    assert q_split(2, 0, min_fill=3) == 2
    assert q_split(4, Q16, avail=0) == 0


def test_hybrid_gate_on_table1():
    """Every Table 1 machine's printed ratio and gate verdict (threshold 2.0)."""
    g = GOLD["gate_table1"]
    rows = {r["system"]: (r["B_P"], r["B_H"]) for r in GOLD["table1"]["rows"]}
    for r in g["rows"]:
        B_P, B_H = rows[r["system"]]
        assert round(B_H / B_P, 2) == pytest.approx(r["ratio"]), r
        assert hybrid_gate(B_P, B_H, g["threshold"]) == r["hybrid"], r
    # the gate is strict: exactly twice B_P does not pass
    assert not hybrid_gate(10.0, 20.0) and hybrid_gate(10.0, 20.000001)


def test_recommendation_is_unanimous_or_offload():
    t1 = [(r["B_P"], r["B_H"]) for r in GOLD["table1"]["rows"]]
    assert recommend_hybrid([t1[1], t1[2], t1[4], t1[5]])  # the four machines that pass
    assert not recommend_hybrid(t1)                        # a mixed verdict resolves to offload
    assert not recommend_hybrid([t1[0]])
    assert not recommend_hybrid([])                        # no benched workload, no upgrade


def test_contended_fraction_closed_forms():
    """Under total contention (the CPU keeps only B_H - B_P while the link runs) the
    contended fraction is Eq. (4) exactly; when the CPU kernel never saturates DRAM
    (cpu_ov = B_H) it is B_P / (B_P + B_H), below Eq. (4)."""
    for r in GOLD["table1"]["rows"]:
        B_P, B_H = r["B_P"], r["B_H"]
        assert frac_q16_contended(B_P, B_H - B_P) == frac_q16(B_P, B_H), r
        low = frac_q16_contended(B_P, B_H)
        assert low == round(B_P / (B_P + B_H) * Q16)
        assert low < frac_q16(B_P, B_H)


def test_contended_fraction_rounding_and_fallback():
    # ties go to even: 2^16 * 1/131072 = 0.5 -> 0, 2^16 * 3/131072 = 1.5 -> 2
    assert frac_q16_contended(1.0, 131071.0) == 0
    assert frac_q16_contended(3.0, 131069.0) == 2
    assert frac_q16_contended(0.0, 5.0) == 0 and frac_q16_contended(5.0, 0.0) == Q16
    # a profile without the pair falls back to Eq. (4)
    assert fetch_fraction_q16(52.7, 77.3) == frac_q16(52.7, 77.3)
    assert fetch_fraction_q16(52.7, 77.3, 0.0, 30.0) == frac_q16(52.7, 77.3)
    assert fetch_fraction_q16(52.7, 77.3, 50.0, 30.0) == frac_q16_contended(50.0, 30.0)
