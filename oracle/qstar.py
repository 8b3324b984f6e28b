"""The bandwidth-adaptive split of a decode step's cache misses.

Test infrastructure (see the package docstring).

[FT] §3.2, Eqs. (1)-(4): the m unique misses M split into a cache-fill set F
(q = |F| experts, copied over PCIe at B_P) and a CPU set C (executed in place
on the host, which has the residual bandwidth B_R = max(B_H - B_P, 0) while
the link is busy).  Balancing T_fill = qS/B_P against T_cpu = (m-q)S/(B_H-B_P)
gives q* ~= m B_P / B_H.  [FT] §3.2 further says q* is rounded to an integer
and at least one fill is kept.

[AIN] "The split, and what it is actually optimising": the shipped rule
works in Q16 fixed point.  With fq = round(2^16 B_P / B_H) computed once,
lo = floor(m fq / 2^16) and the pick is whichever of lo, lo + 1 has the smaller
makespan max(f (2^16 - fq), (m - f) fq), lo on a tie, capped at m.  [AIN]
"How to use it" (flags table): a non-negative max_fetch caps the fetch count
and 0 never fetches; with no bandwidth profile the cap is one fetch.

Readings of this build where the pages disagree or are silent:
  * rounding: the Q16 makespan pick, not round();
  * "at least one fill": a min_fill parameter (the paper's floor when 1, the
    shipped rule when 0), applied after the Q16 pick and before the caps;
  * caps: q <= max_fetch when max_fetch >= 0, then q <= m and q <= avail
    (the number of slots that may be evicted in this call);
  * B_P >= B_H: no residual host bandwidth, fq = 2^16 and q = m;  B_P = 0: fq = 0.
"""
from __future__ import annotations

Q16 = 1 << 16


def frac_q16(B_P: float, B_H: float) -> int:
    """Eq. (4)'s fraction phi = B_P / B_H in Q16, rounded half to even, clamped to [0, 2^16]."""
    if B_P <= 0.0:
        return 0
    if B_P >= B_H:
        return Q16
    v = round((B_P / B_H) * Q16)  # Python round(): ties to even
    return int(min(Q16, max(0, v)))


def makespan_q16(f: int, m: int, fq: int) -> int:
    """Eq. (3) makespan of f fills and m - f CPU experts, scaled to integers by
    (B_P (B_H - B_P) / (S B_H)) * 2^16: max(f (2^16 - fq), (m - f) fq)."""
    fill_side = f * (Q16 - fq)
    cpu_side = (m - f) * fq
    return fill_side if fill_side >= cpu_side else cpu_side


def q_rule(m: int, fq: int) -> int:
    """The Q16 integer pick of the balanced fetch count (no floor, no caps except m)."""
    if m <= 0:
        return 0
    lo = (m * fq) // Q16
    hi = lo + 1
    pick = hi if makespan_q16(hi, m, fq) < makespan_q16(lo, m, fq) else lo
    return pick if pick < m else m


def q_split(m: int, fq: int, min_fill: int = 1, max_fetch: int = -1, avail: int | None = None) -> int:
    """Fetch count q for m unique misses: Q16 pick, then the fill floor, then the caps."""
    if m <= 0:
        return 0
    q = q_rule(m, fq)
    floor = min_fill if min_fill < m else m
    if q < floor:
        q = floor
    if max_fetch >= 0 and q > max_fetch:
        q = max_fetch
    if q > m:
        q = m
    if avail is not None and q > avail:
        q = max(avail, 0)
    return q


def phased_step_time(m: int, q: int, S: float, B_P: float, B_H: float) -> float:
    """Wall time of one layer's miss path under the phase-aware model.

    [AIN] "The split, and what it is actually optimising": the q fills move
    q S bytes at B_P; while they are in flight the CPU branch reads host memory
    at the residual rate max(B_H - B_P, 0) and at the full B_H once the link is
    idle.  Every q <= q* then costs exactly m S / B_H.
    """
    t_fill = q * S / B_P if q > 0 else 0.0
    cpu_bytes = (m - q) * S
    done_during_fill = max(B_H - B_P, 0.0) * t_fill
    if done_during_fill >= cpu_bytes:
        return t_fill
    return t_fill + (cpu_bytes - done_during_fill) / B_H


# ---- the bandwidth profile: contended fraction and the hybrid gate ----------------
#
# [AIN] "How to use it" / "How to maintain it": the fetch fraction is computed once
# at engine start from a per-machine bandwidth profile.  The preferred derivation
# uses a contended pair -- the PCIe gather rate measured while the CPU expert
# kernel runs (pcie_ov) and the CPU kernel's rate measured while the gather runs
# (cpu_ov) -- as pcie_ov / (pcie_ov + cpu_ov); a profile without that pair falls
# back to B_P / B_H, Eq. (4).  The two agree when the contention is total (the CPU
# keeps only the residual B_H - B_P).  [AIN] "Why use it": the hybrid backend is
# chosen only when B_H exceeds twice B_P, and only when every benched workload of
# the expert format agrees; otherwise the plain offload backend.


def frac_q16_contended(pcie_ov: float, cpu_ov: float) -> int:
    """pcie_ov / (pcie_ov + cpu_ov) in Q16, rounded half to even, clamped to [0, 2^16]."""
    if pcie_ov <= 0.0:
        return 0
    if cpu_ov <= 0.0:
        return Q16
    v = round(pcie_ov / (pcie_ov + cpu_ov) * Q16)
    return int(min(Q16, max(0, v)))


def fetch_fraction_q16(B_P: float, B_H: float, pcie_ov: float | None = None, cpu_ov: float | None = None) -> int:
    """The contended pair when the profile has it (both rates positive), else Eq. (4)."""
    if pcie_ov is not None and cpu_ov is not None and pcie_ov > 0.0 and cpu_ov > 0.0:
        return frac_q16_contended(pcie_ov, cpu_ov)
    return frac_q16(B_P, B_H)


def hybrid_gate(B_P: float, B_H: float, threshold: float = 2.0) -> bool:
    """One workload's verdict: hybrid only when B_H > threshold * B_P."""
    return B_H > threshold * B_P


def recommend_hybrid(pairs, threshold: float = 2.0) -> bool:
    """Unanimous or offload: hybrid only when there is at least one benched workload
    and every one of them passes the gate."""
    pairs = list(pairs)
    return len(pairs) > 0 and all(hybrid_gate(p, h, threshold) for p, h in pairs)
