"""Small helpers of the oracle: bf16 decoding and the output tolerance.

Test infrastructure (see the package docstring).
"""
import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 words (uint16) -> float64; a bf16 is the top 16 bits of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def within_tolerance(got, ref, max_rel=2e-2, l1_rel=3e-3):
    """Layer-output tolerance: max|got-ref| <= max_rel*max|ref| and
    sum|got-ref| / sum|ref| <= l1_rel (relative l1, so entries near zero
    cannot dominate).  Returns (ok, max_ratio, l1_ratio)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    mref = float(np.max(np.abs(ref))) if ref.size else 0.0
    sref = float(np.sum(np.abs(ref))) if ref.size else 0.0
    max_ratio = float(diff.max()) / mref if mref > 0 else float(diff.max() if diff.size else 0.0)
    l1_ratio = float(diff.sum()) / sref if sref > 0 else float(diff.sum())
    return (max_ratio <= max_rel and l1_ratio <= l1_rel), max_ratio, l1_ratio
