"""Number formats used at the oracle's edges.

bf16 values enter as uint16 bit patterns and are widened exactly to float64.
The forward outputs handed to the GPU are O rounded to bf16 and LSE rounded to
float32, both round-to-nearest-even (IEEE default; the pages fix no rounding).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even); return uint16 bits.

    Done in two exact-by-construction steps on the float64 value: find the bf16
    spacing at x's binade and round x / spacing to the nearest integer with
    NumPy's round-half-to-even.  Handles zero, subnormal bf16, inf and NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat = x.reshape(-1)
    res = out.reshape(-1)
    finite = np.isfinite(flat)
    # magnitudes beyond the largest bf16 round to inf once past the halfway point
    big = np.float64(np.float32(3.3895313892515355e38))       # 0x7F7F as float
    a = np.abs(flat)
    # bf16 has 8 significant bits; exponent range equals float32's
    _, ex = np.frexp(np.where(a > 0, a, 1.0))                  # a = m * 2**ex, m in [0.5, 1)
    e = np.maximum(ex.astype(np.float64) - 1.0, -126.0)        # binade; subnormal spacing floor
    ulp = np.exp2(e - 7.0)
    q = np.round(a / ulp) * ulp                                # half-to-even on the grid
    overflow = q > big
    with np.errstate(over="ignore", invalid="ignore"):
        q32 = q.astype(np.float32)                             # exact: q is a bf16 value
    bits = (q32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[overflow] = 0x7F80
    sign = np.signbit(flat)
    bits = np.where(sign, bits | np.uint16(0x8000), bits).astype(np.uint16)
    res[:] = bits
    res[~finite & np.isinf(flat) & ~sign] = 0x7F80
    res[~finite & np.isinf(flat) & sign] = 0xFF80
    res[np.isnan(flat)] = 0x7FC0
    return out


def round_to_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> float32, round-to-nearest-even (NumPy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)
