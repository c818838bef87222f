"""bf16 <-> fp32 conversions for the oracle (test infrastructure only).

bf16 values are carried as numpy uint16 bit patterns.

Rounding rule.  The pages name bf16 parameters and fp32 gradient reduction
(AIG6 §6.3.4; DTLM §11 on precision) but never say how the fp32 result is
rounded back to bf16.  The reading taken is IEEE-754's default: round to the
nearest representable bf16 value, ties to the one whose last mantissa bit is
0.  Infinities stay infinite, finite values that round past the largest bf16
become infinite (the carry walks into the exponent), subnormals are kept (no
flush to zero), and a NaN stays a NaN: its sign and top payload bits are kept
and the quiet bit is set.
"""

import numpy as np

_ABS = np.uint32(0x7FFFFFFF)
_INF_BITS = np.uint32(0x7F800000)


def bf16_to_f32(bits):
    """Widen bf16 bit patterns to fp32 values (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(values):
    """Round fp32 values to bf16 bit patterns, nearest-even (see module docstring).

    Written as the definition: keep the top 16 bits (the value truncated toward
    zero), look at the 16 discarded bits, and step one bf16 unit away from zero
    when they exceed half a unit, or equal half a unit and the kept part is odd.
    """
    bits = np.ascontiguousarray(np.asarray(values, dtype=np.float32)).view(np.uint32)
    kept = (bits >> np.uint32(16)).astype(np.uint32)
    dropped = bits & np.uint32(0xFFFF)
    half = np.uint32(0x8000)
    odd = (kept & np.uint32(1)) == 1
    step_up = (dropped > half) | ((dropped == half) & odd)
    out = kept + step_up.astype(np.uint32)
    is_nan = (bits & _ABS) > _INF_BITS
    out = np.where(is_nan, kept | np.uint32(0x0040), out)
    return out.astype(np.uint16)


def bf16_is_nan(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b & np.uint16(0x7FFF)) > np.uint16(0x7F80)


def bf16_ulp_distance(a, b):
    """Distance in units of the last place between two bf16 arrays.

    Bit patterns are mapped onto a monotone integer line (negative values
    mirrored), so +0 and -0 coincide.  Pairs where both sides are NaN count 0;
    a NaN against a non-NaN counts as a very large distance.
    """
    a = np.asarray(a, dtype=np.uint16).astype(np.int64)
    b = np.asarray(b, dtype=np.uint16).astype(np.int64)

    def line(x):
        mag = x & 0x7FFF
        return np.where(x & 0x8000, -mag, mag)

    d = np.abs(line(a) - line(b))
    na, nb = bf16_is_nan(a.astype(np.uint16)), bf16_is_nan(b.astype(np.uint16))
    d = np.where(na & nb, 0, d)
    d = np.where(na ^ nb, 1 << 30, d)
    return d
