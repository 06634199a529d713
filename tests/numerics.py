"""Test-side numerics: exact rational rounding and the parity tolerances.

Nothing here is imported by the oracle or by the product path.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


# ---------------------------------------------------------------- exact rounding
def round_to_binary(v: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Round the rational v to the nearest binary float with ``mant_bits``
    significand bits (implicit bit included) and minimum normal exponent emin
    (subnormals below), ties to even.  No overflow handling (tests stay in range)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (mant_bits - 1))
    q = a / quantum
    lo = q.numerator // q.denominator
    rem = q - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * quantum


def rne_f32(v: Fraction) -> Fraction:
    return round_to_binary(v, 24, -126)


def rne_bf16(v: Fraction) -> Fraction:
    return round_to_binary(v, 8, -126)


def bf16_bits_of(v: Fraction) -> int:
    """bf16 bit pattern of an exactly representable value."""
    f = np.float32(float(v))
    assert Fraction(float(f)) == v
    return int(np.array([f], dtype=np.float32).view(np.uint32)[0] >> 16)


def bits_to_f64(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- tolerances
def bf16_ulp(r: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |r| (for |r| in [2^e, 2^(e+1)) it is 2^(e-7));
    the subnormal spacing 2^-133 below 2^-126."""
    a = np.abs(np.asarray(r, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.exp2(e - 7), 2.0 ** -133)


def bf16_within_ulps(got_bits, ref_bits, ulps: int = 1, floor=None):
    """Element mask: |got - ref| <= ulps * ulp_bf16(ref), or <= floor (optional
    per-element absolute allowance for cancellation)."""
    g = bits_to_f64(got_bits)
    r = bits_to_f64(ref_bits)
    ok = np.abs(g - r) <= ulps * bf16_ulp(r)
    if floor is not None:
        ok |= np.abs(g - r) <= floor
    return ok


def floored_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """|got - ref| / max(|ref|, rms over the row of ref): a relative error
    that stays well-conditioned where an entry of the row is near zero."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt((ref * ref).mean(axis=-1, keepdims=True))
    return np.abs(got - ref) / np.maximum(np.abs(ref), rms)


MIXES_REL_TOL = 1e-4      # mixes: floored relative error
COEF_ABS_TOL = 1e-5       # pre / post / comb: absolute error
