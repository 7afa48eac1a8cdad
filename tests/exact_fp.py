"""Exact fp32 rounding helpers for tests: one correctly rounded fp32 result
per operation, computed without double rounding (test infrastructure; no
part of the method's arithmetic)."""
from fractions import Fraction

import numpy as np


def round_f32(q: Fraction) -> np.float32:
    """The fp32 value nearest to the rational q, ties to even (the candidates
    around q are compared exactly)."""
    f = np.float32(float(q))
    cands = [f, np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))]
    cands = [c for c in cands if np.isfinite(c)]
    best = min(abs(Fraction(float(c)) - q) for c in cands)
    near = [c for c in cands if abs(Fraction(float(c)) - q) == best]
    if len(near) == 1:
        return near[0]
    return [c for c in near if (int(np.array(c).view(np.uint32)) & 1) == 0][0]


def fma32(a, b, c) -> np.float32:
    return round_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def add32(a, b) -> np.float32:
    return round_f32(Fraction(float(a)) + Fraction(float(b)))


def fma32_vec(a, b, c) -> np.ndarray:
    """Elementwise fp32 fma(a, b, c), correctly rounded, for finite inputs
    whose result stays in the normal fp32 range. The product of two fp32
    values is exact in float64; p + c is rounded once to float64 as s, with
    the exact error e (two-sum). Rounding s to fp32 is then the correct
    rounding of p + c unless s lies exactly halfway between two fp32 values
    and e != 0, in which case the sign of e picks the neighbour."""
    a = np.asarray(a, np.float32).astype(np.float64)
    b = np.asarray(b, np.float32).astype(np.float64)
    c = np.asarray(c, np.float32).astype(np.float64)
    p = a * b
    s = p + c
    bb = s - p
    e = (p - (s - bb)) + (c - bb)  # two-sum: p + c == s + e exactly
    r = s.astype(np.float32)
    up = np.nextafter(r, np.float32(np.inf))
    dn = np.nextafter(r, np.float32(-np.inf))
    # s on the midpoint between r and up (rounded to r, the even one): the
    # exact value is above it when e > 0; on the midpoint between dn and r:
    # below it when e < 0. An fp32 midpoint is a float64 value, so rounding
    # to float64 never moves the value across one.
    on_up = s == (r.astype(np.float64) + up.astype(np.float64)) / 2
    on_dn = s == (r.astype(np.float64) + dn.astype(np.float64)) / 2
    r = np.where(on_up & (e > 0), up, r)
    r = np.where(on_dn & (e < 0), dn, r)
    return r.astype(np.float32)
