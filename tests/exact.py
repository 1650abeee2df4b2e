"""Exact reference arithmetic used by the oracle pins (test helpers, no oracle code).

``nearest_bf16`` rounds float64 values that are *exact* (the test makes sure
of that) to the nearest bfloat16 by comparing against the two neighbouring
bf16 values, ties to the one with an even last bit.  It works on magnitudes
and exponents only, unlike the oracle, which rounds binary32 with an integer
carry trick.  ``frac_bf16`` does the same with Python Fractions for values
that double cannot hold exactly.
"""
from fractions import Fraction
import math

import numpy as np

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bits_of_bf16_value(v: np.ndarray) -> np.ndarray:
    """bf16-representable float64 values -> bf16 bit patterns."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    assert np.all((f.astype(np.float64) == v) | np.isnan(v))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def value_of_bf16(h) -> np.ndarray:
    h = np.asarray(h, dtype=np.uint16)
    with np.errstate(invalid="ignore"):          # signalling-NaN patterns
        return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def nearest_bf16(v) -> np.ndarray:
    """Round exact float64 values to bf16 (nearest, ties to even); returns bits."""
    v = np.atleast_1d(np.asarray(v, dtype=np.float64))
    out = np.zeros(v.shape, dtype=np.float64)
    a = np.abs(v)
    fin = np.isfinite(v) & (a > 0)
    m, e = np.frexp(a[fin])                      # a = m * 2^e, m in [0.5, 1)
    ulp_exp = np.maximum(e - 8, -133)
    ulp = np.ldexp(np.ones_like(m), ulp_exp)
    below = np.floor(a[fin] / ulp) * ulp          # bf16 neighbour at or below
    above = below + ulp
    d_lo = a[fin] - below
    d_hi = above - a[fin]
    k = np.floor(a[fin] / ulp)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (np.mod(k, 2) == 1))
    r = np.where(pick_hi, above, below)
    r = np.where(r > BF16_MAX, np.inf, r)
    out[fin] = np.copysign(r, v[fin])
    out[~fin] = v[~fin]                           # zeros, infinities, NaN
    bits = np.empty(v.shape, dtype=np.uint16)
    ok = ~np.isnan(out)
    bits[ok] = bits_of_bf16_value(out[ok])
    bits[~ok] = 0x7FC0
    return bits


def frac_bf16(x: Fraction) -> int:
    """Nearest bf16 (ties to even) of an exact rational; returns bits."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp_exp = max(e - 7, -133)
    ulp = Fraction(2) ** ulp_exp
    k = a // ulp
    rem = a - k * ulp
    if rem * 2 > ulp or (rem * 2 == ulp and k % 2 == 1):
        k += 1
    r = k * ulp
    if r > Fraction(BF16_MAX):
        return sign | 0x7F80
    return sign | int(bits_of_bf16_value(np.array([float(r)]))[0])


def ulp_distance(a_bits, b_bits) -> np.ndarray:
    """Distance in bf16 steps on the monotone integer line (+0 and -0 both map to 0)."""
    def mono(h):
        h = np.asarray(h, dtype=np.int64)
        mag = h & 0x7FFF
        return np.where(h & 0x8000, -mag, mag)
    return np.abs(mono(a_bits) - mono(b_bits))
