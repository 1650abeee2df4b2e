"""CPU check of the identity the E4M3 copy relies on: for a bf16 value x and
a binary32 scale s, (float)((double)x * (1 / (double)s)) equals the IEEE
binary32 quotient x / s bit for bit wherever that quotient is zero, infinite,
NaN or normal, and where it is subnormal both lie below 2^-10 with the same
sign (E4M3 code +0 or -0).  (Reason: x has at most 8 significant bits, so
x / s is never a binary32 midpoint and stays at least 2^-49 (relative) away
from every normal one, while the binary64 product errs by less than 2^-51.9.)

Every bf16 value against power-of-two scales and their neighbours across the
whole binary32 range, special scales and 1500 random bit patterns; numpy's
float32 division and float64 -> float32 conversion are IEEE (round to nearest
even, subnormals kept).
"""
import numpy as np

X = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)


def _scales():
    s = []
    for e in range(-149, 128):
        p = np.float32(np.ldexp(1.0, e))
        s += [p, np.nextafter(p, np.float32(0)), np.nextafter(p, np.float32(np.inf)),
              np.float32(3) * p, -p, np.float32(0.0173) * p]
    s += [np.float32(v) for v in (0.0, -0.0, np.inf, -np.inf, np.nan, 3.4028235e38, 448.0,
                                  0.0173, 3.1, 0.3, 179.2)]
    rng = np.random.default_rng(2024)
    s += list(rng.integers(0, 1 << 32, 1500, dtype=np.uint64).astype(np.uint32).view(np.float32))
    return np.array(s, dtype=np.float32)


def test_binary64_product_equals_ieee_binary32_quotient():
    with np.errstate(all="ignore"):
        for s in _scales():
            a = X / s                                             # IEEE binary32
            b = (X.astype(np.float64) * (1.0 / np.float64(s))).astype(np.float32)
            nan = np.isnan(a) | np.isnan(b)
            assert np.array_equal(np.isnan(a), np.isnan(b)), s
            sub = ~nan & (a != 0) & (np.abs(a) < np.float32(2.0 ** -126))
            same = ~nan & ~sub
            assert np.array_equal(a[same].view(np.uint32), b[same].view(np.uint32)), s
            assert np.all(np.abs(b[sub]) < 2.0 ** -10), s
            assert np.array_equal(np.signbit(a[sub]), np.signbit(b[sub])), s
