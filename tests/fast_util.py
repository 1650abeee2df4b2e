"""FAST-mode tolerance measures shared by the GPU tests.

FAST keeps every bf16 rounding point of the lossless chain; what changes is
the binary32 value entering a rounding (hardware rsqrt, fused multiply-add).
One step of that value can become many steps of the output when the last
operation is an addition that cancels, so the bound is stated in steps of
the largest magnitude taking part in the last rounding: its inputs and its
result (for LN + modulate max(|p|, |shift|, |out|) with p = bf(n * bf(1 +
scale)); for RoPE max(|a c|, |b z|, |o|)).  Without cancellation that is
the output's own step, so the bound is the literal one; under cancellation
it is the inputs' step.  The fraction of elements within one literal step is
checked as it stands.
Sources: page "基于Agent的SGLang扩散模型Kernel优化实践", sections "质量分级机制"
(a lossless level and validated non-bit-exact levels) and "SGLang扩散Kernel的
验证流程" (tolerance checks for kernels that are not bit-exact).
"""
import numpy as np

import oracle
from exact import ulp_distance, value_of_bf16
from gpu_util import is_nan_bits, say


def bf16_step(v):
    """Size of one bf16 step at magnitude |v| (normal range)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def report(name, fast, lossless, scale_mag=None):
    """(literal max steps, fraction within one literal step, max error in
    steps of max(scale_mag, |lossless|)) over the elements that are not NaN
    on either side."""
    ok = ~(is_nan_bits(fast) | is_nan_bits(lossless))
    assert np.array_equal(is_nan_bits(fast), is_nan_bits(lossless)), name + ": NaN positions"
    d = ulp_distance(fast[ok], lossless[ok])
    frac1 = float((d <= 1).mean()) if d.size else 1.0
    lit = int(d.max()) if d.size else 0
    if scale_mag is None:
        scaled = float(lit)
    else:
        lv = value_of_bf16(lossless[ok])
        err = np.abs(value_of_bf16(fast[ok]) - lv)
        mag = np.maximum(np.asarray(scale_mag)[ok], np.abs(lv))
        scaled = float((err / bf16_step(mag)).max()) if d.size else 0.0
    say(f"FAST {name}: literal max {lit} steps, <=1 step {100 * frac1:.4f}%, "
        f"max in steps of the last rounding's input {scaled:.3f}")
    return lit, frac1, scaled


def ln_last_magnitude(x, scale, shift, eps):
    """max(|p|, |shift|) per element of LN + modulate (lossless chain), p =
    bf(n * bf(1 + scale)); x [rows, D]; scale, shift [rows, D] (the
    modulation row of each row)."""
    mag = np.empty(x.shape)
    for r in range(x.shape[0]):
        n, _ = oracle.ln_row(x[r], eps)
        s1 = value_of_bf16(oracle.one_plus(scale[r]))
        p = value_of_bf16(oracle.bf16_round(value_of_bf16(n) * s1))
        mag[r] = np.maximum(np.abs(p), np.abs(value_of_bf16(shift[r])))
    return mag


def tanh_last_magnitude(x, residual, w, gate, eps):
    """max(|residual|, |q|) per element of RMSNorm-tanh-residual (lossless
    chain), q = bf(tanh(gate) * y2); gate [rows, D] per row."""
    mag = np.empty(x.shape)
    for r in range(x.shape[0]):
        y2, _ = oracle.rms_row(x[r], w, eps)
        tau = value_of_bf16(oracle.tanh_bf16(gate[r]))
        q = value_of_bf16(oracle.bf16_round(tau * value_of_bf16(y2)))
        mag[r] = np.maximum(np.abs(q), np.abs(value_of_bf16(residual[r])))
    return mag
