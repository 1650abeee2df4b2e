"""Pins of the CPU oracle against facts fixed outside it (CPU only).

The oracle defines the epilogues' results; these tests tie it to the
mathematics: exhaustive sweeps of every single-input bf16 step, exact rational
rounding of products and sums, closed forms of LayerNorm / RMSNorm / RoPE,
invariants, and float64 brute force on small rows.  A plausible slip in the
oracle (a dropped term or rounding, a wrong sign, index or operand) fails at
least one of them.

Sources: the AdaLN rounding points come from page "基于Agent的SGLang扩散模型
Kernel优化实践" (tahou.com), section "数学等价不代表结果完全一致"; the native bf16
RMSNorm chain from page "#34085 [diffusion] Clean up kernels and shared fast
paths", section "关键源码片段"; the QKV epilogue steps from the first page,
section "合并QKV投影时的数值问题".
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle
from exact import (frac_bf16, nearest_bf16, ulp_distance, value_of_bf16)
from modulation_bf16_row_amd import synth

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _finite16():
    v = value_of_bf16(ALL16)
    return ALL16[np.isfinite(v)]


# --------------------------------------------------------------------------------------
# bf16 conversion
# --------------------------------------------------------------------------------------

def test_bf16_round_all_binary32_vs_torch():
    """All 2^32 binary32 inputs: the oracle's integer rounding equals torch's
    CPU float->bfloat16 conversion (round to nearest even); NaN stays NaN."""
    step = 1 << 24
    for first in range(0, 1 << 32, step):
        got = oracle.bf16_round_bits_range(first, step)
        f = (np.arange(first, first + step, dtype=np.uint64).astype(np.uint32)).view(np.float32)
        ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(f)
        assert np.array_equal(got[~nan], ref[~nan]), hex(first)
        g = got[nan]
        assert np.all((g & 0x7F80) == 0x7F80) and np.all(g & 0x0040)


def test_bf16_round_edges_vs_fractions():
    """Ties, near-ties, subnormals and the overflow boundary against exact
    rational rounding."""
    cases = []
    for base in (0x3F800000, 0x3F810000, 0x00010000, 0x00000001, 0x007F8000, 0x7F7F0000,
                 0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0x80018000, 0xBF808000, 0x3F808001):
        for d in (-1, 0, 1, 0x7FFF, 0x8000, 0x8001):
            cases.append((base + d) & 0xFFFFFFFF)
    f = np.array(cases, dtype=np.uint32).view(np.float32)
    got = oracle.bf16_round(f)
    for v, g in zip(f, got):
        if not np.isfinite(v):
            continue
        assert g == frac_bf16(Fraction(float(v))), (float(v), hex(int(g)))


def test_bf16_round_f64_vs_fractions():
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 128, 3000)))
    vals += [2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -126 * (1 - 2 ** -9),
             1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -40, -(1 + 2 ** -8),
             (2 - 2 ** -8) * 2.0 ** 127, (2 - 2 ** -8 - 2 ** -30) * 2.0 ** 127, 0.999, 1e-300]
    for v in vals:
        assert oracle.bf16_round_f64(v) == frac_bf16(Fraction(v)), v
    # on binary32 inputs the two oracle roundings agree
    f = rng.standard_normal(10000).astype(np.float32)
    assert all(oracle.bf16_round_f64(float(x)) == oracle.bf16_round(x)[()] for x in f[:2000])


# --------------------------------------------------------------------------------------
# declared reduction order
# --------------------------------------------------------------------------------------

def test_sum_wave_exact_for_integer_terms():
    """Integer terms whose partial sums stay below 2^24 sum exactly in any
    order: a dropped or doubled element changes the result."""
    rng = np.random.default_rng(1)
    for D in (8, 16, 64, 520, 1024, 3072, 5120, 8192):
        t = rng.integers(-1000, 1000, D).astype(np.float32)
        assert oracle.sum_wave(t) == np.float32(t.astype(np.int64).sum()), D


def test_sum_wave_small_rows_reduce_to_folds():
    """D = 8: only lane 0 holds data, so R is a left fold from +0.
    D = 16: lanes 0 and 1 each fold 8 terms, then add once."""
    rng = np.random.default_rng(2)
    for _ in range(200):
        t = (rng.standard_normal(16) * np.exp2(rng.integers(-20, 20, 16))).astype(np.float32)
        f8 = np.float32(0)
        for v in t[:8]:
            f8 = np.float32(f8 + v)
        assert oracle.sum_wave(t[:8]) == f8
        g = np.float32(0)
        for v in t[8:]:
            g = np.float32(g + v)
        assert oracle.sum_wave(t) == np.float32(f8 + g)


def test_sum_wave_order_sensitive_case():
    """D = 1024, t[0] = 2^24, all other terms 1.  Lane 0 keeps 2^24 (each +1 is
    a tie that rounds to even); every other lane sums 16 ones exactly; the
    butterfly adds 63 * 16 = 1008 exactly.  A plain left-to-right sum would
    give 2^24 instead."""
    t = np.ones(1024, dtype=np.float32)
    t[0] = 2.0 ** 24
    assert oracle.sum_wave(t) == np.float32(2.0 ** 24 + 1008)
    # the same large term in lane 1 (element 8): lane 1 keeps 2^24, lane 0 has 16
    t = np.ones(1024, dtype=np.float32)
    t[8] = 2.0 ** 24
    assert oracle.sum_wave(t) == np.float32(2.0 ** 24 + 1008)
    # ... but placed as the last element of lane 0's second chunk, lane 0 first
    # sums 15 ones (=15) and then adds 2^24: 2^24 + 15 rounds to 2^24 + 16.
    t = np.ones(1024, dtype=np.float32)
    t[519] = 2.0 ** 24
    assert oracle.sum_wave(t) == np.float32(2.0 ** 24 + 16 + 1008)


def test_sum_head():
    rng = np.random.default_rng(3)
    t = (rng.standard_normal(8)).astype(np.float32)
    f = np.float32(0)
    for v in t:
        f = np.float32(f + v)
    assert oracle.sum_head(t) == f
    ti = rng.integers(-100, 100, 128).astype(np.float32)
    assert oracle.sum_head(ti) == np.float32(ti.sum())


# --------------------------------------------------------------------------------------
# single-input bf16 steps, exhaustively
# --------------------------------------------------------------------------------------

def test_one_plus_exhaustive_vs_fractions():
    h = _finite16()
    got = oracle.one_plus(h)
    v = value_of_bf16(h)
    for hi, vi, gi in zip(h, v, got):
        assert gi == frac_bf16(1 + Fraction(float(vi))), (hex(int(hi)), hex(int(gi)))


def test_one_plus_specials():
    assert oracle.one_plus(np.array([0x7F80, 0xFF80, 0x7FC0], dtype=np.uint16)).tolist()[:2] == \
        [0x7F80, 0xFF80]
    assert oracle.one_plus(np.array([0xBF80], dtype=np.uint16))[0] == 0x0000  # 1 + (-1) = +0


def test_tanh_exhaustive_vs_long_double():
    """All 65536 gates: double tanh rounded once equals long double tanh rounded
    once, and no value is within 2^-40 (relative) of a bf16 rounding boundary,
    so the correctly rounded result is unambiguous."""
    got = oracle.tanh_bf16(ALL16)
    ref, margin = oracle.tanh_check_ld(ALL16)
    v = value_of_bf16(ALL16)
    fin = np.isfinite(v)
    assert np.array_equal(got[fin], ref[fin])
    nz = fin & (v != 0)
    assert margin[nz].min() > 2.0 ** -40


def test_tanh_properties():
    v = value_of_bf16(ALL16)
    t = oracle.tanh_bf16(ALL16)
    tv = value_of_bf16(t)
    fin = np.isfinite(v)
    # odd symmetry, bound, sign
    neg = ALL16 ^ np.uint16(0x8000)
    assert np.array_equal(oracle.tanh_bf16(neg)[fin], t[fin] ^ np.uint16(0x8000))
    assert np.all(np.abs(tv[fin]) <= 1.0)
    assert np.all(np.sign(tv[fin]) == np.sign(v[fin]))
    # monotone in the input
    order = np.argsort(v[fin], kind="stable")
    assert np.all(np.diff(tv[fin][order]) >= 0)
    # closed forms: +-0, +-inf, NaN, saturation, tiny inputs
    assert t[0x0000] == 0x0000 and t[0x8000] == 0x8000
    assert t[0x7F80] == 0x3F80 and t[0xFF80] == 0xBF80
    assert (t[0x7FC0] & 0x7F80) == 0x7F80 and (t[0x7FC0] & 0x7F)
    big = fin & (np.abs(v) >= 4.0)
    assert np.all(tv[big] == np.sign(v[big]))
    tiny = fin & (np.abs(v) <= 2.0 ** -6)
    assert np.array_equal(t[tiny], ALL16[tiny])
    # against float64 tanh within half a bf16 ulp (pins the sign and scale of the rounding)
    mid = fin & (np.abs(v) > 0)
    err = np.abs(tv[mid] - np.tanh(v[mid]))
    ulp = np.exp2(np.floor(np.log2(np.abs(tv[mid]))) - 7)
    assert np.all(err <= 0.5 * ulp * (1 + 1e-9))


def test_rms_rstd_exhaustive():
    """rstd = bf(1 / sqrt(v)) with binary32 sqrt and division, each correctly
    rounded.  float64 sqrt and division, rounded to binary32, are correctly
    rounded too (53 >= 2*24 + 2), which gives an independent evaluation."""
    h = _finite16()
    v = value_of_bf16(h)
    pos = v > 0
    got = oracle.rms_rstd(h[pos])
    s32 = np.sqrt(v[pos]).astype(np.float32)
    q32 = (1.0 / s32.astype(np.float64)).astype(np.float32)
    ref = nearest_bf16(q32.astype(np.float64))
    assert np.array_equal(got, ref)
    # closed forms: v = 4^k -> 2^-k exactly
    for k in range(-60, 60):
        hv = nearest_bf16(np.array([4.0 ** k]))[0]
        assert value_of_bf16(oracle.rms_rstd(np.array([hv])))[0] == 2.0 ** -k
    # zero -> +inf, negative -> NaN
    r = oracle.rms_rstd(np.array([0x0000, 0xBF80], dtype=np.uint16))
    assert r[0] == 0x7F80 and (r[1] & 0x7F80) == 0x7F80 and (r[1] & 0x7F)


# --------------------------------------------------------------------------------------
# two-operand rounding points, by exact arithmetic
# --------------------------------------------------------------------------------------

def _rand_bf16(rng, n, spread=10):
    v = rng.standard_normal(n) * np.exp2(rng.integers(-spread, spread, n))
    return nearest_bf16(v)


def test_residual_gate_add_exact():
    """out = bf(residual + bf(gate * y)): the product of two bf16 values and the
    sum of two bf16 values are exact in float64 here, so one nearest rounding
    of each gives the answer."""
    rng = np.random.default_rng(11)
    rows, D = 64, 256
    res = _rand_bf16(rng, rows * D, 6).reshape(rows, D)
    y = _rand_bf16(rng, rows * D, 6).reshape(rows, D)
    gate = _rand_bf16(rng, 4 * D, 6).reshape(4, D)
    out = oracle.residual_gate_add(res, y, gate)
    g_full = np.repeat(gate, rows // 4, axis=0)          # mod row = r // 16
    gy = value_of_bf16(nearest_bf16(value_of_bf16(g_full) * value_of_bf16(y)))
    s = value_of_bf16(res) + gy
    assert np.all((s - value_of_bf16(res)) == gy)       # the float64 sum is exact
    assert np.array_equal(out, nearest_bf16(s).reshape(rows, D))


def test_residual_gate_add_wide_exponents_fractions():
    rng = np.random.default_rng(12)
    res = _rand_bf16(rng, 512, 60).reshape(2, 256)
    y = _rand_bf16(rng, 512, 60).reshape(2, 256)
    gate = _rand_bf16(rng, 256, 60).reshape(1, 256)
    out = oracle.residual_gate_add(res, y, gate)
    for r in range(2):
        for i in range(256):
            gy = frac_bf16(Fraction(float(value_of_bf16(gate[0, i]))) *
                           Fraction(float(value_of_bf16(y[r, i]))))
            gyv = value_of_bf16(gy)
            if not np.isfinite(gyv):
                continue
            ref = frac_bf16(Fraction(float(value_of_bf16(res[r, i]))) + Fraction(float(gyv)))
            assert out[r, i] == ref


# --------------------------------------------------------------------------------------
# LayerNorm + AdaLN modulate
# --------------------------------------------------------------------------------------

def test_ln_constant_row_gives_shift():
    """x_i = c: the mean is c exactly, every deviation is +0, so n = +0 and
    out = shift bitwise (shift != 0)."""
    rng = np.random.default_rng(21)
    for D in (8, 520, 1024, 3072):
        for c in (0.5, -3.25, 1000.0, 1.0e-30, 7.5e4):
            x = synth.constant_bf16((3, D), c)
            scale = synth.normal_bf16((1, D), 0.1, 1)
            shift = synth.normal_bf16((1, D), 0.1, 2)
            shift[shift & 0x7FFF == 0] = 0x3F80
            out = oracle.ln_modulate(x, scale, shift)
            assert np.array_equal(out, np.repeat(shift, 3, axis=0)), (D, c)
    del rng


def test_ln_scale_zero_shift_negzero_is_plain_ln():
    """scale = 0 gives 1 + scale = 1; shift = -0 adds nothing (x + (-0) = x),
    so the output is the plain LayerNorm n bitwise."""
    x = synth.normal_bf16((16, 1024), 1.0, 31)
    scale = np.zeros((1, 1024), dtype=np.uint16)
    shift = np.full((1, 1024), 0x8000, dtype=np.uint16)
    out = oracle.ln_modulate(x, scale, shift)
    for r in range(16):
        n, _ = oracle.ln_row(x[r], 1e-6)
        assert np.array_equal(out[r], n)


def test_ln_scale_minus_one_gives_shift():
    x = synth.normal_bf16((8, 512), 1.0, 32)
    scale = np.full((1, 512), 0xBF80, dtype=np.uint16)        # -1
    shift = synth.normal_bf16((1, 512), 0.1, 33)
    shift[shift & 0x7FFF == 0] = 0x3F80
    assert np.array_equal(oracle.ln_modulate(x, scale, shift), np.repeat(shift, 8, axis=0))


def test_ln_normalizes_by_multiplying_with_rho():
    """LayerNorm normalizes as d * rho with rho = 1 / sqrt(var + eps) rounded
    to binary32 first (the "RSQ path" of page "基于Agent的SGLang扩散模型Kernel
    优化实践", section "数学等价不代表结果完全一致"), not as d / sqrt(var + eps).
    Hand-derived row, D = 8, eps = 1e-6 (binary32 0x358637BD):
    x = (p, -p, q, -q, r, -r, s, -s) with p, q, r, s = 1.046875, 1.9453125,
    1.6953125, 1.078125.  The mean is exactly 0 and d = x; the squares are
    exact and sum to 17.83325195..., so var = 2.229156494140625 (0x400EAA80)
    exactly; var + eps rounds to 0x400EAA84; its square root to
    sigma = 0x3FBF1BD0; rho = 1 / sigma to 0x3F2B7672.  For d = p:
    p * rho = 0x3F337FFF, just below the bf16 midpoint 0.701171875 =
    0x3F338000, so n = 0x3F33 (0.69921875), which is also where the exact
    p / sqrt(var + eps) = 0.70117182... lies.  Dividing instead, p / sigma
    rounds to the midpoint itself and then to the even 0x3F34."""
    x = np.array([0x3F86, 0xBF86, 0x3FF9, 0xBFF9, 0x3FD9, 0xBFD9, 0x3F8A, 0xBF8A], np.uint16)
    xv = value_of_bf16(x)
    assert list(xv[::2]) == [1.046875, 1.9453125, 1.6953125, 1.078125]
    var = sum(Fraction(float(v)) ** 2 for v in xv) / 8
    assert var == Fraction(2.229156494140625)
    f = np.float32
    sig = np.sqrt(f(2.229156494140625) + f(1e-6))
    assert sig.view(np.uint32) == 0x3FBF1BD0
    rho = f(1) / sig
    assert rho.view(np.uint32) == 0x3F2B7672
    assert (f(xv[0]) * rho).view(np.uint32) == 0x3F337FFF
    assert (f(xv[0]) / sig).view(np.uint32) == 0x3F338000          # the other reading
    n, (mu, v, r) = oracle.ln_row(x, 1e-6)
    assert mu == 0 and v == np.float32(2.229156494140625) and r == rho
    assert n[0] == 0x3F33 and n[1] == 0xBF33


def _ln_double(xv, eps):
    mu = xv.mean()
    var = ((xv - mu) ** 2).mean()
    return (xv - mu) / np.sqrt(var + eps), var


@pytest.mark.parametrize("D", [8, 16, 64, 512, 520, 1024, 3072])
def test_ln_row_vs_double(D):
    """LayerNorm in float64, rounded once: the oracle's n is within 1 bf16 ulp
    everywhere and equal on >= 99% of elements."""
    rng = np.random.default_rng(40 + D)
    rows = max(2, 20000 // D)
    x = nearest_bf16(rng.standard_normal((rows, D)) * 1.7 + 0.3).reshape(rows, D)
    # half the rows have a variance comparable to eps, where eps must count
    x[rows // 2:] = nearest_bf16(rng.standard_normal((rows - rows // 2, D)) * 1e-3).reshape(-1, D)
    tot = eq = 0
    for r in range(rows):
        n, (mu, var, rho) = oracle.ln_row(x[r], 1e-6)
        ref_v, var_d = _ln_double(value_of_bf16(x[r]), 1e-6)
        ref = nearest_bf16(ref_v)
        d = ulp_distance(n, ref)
        assert d.max() <= 1, (D, r)
        eq += int((d == 0).sum())
        tot += D
        assert abs(var - var_d) <= 1e-5 * var_d
    assert eq / tot >= 0.99


def test_ln_invariants():
    """Before modulation: mean(n) ~ 0 and var(n) ~ var/(var+eps); rows whose
    variance is far below eps come out near zero."""
    for seed, (mean, std) in enumerate([(0, 1), (1000, 1), (0, 1e-2), (-5, 30)]):
        x = synth.normal_bf16((8, 3072), std, 50 + seed, mean=mean)
        for r in range(8):
            n, (mu, var, rho) = oracle.ln_row(x[r], 1e-6)
            nv = value_of_bf16(n)
            assert abs(nv.mean()) <= 2.0 ** -9 * np.abs(nv).mean() + 1e-3
            assert abs(nv.var() - var / (var + 1e-6)) <= 2.0 ** -7
    x = synth.normal_bf16((4, 1024), 1e-5, 60, mean=1.0)  # bf16 rounds most to 1.0
    for r in range(4):
        n, (_, var, _) = oracle.ln_row(x[r], 1e-6)
        assert var < 1e-6
        assert np.abs(value_of_bf16(n)).max() < 1.0


def test_ln_modulate_composition_and_mod_rows():
    """Per-batch and per-token modulation: row r uses mod row r // (rows /
    mod_rows); given n, the three roundings are exact float64 products/sums
    rounded once."""
    rng = np.random.default_rng(70)
    for rows, mod_rows in ((12, 1), (12, 3), (12, 12)):
        D = 520
        x = nearest_bf16(rng.standard_normal((rows, D))).reshape(rows, D)
        scale = nearest_bf16(rng.standard_normal((mod_rows, D)) * 0.1).reshape(mod_rows, D)
        shift = nearest_bf16(rng.standard_normal((mod_rows, D)) * 0.1).reshape(mod_rows, D)
        out = oracle.ln_modulate(x, scale, shift)
        per = rows // mod_rows
        for r in range(rows):
            m = r // per
            n, _ = oracle.ln_row(x[r], 1e-6)
            s1 = nearest_bf16(1.0 + value_of_bf16(scale[m]))
            p = nearest_bf16(value_of_bf16(n) * value_of_bf16(s1))
            ref = nearest_bf16(value_of_bf16(p) + value_of_bf16(shift[m]))
            assert np.array_equal(out[r], ref), (rows, mod_rows, r)


def test_ln_strided_rows():
    x_full = synth.normal_bf16((6, 1100), 1.0, 80)
    x = x_full[:, :1024]
    scale = synth.normal_bf16((2, 1024), 0.1, 81)
    shift = synth.normal_bf16((2, 1024), 0.1, 82)
    assert np.array_equal(oracle.ln_modulate(x, scale, shift),
                          oracle.ln_modulate(np.ascontiguousarray(x), scale, shift))


# --------------------------------------------------------------------------------------
# native bf16 RMSNorm chain
# --------------------------------------------------------------------------------------

def test_rms_constant_power_of_two_rows():
    """x = +-2^k (k >= -5): squares, their mean and mean + eps are exactly 4^k
    in bf16, rstd = 2^-k, y1 = +-1, so out = bf(+-w * scale)."""
    rng = np.random.default_rng(90)
    D = 1024
    w = synth.uniform_bf16((D,), 0.5, 1.5, 91)
    scale = synth.normal_bf16((1, D), 0.1, 92)
    for k in (-5, -2, 0, 3, 10):
        for sgn in (1.0, -1.0):
            x = synth.constant_bf16((2, D), sgn * 2.0 ** k)
            out = oracle.rmsnorm_scale(x, w, scale)
            ref = nearest_bf16(sgn * value_of_bf16(w) * value_of_bf16(scale[0]))
            assert np.array_equal(out[0], ref) and np.array_equal(out[1], ref)
    del rng


def test_rms_rounded_squares_closed_form():
    """Row alternating 1 and 1.0703125 (= 1 + 9/128), D = 1024.  The squares
    round to 1 and 1.1484375 (147/128; the exact 1.14556884765625 is 146.63
    steps of 2^-7).  Their sum 512 * 2.1484375 = 1100 is exact, 1100/1024 =
    1.07421875 = 137.5/128 is a tie that rounds to the even 138/128 =
    1.078125.  Without the rounding of the squares the mean square would be
    1.072784423828125, which rounds to 1.0703125."""
    D = 1024
    x = np.empty(D, dtype=np.uint16)
    x[0::2] = 0x3F80                      # 1.0
    x[1::2] = 0x3F89                      # 1.0703125
    assert value_of_bf16(np.array([0x3F89]))[0] == 1.0703125
    w = np.full(D, 0x3F80, dtype=np.uint16)
    _, (ms, v, rstd) = oracle.rms_row(x, w, 1e-6)
    assert ms == np.float32(1.078125)
    assert v == np.float32(1.078125)      # eps is below half a bf16 step here
    # 1/sqrt(1.078125) = 0.96309...; the bf16 steps near it are 2^-8 apart:
    # 246/256 = 0.9609375 and 247/256 = 0.96484375; 0.96309 is 246.55 steps.
    assert rstd == np.float32(0.96484375)
    # The same row scaled by 2^-9 (exact in bf16): ms = 1.078125 * 2^-18.
    # Adding eps = 1e-6 (binary32 9.99999997e-7) gives 5.11272e-6, which is
    # 171.55 steps of 2^-25, so v = 172 * 2^-25.  Had ms not been rounded
    # (1.07421875 * 2^-18), v would be 171.05 steps -> 171 * 2^-25.
    x[0::2] = 0x3B00                      # 2^-9
    x[1::2] = 0x3B09                      # 1.0703125 * 2^-9
    _, (ms, v, rstd) = oracle.rms_row(x, w, 1e-6)
    assert ms == np.float32(1.078125 * 2.0 ** -18)
    assert v == np.float32(172 * 2.0 ** -25)


def test_rms_y1_rounded_before_the_weight():
    """y1 = bf(x * rstd) is rounded before the weight multiplies it (page
    "#34085 [diffusion] Clean up kernels and shared fast paths", section
    "关键源码片段": the normalized row is cast to bf16, then multiplied by the
    weight).  The row of test_rms_rounded_squares_closed_form has rstd =
    247/256.  For x = 137/128 (1.0703125): x * rstd = 33839/32768 =
    132.18 steps of 2^-7, so y1 = 132/128.  With w = 255/128 (1.9921875):
    y1 * w = 33660/16384 = 131.48 steps of 2^-6, so y2 = 131/64 (0x4003);
    without the rounding of y1, 33839 * 255 / 2^22 = 131.67 steps gives
    132/64 (0x4004).  For x = 1: x * rstd = 247/256 is exact and
    y2 = bf(247 * 255 / 2^15) = 246/128 (0x3FF6) either way."""
    D = 1024
    x = np.empty(D, dtype=np.uint16)
    x[0::2] = 0x3F80
    x[1::2] = 0x3F89
    w = np.full(D, 0x3FFF, dtype=np.uint16)
    assert value_of_bf16(np.array([0x3FFF]))[0] == 255 / 128
    y1 = Fraction(137, 128) * Fraction(247, 256)
    assert frac_bf16(y1) == 0x3F84                                   # 132/128
    assert frac_bf16(Fraction(132, 128) * Fraction(255, 128)) == 0x4003
    assert frac_bf16(y1 * Fraction(255, 128)) == 0x4004              # the other reading
    y2, (_, _, rstd) = oracle.rms_row(x, w, 1e-6)
    assert rstd == np.float32(247 / 256)
    assert np.all(y2[1::2] == 0x4003) and np.all(y2[0::2] == 0x3FF6)
    scale = np.full((1, D), 0x3F80, dtype=np.uint16)
    out = oracle.rmsnorm_scale(x[None], w, scale)
    assert np.array_equal(out[0], y2)


def test_rms_rstd_taken_from_the_rounded_mean_square_plus_eps():
    """rstd is computed from v = bf(ms + eps), the bf16 value of the sum (page
    "#34085 [diffusion] Clean up kernels and shared fast paths", section
    "关键源码片段": the mean square plus eps is cast to bf16 before the rsqrt).
    Constant row x = 2^-14, D = 1024, eps = 1e-6 (binary32 0x358637BD):
    squares 2^-28 (exact), ms = 2^-28; ms + eps = 1.00372529e-6 (0x3586B7BD)
    = 134.72 steps of 2^-27, so v = 135 * 2^-27 (bf16 0x3587).  1/sqrt(v) =
    997.10 rounds to 996 (bf16 steps of 4 in [512, 1024)), and y1 =
    996 * 2^-14 = 249 * 2^-12 (0x3D79).  Taken from the unrounded sum,
    1/sqrt(1.00372529e-6) = 998.14 would round to 1000, y1 = 0x3D7A."""
    D = 1024
    x = np.full(D, 0x3880, dtype=np.uint16)
    assert value_of_bf16(x[:1])[0] == 2.0 ** -14
    w = np.full(D, 0x3F80, dtype=np.uint16)
    f = np.float32
    s = f(2.0 ** -28) + f(1e-6)
    assert s.view(np.uint32) == 0x3586B7BD
    assert frac_bf16(Fraction(float(s))) == 0x3587
    v = Fraction(135, 2 ** 27)
    assert frac_bf16(Fraction(float(f(1) / np.sqrt(f(float(v)))))) == 0x4479   # 996
    assert frac_bf16(Fraction(float(f(1) / np.sqrt(s)))) == 0x447A             # 1000
    y2, (ms, vv, rstd) = oracle.rms_row(x, w, 1e-6)
    assert ms == np.float32(2.0 ** -28) and vv == np.float32(float(v)) and rstd == 996
    assert np.all(y2 == 0x3D79)


def test_rms_chain_near_ideal_and_unit_rms():
    """Against float64 RMSNorm the chain (five bf16 roundings) stays within 3
    ulp; with w = 1, mean(y1^2) is 1 within 3 * 2^-8.  Intermediates are bf16
    values (ms, ms + eps, rstd)."""
    rng = np.random.default_rng(93)
    for D in (8, 64, 1024, 3072):
        x = nearest_bf16(rng.standard_normal((4, D)) * 0.8).reshape(4, D)
        # rows whose mean square is comparable to eps, where eps must count
        x[2:] = nearest_bf16(rng.standard_normal((2, D)) * 1e-3).reshape(2, D)
        w = nearest_bf16(rng.uniform(0.5, 1.5, D))
        ones = np.full(D, 0x3F80, dtype=np.uint16)
        for r in range(4):
            xv = value_of_bf16(x[r])
            y2, (ms, v, rstd) = oracle.rms_row(x[r], w, 1e-6)
            for s in (ms, v, rstd):
                assert nearest_bf16(np.array([float(s)]))[0] == \
                    nearest_bf16(np.array([float(np.float32(s))]))[0]
                assert value_of_bf16(nearest_bf16(np.array([float(s)])))[0] == float(s)
            ideal = xv / np.sqrt((xv ** 2).mean() + 1e-6) * value_of_bf16(w)
            assert ulp_distance(y2, nearest_bf16(ideal)).max() <= 3
            if r < 2:
                y1, _ = oracle.rms_row(x[r], ones, 1e-6)
                assert abs((value_of_bf16(y1) ** 2).mean() - 1) <= 3 * 2.0 ** -8


def test_rmsnorm_scale_composition():
    rng = np.random.default_rng(94)
    rows, D = 12, 1024
    x = nearest_bf16(rng.standard_normal((rows, D))).reshape(rows, D)
    w = nearest_bf16(rng.uniform(0.5, 1.5, D))
    scale = nearest_bf16(rng.standard_normal((3, D)) * 0.1).reshape(3, D)
    out = oracle.rmsnorm_scale(x, w, scale)
    for r in range(rows):
        y2, _ = oracle.rms_row(x[r], w, 1e-6)
        ref = nearest_bf16(value_of_bf16(y2) * value_of_bf16(scale[r // 4]))
        assert np.array_equal(out[r], ref)


def test_rmsnorm_tanh_residual_closed_forms():
    rng = np.random.default_rng(95)
    rows, D = 8, 1024
    x = nearest_bf16(rng.standard_normal((rows, D))).reshape(rows, D)
    res = nearest_bf16(rng.standard_normal((rows, D))).reshape(rows, D)
    res[res & 0x7FFF == 0] = 0x3F80
    w = nearest_bf16(rng.uniform(0.5, 1.5, D))
    # gate = 0 -> tanh = +0 -> out = residual (nonzero residual)
    zero = np.zeros((1, D), dtype=np.uint16)
    assert np.array_equal(oracle.rmsnorm_tanh_residual(x, res, w, zero), res)
    # |gate| >= 4 -> tanh = +-1 -> out = bf(residual +- y2)
    sat = np.where(rng.random((1, D)) < 0.5, 0x4080, 0xC080).astype(np.uint16)  # +-4
    out = oracle.rmsnorm_tanh_residual(x, res, w, sat)
    sgn = np.where(sat[0] & 0x8000, -1.0, 1.0)
    for r in range(rows):
        y2, _ = oracle.rms_row(x[r], w, 1e-6)
        ref = nearest_bf16(value_of_bf16(res[r]) + sgn * value_of_bf16(y2))
        assert np.array_equal(out[r], ref)


def test_rmsnorm_tanh_residual_composition():
    rng = np.random.default_rng(96)
    rows, D = 6, 520
    x = nearest_bf16(rng.standard_normal((rows, D))).reshape(rows, D)
    res = nearest_bf16(rng.standard_normal((rows, D))).reshape(rows, D)
    w = nearest_bf16(rng.uniform(0.5, 1.5, D))
    gate = nearest_bf16(rng.standard_normal((rows, D)) * 0.5).reshape(rows, D)
    out = oracle.rmsnorm_tanh_residual(x, res, w, gate)
    for r in range(rows):
        y2, _ = oracle.rms_row(x[r], w, 1e-6)
        tau = value_of_bf16(oracle.tanh_bf16(gate[r]))
        assert ulp_distance(oracle.tanh_bf16(gate[r]),
                            nearest_bf16(np.tanh(value_of_bf16(gate[r])))).max() <= 1
        q = nearest_bf16(tau * value_of_bf16(y2))
        ref = nearest_bf16(value_of_bf16(res[r]) + value_of_bf16(q))
        assert np.array_equal(out[r], ref)


# --------------------------------------------------------------------------------------
# Gated residual + LayerNorm/AdaLN producer (page "基于Agent的SGLang扩散模型Kernel优化实践",
# sections "将FP8量化融合到前序算子" and "NVFP4的三组优化")
# --------------------------------------------------------------------------------------

def _nonzero_shift(shape, seed):
    shift = synth.normal_bf16(shape, 0.1, seed)
    shift[shift & 0x7FFF == 0] = 0x3F80
    return shift


def test_gate_add_ln_zero_gate_constant_residual():
    """gate = +0: bf(gate * y) is a zero, so r' is the residual (a -0 residual
    meeting +0 becomes +0); a constant residual row then gives out = shift."""
    D = 520
    res = synth.constant_bf16((4, D), -3.25)
    res[1] = synth.constant_bf16((1, D), 1000.0)
    y = synth.normal_bf16((4, D), 1.0, 90)
    gate = np.zeros((2, D), dtype=np.uint16)
    scale = synth.normal_bf16((2, D), 0.1, 91)
    shift = _nonzero_shift((2, D), 92)
    rp, out = oracle.gate_add_ln_modulate(res, y, gate, scale, shift)
    assert np.array_equal(rp, res)
    assert np.array_equal(out, np.repeat(shift, 2, axis=0))
    # signed zeros: -0 + (+0) = +0 and -0 + (-0) = -0
    res0 = np.full((2, D), 0x8000, dtype=np.uint16)
    y0 = np.where(np.arange(D) % 2 == 0, 0x3F80, 0xBF80).astype(np.uint16)[None].repeat(2, 0)
    rp0, _ = oracle.gate_add_ln_modulate(res0, y0, gate, scale, shift)
    assert np.array_equal(rp0[:, 0::2], np.zeros((2, D // 2), dtype=np.uint16))
    assert np.array_equal(rp0[:, 1::2], np.full((2, D // 2), 0x8000, dtype=np.uint16))


def test_gate_add_ln_cancellation_gives_shift():
    """gate = 1 and y = -residual: bf(1 * -r) = -r exactly and r + (-r) = +0,
    so r' is a +0 row, a constant row, and out = shift bitwise."""
    D = 1032
    res = synth.normal_bf16((6, D), 1.0, 93)
    y = res ^ np.uint16(0x8000)
    gate = np.full((3, D), 0x3F80, dtype=np.uint16)
    scale = synth.normal_bf16((3, D), 0.1, 94)
    shift = _nonzero_shift((3, D), 95)
    rp, out = oracle.gate_add_ln_modulate(res, y, gate, scale, shift)
    assert np.array_equal(rp, np.zeros_like(res))
    assert np.array_equal(out, np.repeat(shift, 2, axis=0))


@pytest.mark.parametrize("D", [8, 520, 3072])
def test_gate_add_ln_vs_exact_and_double(D):
    """r' is the exact sum of two exactly rounded terms (float64 is exact
    here), and with scale = 0, shift = -0 the output is the LayerNorm of r',
    within 1 ulp of float64 everywhere and equal on >= 99%.  Per-batch
    modulation: rows 0..rows/2-1 use row 0 of gate/scale/shift."""
    rng = np.random.default_rng(96 + D)
    rows = max(4, 8000 // D) * 2
    res = _rand_bf16(rng, rows * D, 3).reshape(rows, D)
    y = _rand_bf16(rng, rows * D, 3).reshape(rows, D)
    gate = _rand_bf16(rng, 2 * D, 2).reshape(2, D)
    scale = np.zeros((2, D), dtype=np.uint16)
    shift = np.full((2, D), 0x8000, dtype=np.uint16)
    rp, out = oracle.gate_add_ln_modulate(res, y, gate, scale, shift)
    g_full = np.repeat(gate, rows // 2, axis=0)
    gy = value_of_bf16(nearest_bf16(value_of_bf16(g_full) * value_of_bf16(y)))
    s = value_of_bf16(res) + gy
    assert np.all((s - value_of_bf16(res)) == gy)
    assert np.array_equal(rp, nearest_bf16(s).reshape(rows, D))
    tot = eq = 0
    for r in range(rows):
        ref_v, _ = _ln_double(value_of_bf16(rp[r]), 1e-6)
        d = ulp_distance(out[r], nearest_bf16(ref_v))
        assert d.max() <= 1, (D, r)
        eq += int((d == 0).sum())
        tot += D
    assert eq / tot >= 0.99


def test_gate_add_ln_per_batch_equals_repeated_per_token():
    """Row r uses modulation row r // (rows / mod_rows): per-batch tensors give
    the same result as the same rows repeated per token."""
    rows, D = 12, 520
    res = synth.normal_bf16((rows, D), 1.0, 97)
    y = synth.normal_bf16((rows, D), 1.0, 98)
    gate, scale, shift = (synth.normal_bf16((3, D), 0.1, 99 + i) for i in range(3))
    a = oracle.gate_add_ln_modulate(res, y, gate, scale, shift)
    rep = [np.repeat(t, rows // 3, axis=0) for t in (gate, scale, shift)]
    b = oracle.gate_add_ln_modulate(res, y, *rep)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# --------------------------------------------------------------------------------------
# Standalone modulate (page "#34085 [diffusion] Clean up kernels and shared fast paths",
# section "实现拆解": modulate_scale_shift)
# --------------------------------------------------------------------------------------

def test_modulate_scale_shift_exact_steps():
    """Each of the three roundings is a single correct rounding of an exact
    float64 value: 1 + scale, the product of two bf16 values, the sum of two
    bf16 values.  Per-batch rows (rows 0-5 use modulation row 0)."""
    rng = np.random.default_rng(150)
    rows, D = 12, 520
    x = _rand_bf16(rng, rows * D, 6).reshape(rows, D)
    scale = nearest_bf16(rng.standard_normal((2, D)) * 0.3).reshape(2, D)
    shift = _rand_bf16(rng, 2 * D, 4).reshape(2, D)
    out = oracle.modulate_scale_shift(x, scale, shift)
    sc, sh = np.repeat(scale, 6, axis=0), np.repeat(shift, 6, axis=0)
    s1 = value_of_bf16(nearest_bf16(1.0 + value_of_bf16(sc)))
    p = value_of_bf16(nearest_bf16(value_of_bf16(x) * s1))
    ref = nearest_bf16(p + value_of_bf16(sh)).reshape(rows, D)
    assert np.array_equal(out, ref)


def test_modulate_scale_shift_identities():
    """scale = 0, shift = -0: x * 1 + (-0) = x bitwise; scale = -1: x * 0 is
    a zero, so out = shift (shift non-zero, x finite)."""
    x = synth.normal_bf16((8, 1032), 1.0, 151)
    zero = np.zeros((1, 1032), dtype=np.uint16)
    negz = np.full((1, 1032), 0x8000, dtype=np.uint16)
    assert np.array_equal(oracle.modulate_scale_shift(x, zero, negz), x)
    shift = _nonzero_shift((1, 1032), 152)
    minus1 = np.full((1, 1032), 0xBF80, dtype=np.uint16)
    assert np.array_equal(oracle.modulate_scale_shift(x, minus1, shift),
                          np.repeat(shift, 8, axis=0))


# --------------------------------------------------------------------------------------
# BF16 + static E4M3 dual output (page "基于Agent的SGLang扩散模型Kernel优化实践", section
# "将FP8量化融合到前序算子")
# --------------------------------------------------------------------------------------

E4M3_CODES = np.arange(256, dtype=np.uint32).astype(np.uint8)


def _torch_e4m3(v):
    """torch's CPU float8_e4m3fn conversion (round to nearest even) of |v| < 464."""
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_codes_roundtrip_and_known_values():
    vals = oracle.e4m3_value(E4M3_CODES)
    fin = np.isfinite(vals)
    assert fin.sum() == 254 and not fin[0x7F] and not fin[0xFF]
    assert np.array_equal(oracle.e4m3(vals[fin].astype(np.float32)), E4M3_CODES[fin])
    known = {1.0: 0x38, 0.5: 0x30, 448.0: 0x7E, 2.0 ** -9: 0x01, 2.0 ** -6: 0x08,
             1.75: 0x3E, 240.0: 0x77, -2.0: 0xC0, 0.0: 0x00}
    for v, c in known.items():
        assert oracle.e4m3(np.float32(v)) == c, (v, hex(c))
    assert oracle.e4m3(np.float32(-0.0)) == 0x80
    # decoded magnitudes: 7 subnormals m * 2^-9, then (8 + m) * 2^(e - 10)
    assert vals[0x07] == 7 * 2.0 ** -9 and vals[0x08] == 2.0 ** -6 and vals[0x7E] == 448.0


def test_e4m3_midpoints_tie_to_even_and_saturate():
    vals = oracle.e4m3_value(E4M3_CODES[:0x7F])
    for c in range(0x7E):
        mid = (vals[c] + vals[c + 1]) / 2                    # exact in binary32
        m32 = np.float32(mid)
        assert float(m32) == mid
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3(m32) == even, hex(c)
        assert oracle.e4m3(np.nextafter(m32, np.float32(0))) == c
        assert oracle.e4m3(np.nextafter(m32, np.float32(np.inf))) == c + 1
        assert oracle.e4m3(-m32) == 0x80 | even
    for v in (448.0, 460.0, 464.0, 500.0, 1e30, np.inf):
        assert oracle.e4m3(np.float32(v)) == 0x7E and oracle.e4m3(np.float32(-v)) == 0xFE
    assert oracle.e4m3(np.float32(np.nan)) & 0x7F == 0x7F
    assert oracle.e4m3(np.float32(2.0 ** -10)) == 0x00        # tie with zero: even
    assert oracle.e4m3(np.float32(-(2.0 ** -11))) == 0x80     # underflow keeps the sign


def test_e4m3_vs_torch():
    rng = np.random.default_rng(120)
    n = 1 << 20
    v = (rng.standard_normal(n) * np.exp2(rng.integers(-14, 9, n))).astype(np.float32)
    v = v[np.abs(v) < 464]
    assert np.array_equal(oracle.e4m3(v), _torch_e4m3(v))


@pytest.mark.parametrize("fp8_scale", [1.0, 0.0173, 2.0 ** -3])
def test_ln_modulate_fp8_vs_torch_quant(fp8_scale):
    """The BF16 output is the plain LN + modulate output; the E4M3 output is
    torch's IEEE division by the scale, clamped to +-448, cast to E4M3."""
    x = synth.normal_bf16((12, 1032), 1.0, 121)
    scale = synth.normal_bf16((2, 1032), 0.1, 122)
    shift = synth.normal_bf16((2, 1032), 0.1, 123)
    out, out8 = oracle.ln_modulate_fp8(x, scale, shift, 1e-6, fp8_scale)
    assert np.array_equal(out, oracle.ln_modulate(x, scale, shift, 1e-6))
    t = torch.from_numpy(value_of_bf16(out).astype(np.float32))
    ref = (t / torch.tensor(fp8_scale, dtype=torch.float32)).clamp(-448, 448)
    assert np.array_equal(out8, ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_fp8_quantization_divides_by_the_scale():
    """Constant rows give out = shift, so out8 = E4M3(shift / s).  For s = 3.1
    these bf16 values give a different E4M3 code when h / s is replaced by
    h * (1 / s) (one binary32 ulp across a rounding midpoint); the division
    decides."""
    s = np.float32(3.1)
    h = value_of_bf16(np.arange(65536, dtype=np.uint32).astype(np.uint16)).astype(np.float32)
    fin = np.isfinite(h)
    with np.errstate(all="ignore"):
        by_div = oracle.e4m3((h / s).astype(np.float32))
        by_rcp = oracle.e4m3((h * (np.float32(1) / s)).astype(np.float32))
    pick = np.flatnonzero((by_div != by_rcp) & fin)[:64]
    assert pick.size >= 8
    D = 8 * ((pick.size + 7) // 8)
    shift = np.full((1, D), 0x3F80, dtype=np.uint16)
    shift[0, :pick.size] = pick.astype(np.uint16)
    x = synth.constant_bf16((2, D), 0.75)
    scale = np.zeros((1, D), dtype=np.uint16)
    out, out8 = oracle.ln_modulate_fp8(x, scale, shift, 1e-6, float(s))
    assert np.array_equal(out, np.repeat(shift, 2, axis=0))
    assert np.array_equal(out8[:, :pick.size], np.repeat(by_div[pick][None], 2, axis=0))


def test_gate_add_ln_modulate_fp8():
    res = synth.normal_bf16((8, 520), 1.0, 124)
    y = synth.normal_bf16((8, 520), 1.0, 125)
    gate, scale, shift = (synth.normal_bf16((2, 520), 0.1, 126 + i) for i in range(3))
    rp, out, out8 = oracle.gate_add_ln_modulate_fp8(res, y, gate, scale, shift, 1e-6, 0.05)
    rp2, out2 = oracle.gate_add_ln_modulate(res, y, gate, scale, shift, 1e-6)
    assert np.array_equal(rp, rp2) and np.array_equal(out, out2)
    t = torch.from_numpy(value_of_bf16(out).astype(np.float32)) / torch.tensor(0.05)
    assert np.array_equal(out8, t.clamp(-448, 448).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy())


# --------------------------------------------------------------------------------------
# Wan per-token modulation table (page "基于Agent的SGLang扩散模型Kernel优化实践", section
# "Wan视频模型的数据搬运优化")
# --------------------------------------------------------------------------------------

def test_wan_mod_table_layout_with_tagged_values():
    """table[k][i] = 4096 k and temb[b][s][k][i] = a small integer tag of
    (b, s, k, i): every sum is exact, so each output element names the
    operands that reached it; out is [n_mod, B, S, D]."""
    B, S, K, D = 2, 5, 6, 24
    table = np.repeat((4096.0 * np.arange(K, dtype=np.float32))[:, None], D, axis=1)
    b, s_, k, i = np.meshgrid(np.arange(B), np.arange(S), np.arange(K), np.arange(D),
                              indexing="ij")
    tag = (b * 101 + s_ * 13 + k * 7 + i) % 250                    # exact in bf16
    temb = nearest_bf16(tag.astype(np.float64)).reshape(B, S, K, D)
    out = oracle.wan_mod_table(table, temb)
    assert out.shape == (K, B, S, D)
    for kk in range(K):
        assert np.array_equal(out[kk], 4096.0 * kk + tag[:, :, kk, :].astype(np.float32))


def test_wan_mod_table_one_rounding():
    """Random fp32 table and bf16 time embedding: each output is the exact sum
    rounded once to binary32 (the float64 sum is exact for these exponent
    ranges, which the test checks)."""
    rng = np.random.default_rng(140)
    B, S, K, D = 1, 64, 6, 520
    table = (rng.standard_normal((K, D)) * 0.05).astype(np.float32)
    temb = nearest_bf16(rng.standard_normal((B, S, K, D)) * 0.3).reshape(B, S, K, D)
    out = oracle.wan_mod_table(table, temb)
    tv = value_of_bf16(temb)
    exact = table[None, None].astype(np.float64) + tv            # [B, S, K, D]
    assert np.all(exact - tv == table[None, None].astype(np.float64))
    ref = np.moveaxis(exact.astype(np.float32), 2, 0)
    assert np.array_equal(out, ref)


# --------------------------------------------------------------------------------------
# Q/K RMSNorm + interleaved RoPE + joint write
# --------------------------------------------------------------------------------------

def _head_inputs(rng, Dh):
    x = nearest_bf16(rng.standard_normal(Dh) * 1.3)
    w = nearest_bf16(rng.uniform(0.5, 1.5, Dh))
    return x, w


@pytest.mark.parametrize("Dh", [8, 128])
def test_qk_head_identity_rotation_is_rmsnorm(Dh):
    """cos = 1, sin = 0: a*1 - b*0 = a, so the output is u = bf(bf(x*rho)*w),
    which is within 1 ulp of float64 RMSNorm (two roundings)."""
    rng = np.random.default_rng(100 + Dh)
    c = np.ones(Dh // 2, dtype=np.float32)
    z = np.zeros(Dh // 2, dtype=np.float32)
    for it in range(50):
        x, w = _head_inputs(rng, Dh)
        if it % 2:
            x = nearest_bf16(value_of_bf16(x) * 1e-3)   # mean square ~ eps
        o = oracle.qk_head(x, w, c, z, 1e-6)
        xv = value_of_bf16(x)
        ideal = xv / np.sqrt((xv ** 2).mean() + 1e-6) * value_of_bf16(w)
        assert ulp_distance(o, nearest_bf16(ideal)).max() <= 1


def test_qk_head_quarter_and_half_turns():
    """cos = 0, sin = 1 maps (a, b) to (-b, a); cos = -1, sin = 0 maps it to
    (-a, -b): exact, so bitwise."""
    rng = np.random.default_rng(110)
    x, w = _head_inputs(rng, 128)
    u = oracle.qk_head(x, w, np.ones(64, np.float32), np.zeros(64, np.float32), 1e-6)
    q = oracle.qk_head(x, w, np.zeros(64, np.float32), np.ones(64, np.float32), 1e-6)
    h = oracle.qk_head(x, w, -np.ones(64, np.float32), np.zeros(64, np.float32), 1e-6)
    assert np.array_equal(value_of_bf16(q[0::2]), -value_of_bf16(u[1::2]))
    assert np.array_equal(value_of_bf16(q[1::2]), value_of_bf16(u[0::2]))
    assert np.array_equal(value_of_bf16(h), -value_of_bf16(u))


def test_qk_head_normalized_value_rounded_before_the_weight():
    """The Q/K head norm rounds bf(x * rho) before the weight multiplies it
    (page "基于Agent的SGLang扩散模型Kernel优化实践", section "合并QKV投影时的数值
    问题": normalize, then apply the per-head-dim weight, each in bf16).
    Hand-derived head, Dh = 128, eps = 1e-6: x = (1.0625, -1.0625, 0.75,
    0.375, 0.1875, 0.0625, 2, then 121 ones), whose squares sum to 128
    exactly, so ms = 1; ms + eps rounds to 1 + 2^-20, its square root to
    1 + 2^-21 and rho = 1 / that to 1 - 2^-21 (0x3F7FFFF8).  x0 * rho =
    1.0625 - 4 * 2^-23 (0x3F87FFFC) rounds to bf16 1.0625; with w0 = 1.1875
    (0x3F98) the product 1.26171875 is exactly the midpoint between 161/128
    and 162/128 and ties to the even 162/128 = 1.265625 (0x3FA2).  Without
    the first rounding, (1.0625 - 4 * 2^-23) * 1.1875 lies below that
    midpoint and gives 161/128 (0x3FA1).  cos = 1, sin = 0 leaves u as it is."""
    vals = [1.0625, -1.0625, 0.75, 0.375, 0.1875, 0.0625, 2.0] + [1.0] * 121
    assert sum(Fraction(v) ** 2 for v in vals) == 128
    x = nearest_bf16(np.array(vals))
    w = np.full(128, 0x3F80, dtype=np.uint16)
    w[0] = 0x3F98
    f = np.float32
    rho = f(1) / np.sqrt(f(1) + f(1e-6))
    assert Fraction(float(rho)) == 1 - Fraction(1, 2 ** 21)
    n0 = f(1.0625) * rho
    assert Fraction(float(n0)) == Fraction(1.0625) - Fraction(4, 2 ** 23)
    assert frac_bf16(Fraction(float(n0))) == 0x3F88
    assert frac_bf16(Fraction(1.0625) * Fraction(1.1875)) == 0x3FA2
    assert frac_bf16(Fraction(float(n0 * f(1.1875)))) == 0x3FA1          # the other reading
    o = oracle.qk_head(x, w, np.ones(64, np.float32), np.zeros(64, np.float32), 1e-6)
    assert o[0] == 0x3FA2
    assert np.array_equal(o[1:], x[1:])          # bf(x * rho) = x for the others, w = 1


def test_qk_head_rope_products_rounded_separately():
    """RoPE rounds each product to binary32 before the sum, with no fused
    multiply-add (the lossless reading of the interleaved rotation on page
    "基于Agent的SGLang扩散模型Kernel优化实践", section "合并QKV投影时的数值问题").
    A constant head x = 1 has ms = 1, so bf(x * rho) = 1 and u = w.  With
    u = (a, a, a, -a, 1, 1, ...) for a = 129/128 and a 45-degree rotation
    (cos = sin = c = 0x3F3504F3): o0 = a*c - a*c and o3 = a*c + (-a)*c are
    differences of two equal rounded products, exactly +0; o1 = o2 = 2 a*c
    rounds to 0x3FB6.  A fused form would leave the rounding error of a*c,
    a*c - fp32(a*c) = -6.05e-9 (bf16 0xB1D0), in o0 and o3."""
    x = np.full(128, 0x3F80, dtype=np.uint16)
    w = np.full(128, 0x3F80, dtype=np.uint16)
    w[0] = w[1] = w[2] = 0x3F81
    w[3] = 0xBF81
    c = np.full(64, np.sqrt(0.5), dtype=np.float32)
    assert c[0].view(np.uint32) == 0x3F3504F3
    u = oracle.qk_head(x, w, np.ones(64, np.float32), np.zeros(64, np.float32), 1e-6)
    assert np.array_equal(u, w)
    a, cc = Fraction(129, 128), Fraction(float(c[0]))
    ac = Fraction(float(np.float32(float(a * cc))))          # a*c is exact in float64
    assert ac != a * cc
    assert frac_bf16(a * cc - ac) == 0xB1D0                   # the fused form's o0
    assert frac_bf16(2 * ac) == 0x3FB6
    o = oracle.qk_head(x, w, c, c, 1e-6)
    assert list(o[:4]) == [0x0000, 0x3FB6, 0x3FB6, 0x0000]
    assert np.all(o[4::2] == 0x0000)                          # (1, 1): c - c


def test_qk_head_rotation_preserves_norm_and_matches_double():
    cos_t, sin_t = synth.rope_tables_axial()
    assert np.abs(cos_t.astype(np.float64) ** 2 + sin_t.astype(np.float64) ** 2 - 1).max() \
        <= 2.0 ** -22
    rng = np.random.default_rng(111)
    ones = np.full(128, 0x3F80, dtype=np.uint16)
    for tok in rng.integers(0, cos_t.shape[0], 40):
        x, w = _head_inputs(rng, 128)
        u = oracle.qk_head(x, w, np.ones(64, np.float32), np.zeros(64, np.float32), 1e-6)
        o = oracle.qk_head(x, w, cos_t[tok], sin_t[tok], 1e-6)
        a, b = value_of_bf16(u[0::2]), value_of_bf16(u[1::2])
        oa, ob = value_of_bf16(o[0::2]), value_of_bf16(o[1::2])
        n_in, n_out = np.hypot(a, b), np.hypot(oa, ob)
        assert np.all(np.abs(n_out - n_in) <= 2.0 ** -7 * n_in + 1e-30)
        c, s = cos_t[tok].astype(np.float64), sin_t[tok].astype(np.float64)
        ideal = np.empty(128)
        ideal[0::2] = a * c - b * s
        ideal[1::2] = a * s + b * c
        d = ulp_distance(o, nearest_bf16(ideal))
        assert d.max() <= 1
        n1 = oracle.qk_head(x, ones, np.ones(64, np.float32), np.zeros(64, np.float32), 1e-6)
        assert abs((value_of_bf16(n1) ** 2).mean() - 1) <= 2.0 ** -7


def test_qk_norm_rope_joint_placement_and_v_copy():
    """Joint rows: text tokens first, then image tokens; V is copied bit for
    bit; Q and K heads use their stream's weights and the joint row's table."""
    rng = np.random.default_rng(120)
    B, S_txt, S_img, H, Dh = 2, 3, 5, 2, 128
    W = 3 * H * Dh
    txt = nearest_bf16(rng.standard_normal(B * S_txt * W)).reshape(B, S_txt, W)
    img = nearest_bf16(rng.standard_normal(B * S_img * W)).reshape(B, S_img, W)
    wts = [nearest_bf16(rng.uniform(0.5, 1.5, Dh)) for _ in range(4)]
    ang = rng.uniform(-3, 3, (S_txt + S_img, Dh // 2))
    cos_t, sin_t = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)

    def views(a):
        b, s, _ = a.shape
        return [a[:, :, i * H * Dh:(i + 1) * H * Dh].reshape(b, s, H, Dh) for i in range(3)]

    tq, tk, tv = views(txt)
    iq, ik, iv = views(img)
    q, k, v = oracle.qk_norm_rope(dict(q=tq, k=tk, v=tv, q_weight=wts[0], k_weight=wts[1]),
                                  dict(q=iq, k=ik, v=iv, q_weight=wts[2], k_weight=wts[3]),
                                  cos_t, sin_t)
    for b in range(B):
        for j in range(S_txt + S_img):
            src, s, wq, wk = (txt, j, wts[0], wts[1]) if j < S_txt else (img, j - S_txt, wts[2],
                                                                          wts[3])
            for h in range(H):
                qs = src[b, s, h * Dh:(h + 1) * Dh]
                ks = src[b, s, H * Dh + h * Dh:H * Dh + (h + 1) * Dh]
                vs = src[b, s, 2 * H * Dh + h * Dh:2 * H * Dh + (h + 1) * Dh]
                assert np.array_equal(v[b, j, h], vs)
                assert np.array_equal(q[b, j, h], oracle.qk_head(qs, wq, cos_t[j], sin_t[j], 1e-6))
                assert np.array_equal(k[b, j, h], oracle.qk_head(ks, wk, cos_t[j], sin_t[j], 1e-6))


def test_qk_norm_rope_destination_major_layout():
    """Destination-major output for Ulysses sequence parallelism (page
    "基于Agent的SGLang扩散模型Kernel优化实践", section "Ulysses QKV仅执行一次All-to-All"):
    chunk p of the packed [P, B, S, 3, H/P, Dh] buffer holds heads p H/P ..
    (p + 1) H/P - 1 of q, k and v for every token, in the joint order.  Checked
    against the plain joint outputs through an independent index permutation,
    and V (a bit copy) against its source heads directly."""
    rng = np.random.default_rng(121)
    B, S_txt, S_img, H, Dh = 2, 3, 5, 8, 128
    W = 3 * H * Dh
    txt = nearest_bf16(rng.standard_normal(B * S_txt * W)).reshape(B, S_txt, W)
    img = nearest_bf16(rng.standard_normal(B * S_img * W)).reshape(B, S_img, W)
    wts = [nearest_bf16(rng.uniform(0.5, 1.5, Dh)) for _ in range(4)]
    ang = rng.uniform(-3, 3, (S_txt + S_img, Dh // 2))
    cos_t, sin_t = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)

    def views(a):
        b, s, _ = a.shape
        return [a[:, :, i * H * Dh:(i + 1) * H * Dh].reshape(b, s, H, Dh) for i in range(3)]

    tq, tk, tv = views(txt)
    iq, ik, iv = views(img)
    ts = dict(q=tq, k=tk, v=tv, q_weight=wts[0], k_weight=wts[1])
    ims = dict(q=iq, k=ik, v=iv, q_weight=wts[2], k_weight=wts[3])
    joint = np.stack(oracle.qk_norm_rope(ts, ims, cos_t, sin_t), axis=2)   # [B, S, 3, H, Dh]
    for P in (1, 2, 4, 8):
        packed = oracle.qk_norm_rope_packed(ts, ims, cos_t, sin_t, P)
        hp = H // P
        assert packed.shape == (P, B, S_txt + S_img, 3, hp, Dh)
        ref = np.moveaxis(joint.reshape(B, S_txt + S_img, 3, P, hp, Dh), 3, 0)
        assert np.array_equal(packed, ref), P
        for p in range(P):
            for h in range(hp):
                g = p * hp + h
                assert np.array_equal(packed[p, :, :S_txt, 2, h],
                                      txt[:, :, 2 * H * Dh + g * Dh:2 * H * Dh + (g + 1) * Dh])
                assert np.array_equal(packed[p, :, S_txt:, 2, h],
                                      img[:, :, 2 * H * Dh + g * Dh:2 * H * Dh + (g + 1) * Dh])
