"""Exhaustive checks of the kernels' own device primitives against the oracle
and IEEE-754 binary32 on the CPU.

- bf16 rounding of all 2^32 binary32 inputs (the packer the kernels use);
- 1 + scale, the table tanh and the RMSNorm rstd over all 65536 bf16 inputs;
- binary32 division and square root against numpy (IEEE, correctly rounded);
- the two reduction trees on rows built so that summation order matters.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bits_equal, is_nan_bits, say

pytestmark = pytest.mark.gpu

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


@pytest.fixture(scope="module", autouse=True)
def _dit():
    import modulation_bf16_row_amd as m
    assert torch.cuda.is_available()
    m.lib()


def m():
    import modulation_bf16_row_amd as mod
    return mod


def test_bf16_round_all_binary32():
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.int16, device="cuda:0")
    for first in range(0, 1 << 32, chunk):
        say(f"bf16 round slice {first:#x}")
        # slices are aligned to 2^28, so none crosses the int32 sign boundary
        start = first - (1 << 32) if first >= (1 << 31) else first
        bits = torch.arange(start, start + chunk, dtype=torch.int32, device="cuda:0")
        f = bits.view(torch.float32)
        m().dit_probe_bf16_round(f, out)
        got = out.cpu().numpy().view(np.uint16)
        ref = oracle.bf16_round_bits_range(first, chunk)
        nan_in = ((np.arange(first, first + chunk, dtype=np.uint64) & 0x7FFFFFFF)
                  > 0x7F800000)
        assert np.array_equal(got[~nan_in], ref[~nan_in]), hex(first)
        assert np.all(is_nan_bits(got[nan_in]))
        del bits, f


@pytest.mark.parametrize("op,name", [(0, "one_plus"), (2, "rms_rstd"), (3, "tanh_table")])
def test_unary_exhaustive_lossless(op, name):
    say("unary", name)
    h = torch.from_numpy(ALL16.view(np.int16)).cuda()
    got = m().dit_probe_unary(op, h, "lossless").cpu().numpy().view(np.uint16)
    ref = {0: oracle.one_plus, 2: oracle.rms_rstd, 3: oracle.tanh_bf16}[op](ALL16)
    assert_bits_equal(got, ref, name)


def test_unary_reserved_op_is_rejected():
    h = torch.from_numpy(ALL16[:8].view(np.int16)).cuda()
    with pytest.raises(RuntimeError):
        m().dit_probe_unary(1, h, "lossless")


def test_tanh_table_is_mode_independent():
    """The row kernels take tanh(gate) from the table in both modes."""
    say("unary fast tanh_table")
    h = torch.from_numpy(ALL16.view(np.int16)).cuda()
    got = m().dit_probe_unary(3, h, "fast").cpu().numpy().view(np.uint16)
    assert_bits_equal(got, oracle.tanh_bf16(ALL16), "tanh_table fast")


def test_rms_rstd_fast_equals_lossless():
    """FAST takes the hardware rsqrt with a rounding test (the IEEE path
    decides within 4 binary32 steps of a bf16 midpoint, and for inputs that
    are not positive normal numbers), so its bf16 rstd equals LOSSLESS's on
    every one of the 65536 bf16 inputs."""
    say("unary fast rms_rstd")
    h = torch.from_numpy(ALL16.view(np.int16)).cuda()
    got = m().dit_probe_unary(2, h, "fast").cpu().numpy().view(np.uint16)
    assert_bits_equal(got, oracle.rms_rstd(ALL16), "rms_rstd fast")


@pytest.mark.parametrize("flags", range(8))
def test_copy_probe_copies_in_both_layouts(flags):
    """The streaming-copy probe (the bench's ceiling and the counters'
    calibration) moves every byte, in the grid-stride and the flat layout, on
    sizes that leave partial workgroups."""
    say("copy probe flags", flags)
    for n in (8, 8 * 1000 + 8, 8 * 64 * 1024 * 3 + 8 * 17):
        src = torch.arange(n, dtype=torch.int32, device="cuda:0").to(torch.int16).view(
            torch.bfloat16)
        dst = torch.zeros_like(src)
        m().dit_probe_copy(dst, src, flags)
        torch.cuda.synchronize()
        assert torch.equal(dst.view(torch.int16), src.view(torch.int16)), (flags, n)


def _f32_cases(n, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    special = np.array([0.0, -0.0, 1.0, 2.0, 3.0, 1e-45, 1e-38, 1.1754942e-38, 3.4e38, np.inf,
                        -np.inf, np.nan, 0.5, 1e-30, 7.0, 1e6], dtype=np.float32)
    return np.concatenate([special, f, np.abs(rng.standard_normal(n)).astype(np.float32)])


def test_f32_division_and_sqrt_are_ieee():
    say("f32 div/sqrt")
    a = _f32_cases(1 << 20, 1)
    b = _f32_cases(1 << 20, 2)
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    with np.errstate(all="ignore"):
        for op, ref in ((0, a / b), (1, np.sqrt(a)), (2, np.float32(1) / np.sqrt(a))):
            got = m().dit_probe_f32(op, ta, tb, "lossless").cpu().numpy()
            ref = ref.astype(np.float32)
            both_nan = np.isnan(got) & np.isnan(ref)
            assert np.array_equal(got.view(np.uint32)[~both_nan], ref.view(np.uint32)[~both_nan]), op


def _sum_rows(dim, n_rows, seed):
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((n_rows, dim)) * np.exp2(rng.integers(-24, 24, (n_rows, dim))))
    t = t.astype(np.float32)
    # rows where one large term makes the result depend on the order
    for r in range(0, n_rows, 4):
        t[r] = 1.0
        t[r, rng.integers(0, dim)] = 2.0 ** 24
    return t


@pytest.mark.parametrize("dim", [8, 16, 520, 1024, 3072, 5120, 8192])
def test_wave_sum_order(dim):
    say("wave sum", dim)
    t = _sum_rows(dim, 64, dim)
    got = m().dit_probe_row_sum(torch.from_numpy(t).cuda()).cpu().numpy()
    ref = np.array([oracle.sum_wave(r) for r in t], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_head_sum_order():
    say("head sum")
    t = _sum_rows(128, 256, 5)
    got = m().dit_probe_row_sum(torch.from_numpy(t).cuda(), head=True).cpu().numpy()
    ref = np.array([oracle.sum_head(r) for r in t], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
