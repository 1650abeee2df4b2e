"""Every row-kernel instantiation against the oracle, bit for bit.

The row kernels are compiled once per chunk count NC = ceil(D / 512), 1..16.
For each NC the width D = 512 NC - 56 ((NC - 1) mod 3) is taken (the last
chunk partly outside the row for two of every three NC), with per-batch
modulation (the staged layout: 4 modulation rows, 8 rows each) and per-token
modulation (the layout that loads the modulation rows per wave), for LN +
AdaLN, RMSNorm-scale, RMSNorm-tanh-residual, the gated residual + LN
producer and both E4M3 producers; the flat kernels (gate-add, modulate) ride
along at the same shapes.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bits_equal, dev, host, say
from modulation_bf16_row_amd import synth

pytestmark = pytest.mark.gpu

EPS = 1e-6
FP8_SCALE = 0.05
WIDTHS = [512 * nc - 8 * ((nc - 1) % 3) * 7 for nc in range(1, 17)]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import modulation_bf16_row_amd as m
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    m.lib()


def m():
    import modulation_bf16_row_amd as mod
    return mod


def test_widths_cover_every_chunk_count():
    assert sorted({(d + 511) // 512 for d in WIDTHS}) == list(range(1, 17))
    assert all(d % 8 == 0 and 0 < d <= 8192 for d in WIDTHS)


def _e4m3_equal(got, ref, what):
    got, ref = np.asarray(got, dtype=np.uint8), np.asarray(ref, dtype=np.uint8)
    gn, rn = (got & 0x7F) == 0x7F, (ref & 0x7F) == 0x7F
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ"
    bad = np.flatnonzero((got != ref) & ~gn)
    assert bad.size == 0, f"{what}: {bad.size} E4M3 codes differ"


@pytest.mark.parametrize("dim", WIDTHS)
@pytest.mark.parametrize("rows,mod_rows", [(32, 4), (9, 9)])
def test_every_chunk_count(dim, rows, mod_rows):
    say("all widths", dim, rows, mod_rows)
    seed = 9000 + dim + rows
    x = synth.student_t_bf16((rows, dim), 3.0, 1.0, seed)
    res = synth.normal_bf16((rows, dim), 1.0, seed + 1)
    sc = synth.normal_bf16((mod_rows, dim), 0.2, seed + 2)
    sh = synth.normal_bf16((mod_rows, dim), 0.2, seed + 3)
    g = synth.normal_bf16((mod_rows, dim), 0.5, seed + 4)
    w = synth.uniform_bf16((dim,), 0.5, 1.5, seed + 5)
    dx, dres, dsc, dsh, dg, dw = (dev(t) for t in (x, res, sc, sh, g, w))
    fs = torch.tensor([FP8_SCALE], dtype=torch.float32, device="cuda")
    M = m()
    tag = f"dim={dim} rows={rows}/{mod_rows}"

    assert_bits_equal(host(M.dit_ln_modulate(dx, dsc, dsh, EPS)),
                      oracle.ln_modulate(x, sc, sh, EPS), "ln " + tag)
    assert_bits_equal(host(M.dit_rmsnorm_scale(dx, dw, dsc, EPS)),
                      oracle.rmsnorm_scale(x, w, sc, EPS), "rms " + tag)
    assert_bits_equal(host(M.dit_rmsnorm_tanh_residual(dx, dres, dw, dg, EPS)),
                      oracle.rmsnorm_tanh_residual(x, res, w, g, EPS), "tanh " + tag)
    assert_bits_equal(host(M.dit_residual_gate_add(dres, dx, dg)),
                      oracle.residual_gate_add(res, x, g), "gate " + tag)
    assert_bits_equal(host(M.dit_modulate_scale_shift(dx, dsc, dsh)),
                      oracle.modulate_scale_shift(x, sc, sh), "modulate " + tag)

    rp, out = M.dit_gate_add_ln_modulate(dres, dx, dg, dsc, dsh, EPS)
    ref_rp, ref_out = oracle.gate_add_ln_modulate(res, x, g, sc, sh, EPS)
    assert_bits_equal(host(rp), ref_rp, "gate_ln r' " + tag)
    assert_bits_equal(host(out), ref_out, "gate_ln out " + tag)

    out, q = M.dit_ln_modulate_fp8(dx, dsc, dsh, fs, EPS)
    ref_out, ref_q = oracle.ln_modulate_fp8(x, sc, sh, EPS, FP8_SCALE)
    assert_bits_equal(host(out), ref_out, "ln_fp8 out " + tag)
    _e4m3_equal(q.view(torch.uint8).cpu().numpy(), ref_q, "ln_fp8 e4m3 " + tag)

    rp, out, q = M.dit_gate_add_ln_modulate_fp8(dres, dx, dg, dsc, dsh, fs, EPS)
    ref_rp, ref_out, ref_q = oracle.gate_add_ln_modulate_fp8(res, x, g, sc, sh, EPS, FP8_SCALE)
    assert_bits_equal(host(rp), ref_rp, "gate_ln_fp8 r' " + tag)
    assert_bits_equal(host(out), ref_out, "gate_ln_fp8 out " + tag)
    _e4m3_equal(q.view(torch.uint8).cpu().numpy(), ref_q, "gate_ln_fp8 e4m3 " + tag)
