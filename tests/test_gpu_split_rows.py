"""The split-row layout (taken without per-batch staging: per-token
modulation, or fewer than four rows per modulation row) with strided views
and in-place calls, against the oracle bit for bit.

Rows and outputs sit inside wider buffers (row stride > dim) and the
modulation rows inside a wider buffer of their own (modulation row stride >
dim); D = 1032 leaves the last chunk almost empty (NC = 3, two waves per
row).  In place: LN + AdaLN and RMSNorm-scale into x, the gated residual +
LN producer with r' into the residual and the output into y, and the E4M3
producer into x.  Both per-token modulation (37 rows) and three rows per
modulation row (36 rows, 12 modulation rows).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bits_equal, dev, host, say
from modulation_bf16_row_amd import synth

pytestmark = pytest.mark.gpu

EPS = 1e-6
DIM = 1032
PAD = 1536


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import modulation_bf16_row_amd as m
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    m.lib()


def m():
    import modulation_bf16_row_amd as mod
    return mod


def _wide(h, off):
    """bf16 bits h [n, DIM] placed at column `off` of a zeroed [n, PAD] device
    buffer; returns (buffer, [n, DIM] view)."""
    buf = np.zeros((h.shape[0], PAD), dtype=np.uint16)
    buf[:, off:off + DIM] = h
    d = dev(buf)
    return d, d[:, off:off + DIM]


@pytest.mark.parametrize("rows,mod_rows", [(37, 37), (36, 12)])
def test_split_rows_strided(rows, mod_rows):
    say("split rows strided", rows, mod_rows)
    seed = 7100 + rows
    x = synth.student_t_bf16((rows, DIM), 3.0, 1.0, seed)
    res = synth.normal_bf16((rows, DIM), 1.0, seed + 1)
    mods = np.concatenate([synth.normal_bf16((mod_rows, DIM), 0.2, seed + 2 + k)
                           for k in range(3)], axis=1)             # scale | shift | gate
    w = synth.uniform_bf16((DIM,), 0.5, 1.5, seed + 5)
    sc, sh, g = (np.ascontiguousarray(mods[:, k * DIM:(k + 1) * DIM]) for k in range(3))
    _, xv = _wide(x, 8)
    _, rv = _wide(res, 24)
    mbuf = dev(np.concatenate([mods, np.zeros((mod_rows, 8), dtype=np.uint16)], axis=1))
    scv, shv, gv = (mbuf[:, k * DIM:(k + 1) * DIM] for k in range(3))
    assert scv.stride(0) == 3 * DIM + 8 and xv.stride(0) == PAD
    wd = dev(w)
    M = m()

    outb = torch.zeros((rows, PAD), dtype=torch.bfloat16, device="cuda")
    ov = outb[:, 40:40 + DIM]
    M.dit_ln_modulate(xv, scv, shv, EPS, out=ov)
    assert_bits_equal(host(ov), oracle.ln_modulate(x, sc, sh, EPS), "ln strided")
    assert not host(outb)[:, :40].any() and not host(outb)[:, 40 + DIM:].any()
    M.dit_rmsnorm_scale(xv, wd, scv, EPS, out=ov)
    assert_bits_equal(host(ov), oracle.rmsnorm_scale(x, w, sc, EPS), "rms strided")
    M.dit_modulate_scale_shift(xv, scv, shv, out=ov)
    assert_bits_equal(host(ov), oracle.modulate_scale_shift(x, sc, sh), "modulate strided")

    both = torch.zeros((rows, 2 * PAD), dtype=torch.bfloat16, device="cuda")
    rp, out = M.dit_gate_add_ln_modulate(rv, xv, gv, scv, shv, EPS,
                                         out_residual=both[:, 16:16 + DIM],
                                         out=both[:, PAD:PAD + DIM])
    ref_rp, ref_out = oracle.gate_add_ln_modulate(res, x, g, sc, sh, EPS)
    assert_bits_equal(host(rp), ref_rp, "gate_ln r' strided")
    assert_bits_equal(host(out), ref_out, "gate_ln out strided")


@pytest.mark.parametrize("rows,mod_rows", [(37, 37), (36, 12)])
def test_split_rows_in_place(rows, mod_rows):
    say("split rows in place", rows, mod_rows)
    seed = 7200 + rows
    x = synth.normal_bf16((rows, DIM), 1.0, seed)
    res = synth.normal_bf16((rows, DIM), 1.0, seed + 1)
    sc = synth.normal_bf16((mod_rows, DIM), 0.2, seed + 2)
    sh = synth.normal_bf16((mod_rows, DIM), 0.2, seed + 3)
    g = synth.normal_bf16((mod_rows, DIM), 0.2, seed + 4)
    w = synth.uniform_bf16((DIM,), 0.5, 1.5, seed + 5)
    M = m()

    d = dev(x)
    M.dit_ln_modulate(d, dev(sc), dev(sh), EPS, out=d)
    assert_bits_equal(host(d), oracle.ln_modulate(x, sc, sh, EPS), "ln in place")
    d = dev(x)
    M.dit_rmsnorm_scale(d, dev(w), dev(sc), EPS, out=d)
    assert_bits_equal(host(d), oracle.rmsnorm_scale(x, w, sc, EPS), "rms in place")
    r, y = dev(res), dev(x)
    M.dit_gate_add_ln_modulate(r, y, dev(g), dev(sc), dev(sh), EPS, out_residual=r, out=y)
    ref_rp, ref_out = oracle.gate_add_ln_modulate(res, x, g, sc, sh, EPS)
    assert_bits_equal(host(r), ref_rp, "gate_ln r' into residual")
    assert_bits_equal(host(y), ref_out, "gate_ln out into y")
    fs = torch.tensor([0.05], dtype=torch.float32, device="cuda")
    d = dev(x)
    out, q = M.dit_ln_modulate_fp8(d, dev(sc), dev(sh), fs, EPS, out=d)
    ref_out, ref_q = oracle.ln_modulate_fp8(x, sc, sh, EPS, 0.05)
    assert_bits_equal(host(d), ref_out, "ln_fp8 in place")
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), ref_q)
