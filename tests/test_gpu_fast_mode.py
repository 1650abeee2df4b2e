"""FAST mode against LOSSLESS on every row-kernel instantiation and at the
Wan 720p shape (per-token modulation).

FAST differs from LOSSLESS in the binary32 values entering some bf16
roundings (the LayerNorm rho from the hardware rsqrt, fused multiply-add in
the sum of squared deviations), never in where the roundings are.  Checked
here:
- LN + AdaLN modulate (and the LN half of the gated residual + LN producer,
  and the bf16 output of the E4M3 producer): >= 99.9% of elements within one
  bf16 step, and at most 2 steps of the largest magnitude taking part in
  the last rounding, max(|p|, |shift|, |out|);
- the native-bf16 RMSNorm ops: the bf16 rstd is the same in both modes (the
  hardware rsqrt passes a rounding test; checked on all 65536 inputs by the
  primitive tests), so RMSNorm-scale and RMSNorm-tanh-residual are equal to
  LOSSLESS bit for bit -- which implies the 2-step bound in steps of
  max(|residual|, |q|), also computed;
- the residual gate-add: the same arithmetic in both modes, bitwise;
- the E4M3 copy of a FAST output is the quantization of that bf16 output.
Sources: page "基于Agent的SGLang扩散模型Kernel优化实践", sections "质量分级机制"
and "SGLang扩散Kernel的验证流程".
"""
import numpy as np
import pytest
import torch

import oracle
from fast_util import ln_last_magnitude, report, tanh_last_magnitude
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


def _per_row(t, rows):
    """Modulation rows expanded to one per row."""
    return np.repeat(t, rows // t.shape[0], axis=0)


def _check_ln(name, fast, lossless, mag):
    _, frac1, scaled = report(name, fast, lossless, mag)
    assert frac1 >= 0.999, name
    assert scaled <= 2.0, name


@pytest.mark.parametrize("dim", WIDTHS)
@pytest.mark.parametrize("rows,mod_rows", [(32, 4), (9, 9)])
def test_fast_every_chunk_count(dim, rows, mod_rows):
    say("fast all widths", dim, rows, mod_rows)
    seed = 9500 + dim + rows
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
    scr, shr, gr = _per_row(sc, rows), _per_row(sh, rows), _per_row(g, rows)

    ln_l = host(M.dit_ln_modulate(dx, dsc, dsh, EPS, "lossless"))
    ln_f = host(M.dit_ln_modulate(dx, dsc, dsh, EPS, "fast"))
    _check_ln("ln " + tag, ln_f, ln_l, ln_last_magnitude(x, scr, shr, EPS))

    for name, call in (
            ("rms", lambda md: M.dit_rmsnorm_scale(dx, dw, dsc, EPS, md)),
            ("tanh", lambda md: M.dit_rmsnorm_tanh_residual(dx, dres, dw, dg, EPS, md)),
            ("gate", lambda md: M.dit_residual_gate_add(dres, dx, dg, md)),
            ("modulate", lambda md: M.dit_modulate_scale_shift(dx, dsc, dsh, md))):
        fl, ff = host(call("lossless")), host(call("fast"))
        assert_bits_equal(ff, fl, f"fast {name} {tag}")
        if name == "tanh":
            _, _, scaled = report("tanh " + tag, ff, fl, tanh_last_magnitude(x, res, w, gr, EPS))
            assert scaled <= 2.0

    rp_l, out_l = M.dit_gate_add_ln_modulate(dres, dx, dg, dsc, dsh, EPS, "lossless")
    rp_f, out_f = M.dit_gate_add_ln_modulate(dres, dx, dg, dsc, dsh, EPS, "fast")
    rp_h = host(rp_l)
    assert_bits_equal(host(rp_f), rp_h, "fast gate_ln r' " + tag)
    _check_ln("gate_ln out " + tag, host(out_f), host(out_l),
              ln_last_magnitude(rp_h, scr, shr, EPS))

    out8, q = M.dit_ln_modulate_fp8(dx, dsc, dsh, fs, EPS, "fast")
    out8_h = host(out8)
    assert_bits_equal(out8_h, ln_f, "fast ln_fp8 bf16 output " + tag)
    ref_q = oracle.e4m3(oracle.bf16_value(out8_h) / np.float32(FP8_SCALE))
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), ref_q), "fast ln_fp8 e4m3 " + tag


def _sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, n - 2, n - 1], rng.integers(0, n, k)]))


def test_fast_wan_720p_per_token():
    """The Wan 720p block ([75600, 5120], per-token scale/shift/gate, and a
    per-batch gate; drawn on the device) in FAST against LOSSLESS: LN +
    modulate within the tolerances (scaled bound on 300 sampled rows, literal
    fraction over all rows); RMSNorm-tanh-residual equal in both gate
    layouts."""
    d = synth.wan_720p_block_device(seed=4100)
    eps = d["eps"]
    M = m()
    say("fast wan ln_modulate per-token [75600,5120]")
    ln_l = host(M.dit_ln_modulate(d["x"], d["scale"], d["shift"], eps, "lossless"))
    ln_f = host(M.dit_ln_modulate(d["x"], d["scale"], d["shift"], eps, "fast"))
    _, frac1, _ = report("wan ln per-token (all rows)", ln_f, ln_l)
    assert frac1 >= 0.999
    idx = _sample_rows(ln_l.shape[0], 300, 13)
    sel = torch.from_numpy(idx).cuda()
    hx, hsc, hsh = (host(d[k].index_select(0, sel)) for k in ("x", "scale", "shift"))
    _check_ln("wan ln per-token (sampled rows, scaled)", ln_f[idx], ln_l[idx],
              ln_last_magnitude(hx, hsc, hsh, eps))
    del ln_l, ln_f
    for gate, tag in ((d["gate"], "per-token gate"), (d["gate1"], "per-batch gate")):
        say("fast wan rmsnorm_tanh_residual", tag)
        tl = host(M.dit_rmsnorm_tanh_residual(d["x"], d["residual"], d["weight"], gate, eps,
                                              "lossless"))
        tf = host(M.dit_rmsnorm_tanh_residual(d["x"], d["residual"], d["weight"], gate, eps,
                                              "fast"))
        assert_bits_equal(tf, tl, "fast wan tanh " + tag)
