"""LOSSLESS parity of the fused producers with the CPU oracle, bit for bit.

Gated residual + LayerNorm/AdaLN (page "基于Agent的SGLang扩散模型Kernel优化实践",
sections "将FP8量化融合到前序算子" and "NVFP4的三组优化"): r' = bf(residual +
bf(gate * y)) and LN + AdaLN modulate of r', both outputs compared with the
oracle over several 512-element chunks and ragged tails, per-batch, grouped
and per-token modulation, the staged and the unstaged launch (dim 8192
loads its modulation per wave), in-place calls, and the full Qwen-Image
block.  The fused call must also equal the two unfused calls in both modes.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bits_equal, dev, host, say
from modulation_bf16_row_amd import synth

pytestmark = pytest.mark.gpu

EPS = 1e-6
DIMS = [8, 520, 1024, 1032, 3072, 5120, 8192]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import modulation_bf16_row_amd as m
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    m.lib()


def m():
    import modulation_bf16_row_amd as mod
    return mod


def _inputs(seed, rows, dim, mod_rows):
    return dict(
        res=synth.normal_bf16((rows, dim), 1.0, seed),
        y=synth.normal_bf16((rows, dim), 1.0, seed + 1),
        gate=synth.normal_bf16((mod_rows, dim), 0.1, seed + 2),
        scale=synth.normal_bf16((mod_rows, dim), 0.1, seed + 3),
        shift=synth.normal_bf16((mod_rows, dim), 0.1, seed + 4),
    )


def _dev_all(inp):
    return [dev(inp[k]) for k in ("res", "y", "gate", "scale", "shift")]


@pytest.mark.parametrize("dim", DIMS)
@pytest.mark.parametrize("rows,mod_rows", [(1, 1), (37, 1), (36, 3), (37, 37), (64, 2)])
def test_gate_add_ln_shapes(dim, rows, mod_rows):
    say("gate_add_ln", dim, rows, mod_rows)
    inp = _inputs(20 * dim + rows, rows, dim, mod_rows)
    rp, out = m().dit_gate_add_ln_modulate(*_dev_all(inp), EPS)
    ref_rp, ref_out = oracle.gate_add_ln_modulate(inp["res"], inp["y"], inp["gate"],
                                                  inp["scale"], inp["shift"], EPS)
    assert_bits_equal(host(rp), ref_rp, f"r' dim={dim} rows={rows}/{mod_rows}")
    assert_bits_equal(host(out), ref_out, f"out dim={dim} rows={rows}/{mod_rows}")


@pytest.mark.parametrize("mode", ["lossless", "fast"])
def test_gate_add_ln_equals_unfused_calls(mode):
    say("gate_add_ln vs unfused", mode)
    inp = _inputs(777, 96, 3072, 2)
    res, y, g, sc, sh = _dev_all(inp)
    rp, out = m().dit_gate_add_ln_modulate(res, y, g, sc, sh, EPS, mode)
    rp2 = m().dit_residual_gate_add(res, y, g, mode)
    out2 = m().dit_ln_modulate(rp2, sc, sh, EPS, mode)
    assert_bits_equal(host(rp), host(rp2), f"r' {mode}")
    assert_bits_equal(host(out), host(out2), f"out {mode}")


def test_gate_add_ln_in_place_and_strided():
    say("gate_add_ln in place")
    rows, dim = 40, 1032
    inp = _inputs(888, rows, dim, 4)
    ref_rp, ref_out = oracle.gate_add_ln_modulate(inp["res"], inp["y"], inp["gate"],
                                                  inp["scale"], inp["shift"], EPS)
    res, y, g, sc, sh = _dev_all(inp)
    m().dit_gate_add_ln_modulate(res, y, g, sc, sh, EPS, out_residual=res, out=y)
    assert_bits_equal(host(res), ref_rp, "r' into residual")
    assert_bits_equal(host(y), ref_out, "out into y")
    # strided row views: both outputs interleaved in one [rows, 2 * dim] buffer
    res, y, g, sc, sh = _dev_all(inp)
    both = torch.zeros((rows, 2 * dim), dtype=torch.bfloat16, device="cuda")
    m().dit_gate_add_ln_modulate(res, y, g, sc, sh, EPS, out_residual=both[:, :dim],
                                 out=both[:, dim:])
    h = host(both)
    assert_bits_equal(np.ascontiguousarray(h[:, :dim]), ref_rp, "strided r'")
    assert_bits_equal(np.ascontiguousarray(h[:, dim:]), ref_out, "strided out")


def test_gate_add_ln_rejects_overlapping_outputs():
    inp = _inputs(999, 8, 512, 1)
    res, y, g, sc, sh = _dev_all(inp)
    o = torch.empty_like(res)
    with pytest.raises(m().DitInvalid):
        m().dit_gate_add_ln_modulate(res, y, g, sc, sh, EPS, out_residual=o, out=o)


def test_gate_add_ln_qwen_block_full_size():
    """The Qwen-Image 1024x1024 block: [9216, 3072] rows, per-batch gate,
    scale and shift [2, 3072]; every element of both outputs."""
    w = synth.qwen_image_block()
    say("gate_add_ln qwen block [9216,3072]")
    y = w["x"]
    rp, out = m().dit_gate_add_ln_modulate(dev(w["residual"]), dev(y), dev(w["gate"]),
                                           dev(w["scale"]), dev(w["shift"]), w["eps"])
    ref_rp, ref_out = oracle.gate_add_ln_modulate(w["residual"], y, w["gate"], w["scale"],
                                                  w["shift"], w["eps"])
    assert_bits_equal(host(rp), ref_rp, "qwen r'")
    assert_bits_equal(host(out), ref_out, "qwen out")
