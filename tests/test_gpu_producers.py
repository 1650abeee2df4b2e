"""LOSSLESS parity of the fused producers with the CPU oracle, bit for bit
(E4M3 outputs code for code).

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
from exact import value_of_bf16
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


# --------------------------------------------------------------------------------------
# BF16 + static E4M3 dual output (page "基于Agent的SGLang扩散模型Kernel优化实践", section
# "将FP8量化融合到前序算子")
# --------------------------------------------------------------------------------------

def _e4m3_equal(got, ref, what):
    """Code equality; NaN codes (0x7F / 0xFF) compare as NaN on both sides."""
    got, ref = np.asarray(got, dtype=np.uint8), np.asarray(ref, dtype=np.uint8)
    gn, rn = (got & 0x7F) == 0x7F, (ref & 0x7F) == 0x7F
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ"
    bad = np.flatnonzero((got != ref) & ~gn)
    assert bad.size == 0, (f"{what}: {bad.size} codes differ, first "
                           f"got={[hex(int(v)) for v in got[bad[:6]]]} "
                           f"ref={[hex(int(v)) for v in ref[bad[:6]]]}")


def test_e4m3_conversion_every_input_in_range():
    """The kernels' conversion against the oracle on every positive binary32
    value in [2^-11, 2^10) (zero codes below, saturation above), a sample of
    negatives, and the edges outside the range."""
    say("e4m3 conversion, every positive binary32 in [2^-11, 2^10)")
    first, last = 0x3A000000, 0x44800000
    chunk = 1 << 24
    for start in range(first, last, chunk):
        n = min(chunk, last - start)
        bits = torch.arange(start, start + n, dtype=torch.int32, device="cuda")
        got = m().dit_probe_fp8(0, bits.view(torch.float32)).cpu().numpy()
        _e4m3_equal(got, oracle.e4m3_bits_range(start, n), hex(start))
        del bits
    say("e4m3 conversion, negatives and edges")
    rng = np.random.default_rng(130)
    neg = (rng.integers(first, last, 1 << 20, dtype=np.uint64) | 0x80000000).astype(np.uint32)
    edges = []
    for e in range(256):
        for mant in (0, 1, 0x400000, 0x7FFFFF):
            edges += [(e << 23) | mant, 0x80000000 | (e << 23) | mant]
    bits = np.concatenate([neg, np.array(edges, dtype=np.uint32)])
    got = m().dit_probe_fp8(0, torch.from_numpy(bits.view(np.float32)).cuda()).cpu().numpy()
    _e4m3_equal(got, oracle.e4m3(bits.view(np.float32)), "negatives and edges")


@pytest.mark.parametrize("fp8_scale", [1.0, 3.1, 0.3, 0.0173, 2.0 ** -3, 179.2, -0.37,
                                       2.0 ** -140, 3.0e38, 1e-30, 0.0])
def test_fp8_quantization_every_bf16(fp8_scale):
    """E4M3(h / s) for every bf16 h: the kernels' division and conversion
    against an IEEE binary32 division and the oracle's encoder."""
    say("fp8 quantization, every bf16, scale", fp8_scale)
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s = torch.tensor([fp8_scale], dtype=torch.float32, device="cuda")
    got = m().dit_probe_fp8(1, dev(codes), s).cpu().numpy()
    with np.errstate(all="ignore"):
        q = (value_of_bf16(codes).astype(np.float32) / np.float32(fp8_scale)).astype(np.float32)
    _e4m3_equal(got, oracle.e4m3(q), f"scale {fp8_scale}")


def _fs(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def _u8(t):
    return t.view(torch.uint8).cpu().numpy()


@pytest.mark.parametrize("dim", [8, 520, 3072, 5120, 8192])
@pytest.mark.parametrize("rows,mod_rows", [(1, 1), (37, 1), (36, 3), (37, 37)])
def test_ln_modulate_fp8_shapes(dim, rows, mod_rows):
    say("ln_modulate_fp8", dim, rows, mod_rows)
    inp = _inputs(30 * dim + rows, rows, dim, mod_rows)
    x, sc, sh = dev(inp["res"]), dev(inp["scale"]), dev(inp["shift"])
    out, q = m().dit_ln_modulate_fp8(x, sc, sh, _fs(0.0173), EPS)
    ref, ref8 = oracle.ln_modulate_fp8(inp["res"], inp["scale"], inp["shift"], EPS, 0.0173)
    assert_bits_equal(host(out), ref, f"bf16 dim={dim} rows={rows}/{mod_rows}")
    _e4m3_equal(_u8(q), ref8, f"e4m3 dim={dim} rows={rows}/{mod_rows}")


@pytest.mark.parametrize("dim,rows,mod_rows", [(520, 37, 1), (3072, 64, 2), (5120, 12, 12),
                                              (8192, 8, 2)])
def test_gate_add_ln_modulate_fp8_shapes(dim, rows, mod_rows):
    say("gate_add_ln_modulate_fp8", dim, rows, mod_rows)
    inp = _inputs(40 * dim + rows, rows, dim, mod_rows)
    rp, out, q = m().dit_gate_add_ln_modulate_fp8(*_dev_all(inp), _fs(3.1), EPS)
    refs = oracle.gate_add_ln_modulate_fp8(inp["res"], inp["y"], inp["gate"], inp["scale"],
                                           inp["shift"], EPS, 3.1)
    assert_bits_equal(host(rp), refs[0], "r'")
    assert_bits_equal(host(out), refs[1], "out")
    _e4m3_equal(_u8(q), refs[2], "e4m3")


@pytest.mark.parametrize("mode", ["lossless", "fast"])
def test_fp8_bf16_outputs_equal_bf16_only_calls(mode):
    say("fp8 producers: bf16 outputs vs bf16-only calls", mode)
    inp = _inputs(555, 96, 3072, 2)
    res, y, g, sc, sh = _dev_all(inp)
    out, q = m().dit_ln_modulate_fp8(res, sc, sh, _fs(0.05), EPS, mode)
    assert_bits_equal(host(out), host(m().dit_ln_modulate(res, sc, sh, EPS, mode)), "ln")
    rp, out2, q2 = m().dit_gate_add_ln_modulate_fp8(res, y, g, sc, sh, _fs(0.05), EPS, mode)
    rp_ref, out_ref = m().dit_gate_add_ln_modulate(res, y, g, sc, sh, EPS, mode)
    assert_bits_equal(host(rp), host(rp_ref), "r'")
    assert_bits_equal(host(out2), host(out_ref), "gated out")
    # the E4M3 copy is the quantization of the BF16 output, in both modes
    ref8 = m().dit_probe_fp8(1, out2, _fs(0.05)).cpu().numpy()
    _e4m3_equal(_u8(q2), ref8, "e4m3 of out")


def test_fp8_in_place_and_uint8_output():
    say("fp8 producers in place")
    rows, dim = 24, 1032
    inp = _inputs(556, rows, dim, 2)
    refs = oracle.gate_add_ln_modulate_fp8(inp["res"], inp["y"], inp["gate"], inp["scale"],
                                           inp["shift"], EPS, 0.3)
    res, y, g, sc, sh = _dev_all(inp)
    q = torch.empty((rows, dim), dtype=torch.uint8, device="cuda")
    m().dit_gate_add_ln_modulate_fp8(res, y, g, sc, sh, _fs(0.3), EPS, out_residual=res, out=y,
                                     out_fp8=q)
    assert_bits_equal(host(res), refs[0], "r' in residual")
    assert_bits_equal(host(y), refs[1], "out in y")
    _e4m3_equal(q.cpu().numpy(), refs[2], "e4m3 uint8")


def test_fp8_qwen_block_full_size():
    """The Qwen-Image 1024x1024 block [9216, 3072]: both dual-output
    producers, every element of every output."""
    w = synth.qwen_image_block()
    say("ln_modulate_fp8 qwen block [9216,3072]")
    out, q = m().dit_ln_modulate_fp8(dev(w["x"]), dev(w["scale"]), dev(w["shift"]), _fs(0.0173),
                                     w["eps"])
    ref, ref8 = oracle.ln_modulate_fp8(w["x"], w["scale"], w["shift"], w["eps"], 0.0173)
    assert_bits_equal(host(out), ref, "qwen ln bf16")
    _e4m3_equal(_u8(q), ref8, "qwen ln e4m3")
    say("gate_add_ln_modulate_fp8 qwen block")
    rp, out, q = m().dit_gate_add_ln_modulate_fp8(
        dev(w["residual"]), dev(w["x"]), dev(w["gate"]), dev(w["scale"]), dev(w["shift"]),
        _fs(0.0173), w["eps"])
    refs = oracle.gate_add_ln_modulate_fp8(w["residual"], w["x"], w["gate"], w["scale"],
                                           w["shift"], w["eps"], 0.0173)
    assert_bits_equal(host(rp), refs[0], "qwen r'")
    assert_bits_equal(host(out), refs[1], "qwen out")
    _e4m3_equal(_u8(q), refs[2], "qwen e4m3")


# --------------------------------------------------------------------------------------
# Wan per-token modulation table (page "基于Agent的SGLang扩散模型Kernel优化实践", section
# "Wan视频模型的数据搬运优化")
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("B,S,K,D", [(1, 1, 6, 8), (1, 37, 6, 520), (2, 100, 6, 3072),
                                     (1, 300, 6, 5120), (3, 7, 2, 1032), (2, 64, 6, 1024),
                                     (1, 2, 1, 16)])
def test_wan_modulation_table_shapes(B, S, K, D):
    say("wan modulation table", B, S, K, D)
    rng = np.random.default_rng(B * 1000 + S + D)
    table = (rng.standard_normal((K, D)) * 0.05).astype(np.float32)
    temb = synth.normal_bf16((B, S, K, D), 0.3, 7000 + S)
    got = m().dit_wan_modulation_table(torch.from_numpy(table).cuda(), dev(temb))
    ref = oracle.wan_mod_table(table, temb)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_wan_modulation_table_full_size():
    """The Wan 720p block: 75600 tokens x 6 x 5120 (4.6 GB in, 9.3 GB out),
    inputs drawn on the device; every element against torch's binary32
    addition of the same operands (the unfused expression), and sampled
    tokens against the oracle."""
    say("wan modulation table [1, 75600, 6, 5120]")
    g = torch.Generator(device="cuda").manual_seed(4100)
    table = torch.randn((6, 5120), device="cuda", generator=g) * 0.05
    temb = (torch.randn((1, 75600, 6, 5120), device="cuda", generator=g) * 0.3).to(
        torch.bfloat16)
    out = m().dit_wan_modulation_table(table, temb)
    for k in range(6):
        ref = table[k][None, None, :] + temb[:, :, k, :].float()
        assert torch.equal(out[k].view(torch.int32), ref.view(torch.int32)), k
        del ref
    tok = torch.tensor([0, 1, 37777, 75599], device="cuda")
    t_h = table.cpu().numpy()
    e_h = host(temb.index_select(1, tok))
    ref = oracle.wan_mod_table(t_h, e_h)
    got = out.index_select(2, tok).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_wan_modulation_table_beyond_32_bit_indices():
    """6 x 2^20 tokens x 2736: 4.30e9 groups of four outputs, past 2^32, so the
    launch takes the 64-bit grid-stride kernel (69 GB out, 34 GB in, drawn on
    the device in slices).  Chunk k = 5, which holds the groups past 2^32,
    against torch's binary32 addition on every element; sampled tokens of
    every chunk against the oracle."""
    S, K, D = 1 << 20, 6, 2736
    say("wan modulation table beyond 2^32 groups [1, %d, %d, %d]" % (S, K, D))
    g = torch.Generator(device="cuda").manual_seed(4200)
    table = torch.randn((K, D), device="cuda", generator=g) * 0.05
    temb = torch.empty((1, S, K, D), dtype=torch.bfloat16, device="cuda")
    step = 1 << 16
    for s0 in range(0, S, step):
        temb[:, s0:s0 + step] = (torch.randn((1, step, K, D), device="cuda", generator=g)
                                 * 0.3).to(torch.bfloat16)
    out = m().dit_wan_modulation_table(table, temb)
    ref = table[K - 1][None, None, :] + temb[:, :, K - 1, :].float()
    assert torch.equal(out[K - 1].view(torch.int32), ref.view(torch.int32))
    del ref
    tok = torch.tensor([0, 1, (1 << 19) + 3, S - 2, S - 1], device="cuda")
    ref = oracle.wan_mod_table(table.cpu().numpy(), host(temb.index_select(1, tok)))
    got = out.index_select(2, tok).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    del out, temb
    torch.cuda.empty_cache()
