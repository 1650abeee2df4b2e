"""LOSSLESS parity of the HIP epilogues with the CPU oracle, bit for bit.

Every case draws seeded bf16 inputs, runs the kernel through the C ABI (via
the ctypes binding) and the oracle on the same bits, and compares the output
bit patterns (NaN positions must agree).  Shapes span several 512-element
chunks with ragged tails, single rows, per-batch and per-token modulation,
strided views, in-place calls, and stress rows (large offsets, constant
rows, heavy tails, tiny variance, subnormals, infinities).
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
def _dit():
    import modulation_bf16_row_amd as m
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    m.lib()
    return m


def dit():
    import modulation_bf16_row_amd as m
    return m


def _inputs(seed, rows, dim, mod_rows, x_std=1.0, x_mean=0.0):
    return dict(
        x=synth.normal_bf16((rows, dim), x_std, seed, mean=x_mean),
        res=synth.normal_bf16((rows, dim), 1.0, seed + 1),
        scale=synth.normal_bf16((mod_rows, dim), 0.1, seed + 2),
        shift=synth.normal_bf16((mod_rows, dim), 0.1, seed + 3),
        gate=synth.normal_bf16((mod_rows, dim), 0.1, seed + 4),
        w=synth.uniform_bf16((dim,), 0.5, 1.5, seed + 5),
    )


def _run_all_ops(inp, tag):
    say("row ops", tag)
    x, res, sc, sh, g, w = (dev(inp[k]) for k in ("x", "res", "scale", "shift", "gate", "w"))
    m = dit()
    got = dict(
        ln=host(m.dit_ln_modulate(x, sc, sh, EPS)),
        rms=host(m.dit_rmsnorm_scale(x, w, sc, EPS)),
        tanh=host(m.dit_rmsnorm_tanh_residual(x, res, w, g, EPS)),
        gate=host(m.dit_residual_gate_add(res, x, g)),
    )
    torch.cuda.synchronize()
    ref = dict(
        ln=oracle.ln_modulate(inp["x"], inp["scale"], inp["shift"], EPS),
        rms=oracle.rmsnorm_scale(inp["x"], inp["w"], inp["scale"], EPS),
        tanh=oracle.rmsnorm_tanh_residual(inp["x"], inp["res"], inp["w"], inp["gate"], EPS),
        gate=oracle.residual_gate_add(inp["res"], inp["x"], inp["gate"]),
    )
    for k in got:
        assert_bits_equal(got[k], ref[k], f"{k} {tag}")


@pytest.mark.parametrize("dim", DIMS)
@pytest.mark.parametrize("rows,mod_rows", [(1, 1), (37, 1), (36, 3), (37, 37)])
def test_row_ops_shapes(dim, rows, mod_rows):
    _run_all_ops(_inputs(10 * dim + rows, rows, dim, mod_rows), f"dim={dim} rows={rows}/{mod_rows}")


@pytest.mark.parametrize("rows,mod_rows,dim,path", [(128, 128, 512, "per-token"),
                                                    (64, 8, 8192, "staged")])
def test_tanh_residual_every_gate_code(rows, mod_rows, dim, path):
    """All 65536 bf16 codes as gates (NaN and infinities included), through
    the per-token path and through the staged per-batch path."""
    say("tanh every gate code", path)
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    gate = np.random.default_rng(77).permutation(codes).reshape(mod_rows, dim)
    x = synth.normal_bf16((rows, dim), 1.0, 7001)
    res = synth.normal_bf16((rows, dim), 1.0, 7002)
    w = synth.uniform_bf16((dim,), 0.5, 1.5, 7003)
    got = host(dit().dit_rmsnorm_tanh_residual(dev(x), dev(res), dev(w), dev(gate), EPS))
    assert_bits_equal(got, oracle.rmsnorm_tanh_residual(x, res, w, gate, EPS), path)


def test_small_adaln_workload():
    """[1, 256, 1024] LN + AdaLN modulate (per-batch scale/shift), then the
    residual gate-add on its output."""
    w = synth.small_adaln()
    say("small AdaLN [1,256,1024]")
    m = dit()
    x = dev(w["x"])
    h = m.dit_ln_modulate(x, dev(w["scale"]), dev(w["shift"]), w["eps"])
    o = m.dit_residual_gate_add(x, h, dev(w["gate"]))
    ref_h = oracle.ln_modulate(w["x"], w["scale"], w["shift"], w["eps"])
    assert_bits_equal(host(h), ref_h, "ln_modulate")
    assert_bits_equal(host(o), oracle.residual_gate_add(w["x"], ref_h, w["gate"]), "gate_add")


@pytest.mark.parametrize("kind", ["offset", "constant", "student_t", "tiny_var", "subnormal",
                                  "huge", "zeros"])
def test_stress_rows(kind):
    rows, dim = 24, 3072
    inp = _inputs(777, rows, dim, 2)
    if kind == "offset":
        inp["x"] = synth.normal_bf16((rows, dim), 1.0, 91, mean=1000.0)
    elif kind == "constant":
        inp["x"] = np.repeat(synth.normal_bf16((rows, 1), 3.0, 92), dim, axis=1)
    elif kind == "student_t":
        inp["x"] = synth.student_t_bf16((rows, dim), 3.0, 1.0, 93)
    elif kind == "tiny_var":
        inp["x"] = synth.normal_bf16((rows, dim), 1e-4, 94, mean=0.5)
    elif kind == "subnormal":
        inp["x"] = synth.normal_bf16((rows, dim), 1e-39, 95)
        inp["scale"] = synth.normal_bf16((2, dim), 1e-39, 96)
    elif kind == "huge":
        inp["x"] = synth.normal_bf16((rows, dim), 1e30, 97)
        inp["x"][0, :5] = [0x7F80, 0xFF80, 0x7FC0, 0x7F7F, 0xFF7F]   # inf, -inf, nan, +-max
    elif kind == "zeros":
        inp["x"] = np.zeros((rows, dim), dtype=np.uint16)
        inp["x"][1::2] = 0x8000
    _run_all_ops(inp, kind)


def test_strided_views_and_in_place():
    """Rows read from a wider buffer (row stride > dim), modulation as
    [B, 1, D] views, output into a strided view, and in-place calls."""
    m = dit()
    rows, dim, pad = 40, 1024, 1536
    inp = _inputs(500, rows, dim, 4)
    wide = np.zeros((rows, pad), dtype=np.uint16)
    wide[:, 256:256 + dim] = inp["x"]
    xw = dev(wide)[:, 256:256 + dim]
    sc = dev(inp["scale"]).view(4, 1, dim)
    sh = dev(inp["shift"]).view(4, 1, dim)
    say("strided ln_modulate")
    outw = torch.zeros((rows, pad), dtype=torch.bfloat16, device="cuda:0")
    m.dit_ln_modulate(xw, sc, sh, EPS, out=outw[:, 512:512 + dim])
    ref = oracle.ln_modulate(inp["x"], inp["scale"], inp["shift"], EPS)
    assert_bits_equal(host(outw)[:, 512:512 + dim], ref, "strided out")
    assert not host(outw)[:, :512].any()                           # nothing else written
    say("in-place ops")
    x = dev(inp["x"])
    m.dit_ln_modulate(x, dev(inp["scale"]), dev(inp["shift"]), EPS, out=x)
    assert_bits_equal(host(x), ref, "in-place ln")
    x = dev(inp["x"])
    m.dit_rmsnorm_scale(x, dev(inp["w"]), dev(inp["scale"]), EPS, out=x)
    assert_bits_equal(host(x), oracle.rmsnorm_scale(inp["x"], inp["w"], inp["scale"], EPS), "rms")
    r = dev(inp["res"])
    m.dit_rmsnorm_tanh_residual(dev(inp["x"]), r, dev(inp["w"]), dev(inp["gate"]), EPS, out=r)
    assert_bits_equal(host(r), oracle.rmsnorm_tanh_residual(inp["x"], inp["res"], inp["w"],
                                                            inp["gate"], EPS), "tanh in-place")
    r = dev(inp["res"])
    m.dit_residual_gate_add(r, dev(inp["x"]), dev(inp["gate"]), out=r)
    assert_bits_equal(host(r), oracle.residual_gate_add(inp["res"], inp["x"], inp["gate"]), "gate")


def test_empty_and_rejected_problems():
    m = dit()
    x = torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda:0")
    sc = torch.zeros((1, 1024), dtype=torch.bfloat16, device="cuda:0")
    assert m.dit_ln_modulate(x, sc, sc).shape == (0, 1024)
    bad = torch.zeros((4, 8200), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(m.DitUnsupported):
        m.dit_ln_modulate(bad, bad[:1], bad[:1])
    odd = torch.zeros((4, 1020), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(m.DitUnsupported):
        m.dit_rmsnorm_scale(odd, odd[0], odd[:1])
    x = torch.zeros((6, 1024), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(m.DitUnsupported):
        m.dit_residual_gate_add(x, x, torch.zeros((4, 1024), dtype=torch.bfloat16,
                                                  device="cuda:0"))
    buf = torch.zeros((7, 1024), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(m.DitInvalid):                       # out shifted one row from x
        m.dit_ln_modulate(buf[:6], sc, sc, out=buf[1:])


# --------------------------------------------------------------------------------------
# QKV epilogue
# --------------------------------------------------------------------------------------

def _qkv_case(B, S_txt, S_img, H, seed, grid=None):
    Dh = 128
    W = 3 * H * Dh
    txt = synth.normal_bf16((B, S_txt, W), 1.0, seed)
    img = synth.normal_bf16((B, S_img, W), 1.0, seed + 1)
    wts = [synth.uniform_bf16((Dh,), 0.5, 1.5, seed + 2 + i) for i in range(4)]
    if grid is None:
        rng = np.random.default_rng(seed)
        ang = rng.uniform(-6, 6, (S_txt + S_img, Dh // 2))
        cos_t, sin_t = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    else:
        cos_t, sin_t = synth.rope_tables_axial(S_txt, grid[0], grid[1], Dh)
    return txt, img, wts, cos_t, sin_t


def _views(a, H, Dh=128):
    return [a[:, :, i * H * Dh:(i + 1) * H * Dh].reshape(a.shape[0], a.shape[1], H, Dh)
            if isinstance(a, np.ndarray) else
            a[:, :, i * H * Dh:(i + 1) * H * Dh].view(a.shape[0], a.shape[1], H, Dh)
            for i in range(3)]


def _run_qkv(B, S_txt, S_img, H, seed, grid=None, mode="lossless", joint=False):
    txt, img, wts, cos_t, sin_t = _qkv_case(B, S_txt, S_img, H, seed, grid)
    m = dit()
    tq, tk, tv = _views(dev(txt), H)
    iq, ik, iv = _views(dev(img), H)
    dw = [dev(w) for w in wts]
    out = None
    if joint:     # one [B, S, 3, H, Dh] buffer holding q, k, v interleaved per token
        buf = torch.empty((B, S_txt + S_img, 3, H, 128), dtype=torch.bfloat16, device="cuda:0")
        out = (buf[:, :, 0], buf[:, :, 1], buf[:, :, 2])
    say(f"qkv B={B} txt={S_txt} img={S_img} H={H} joint={joint} mode={mode}")
    q, k, v = m.dit_qk_norm_rope(dict(q=tq, k=tk, v=tv, q_weight=dw[0], k_weight=dw[1]),
                                 dict(q=iq, k=ik, v=iv, q_weight=dw[2], k_weight=dw[3]),
                                 torch.from_numpy(cos_t).cuda(), torch.from_numpy(sin_t).cuda(),
                                 EPS, mode=mode, out=out)
    got = [host(t) for t in (q, k, v)]
    return got, (txt, img, wts, cos_t, sin_t)


def _qkv_ref(txt, img, wts, cos_t, sin_t, H):
    tq, tk, tv = _views(txt, H)
    iq, ik, iv = _views(img, H)
    return oracle.qk_norm_rope(dict(q=tq, k=tk, v=tv, q_weight=wts[0], k_weight=wts[1]),
                               dict(q=iq, k=ik, v=iv, q_weight=wts[2], k_weight=wts[3]),
                               cos_t, sin_t, EPS)


@pytest.mark.parametrize("B,S_txt,S_img,H", [(2, 3, 5, 24), (1, 0, 7, 24), (2, 5, 0, 4),
                                             (3, 2, 9, 5), (1, 1, 1, 1), (2, 64, 256, 24),
                                             (1, 2, 3, 64), (2, 3, 2, 63)])
@pytest.mark.parametrize("joint", [False, True])
def test_qk_norm_rope(B, S_txt, S_img, H, joint):
    got, inp = _run_qkv(B, S_txt, S_img, H, 40 + H + S_img, joint=joint)
    ref = _qkv_ref(*inp, H)
    for name, g, r in zip("qkv", got, ref):
        assert_bits_equal(g, r, f"{name} B={B} txt={S_txt} img={S_img} H={H}")


def test_qk_norm_rope_axial_tables_small_grid():
    """Axial 2-D RoPE tables (16 x 16 image grid + 32 text tokens)."""
    got, inp = _run_qkv(2, 32, 256, 24, 77, grid=(16, 16))
    ref = _qkv_ref(*inp, 24)
    for name, g, r in zip("qkv", got, ref):
        assert_bits_equal(g, r, name)
