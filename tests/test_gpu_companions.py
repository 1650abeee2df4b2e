"""LOSSLESS parity of the two companion kernels with the CPU oracle, bit for bit.

Standalone AdaLN modulate (page "#34085 [diffusion] Clean up kernels and
shared fast paths", section "实现拆解", modulate_scale_shift): out =
bf(bf(x * bf(1 + scale)) + shift), over several 512-element chunks and
ragged tails, per-batch, grouped and per-token modulation, every bf16 scale
code, in-place and strided calls, and the Qwen-Image and Wan 720p shapes.

Destination-major QKV epilogue (page "基于Agent的SGLang扩散模型Kernel优化实践",
section "Ulysses QKV仅执行一次All-to-All"): the packed [P, B, S, 3, H/P, 128]
buffer equals the oracle for P = 1 .. H, and, at the full Qwen-Image shape,
the oracle (P = 8) and a re-indexing of the plain joint output (P = 2, 4).
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


# --------------------------------------------------------------------------------------
# modulate_scale_shift
# --------------------------------------------------------------------------------------

def _mod_inputs(seed, rows, dim, mod_rows):
    return (synth.student_t_bf16((rows, dim), 3.0, 1.0, seed),
            synth.normal_bf16((mod_rows, dim), 0.2, seed + 1),
            synth.normal_bf16((mod_rows, dim), 0.2, seed + 2))


@pytest.mark.parametrize("dim", DIMS)
@pytest.mark.parametrize("rows,mod_rows", [(1, 1), (37, 1), (36, 3), (37, 37), (64, 2),
                                           (600, 2)])
def test_modulate_shapes(dim, rows, mod_rows):
    say("modulate", dim, rows, mod_rows)
    x, sc, sh = _mod_inputs(30 * dim + rows, rows, dim, mod_rows)
    out = m().dit_modulate_scale_shift(dev(x), dev(sc), dev(sh))
    assert_bits_equal(host(out), oracle.modulate_scale_shift(x, sc, sh),
                      f"dim={dim} rows={rows}/{mod_rows}")


@pytest.mark.parametrize("per_mod", [1, 3])
def test_modulate_every_scale_code(per_mod):
    """Every bf16 pattern as a scale value (NaN, infinities, subnormals, the
    values where 1 + scale rounds to a tie), each used by per_mod rows."""
    say("modulate every scale code", per_mod)
    dim, mod_rows = 8192, 8
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(mod_rows, dim)
    x = synth.student_t_bf16((mod_rows * per_mod, dim), 3.0, 2.0, 61 + per_mod)
    sh = synth.normal_bf16((mod_rows, dim), 0.5, 62)
    out = m().dit_modulate_scale_shift(dev(x), dev(codes), dev(sh))
    assert_bits_equal(host(out), oracle.modulate_scale_shift(x, codes, sh), "every scale code")


def test_modulate_in_place_strided_and_modes():
    say("modulate in place / strided / modes")
    rows, dim = 48, 1032
    x, sc, sh = _mod_inputs(71, rows, dim, 4)
    ref = oracle.modulate_scale_shift(x, sc, sh)
    # strided input and output rows inside wider buffers
    xb = torch.zeros((rows, dim + 24), dtype=torch.bfloat16, device="cuda:0")
    xb[:, 8:8 + dim] = dev(x)
    ob = torch.zeros((rows, dim + 40), dtype=torch.bfloat16, device="cuda:0")
    scb = torch.zeros((4, dim + 8), dtype=torch.bfloat16, device="cuda:0")
    shb = torch.zeros((4, dim + 8), dtype=torch.bfloat16, device="cuda:0")
    scb[:, :dim] = dev(sc)
    shb[:, :dim] = dev(sh)
    m().dit_modulate_scale_shift(xb[:, 8:8 + dim], scb[:, :dim], shb[:, :dim],
                                 out=ob[:, 16:16 + dim])
    assert_bits_equal(host(ob[:, 16:16 + dim]), ref, "strided")
    assert not host(ob[:, :16]).any() and not host(ob[:, 16 + dim:]).any(), "wrote outside rows"
    # in place, both modes
    for mode in ("lossless", "fast"):
        xt = dev(x)
        m().dit_modulate_scale_shift(xt, dev(sc), dev(sh), mode=mode, out=xt)
        assert_bits_equal(host(xt), ref, f"in place {mode}")


def _device_normal(shape, std, seed):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda:0") * std).to(torch.bfloat16)


@pytest.mark.parametrize("name,rows,dim,mod_rows", [
    ("qwen-image 1024^2, per-batch", 2 * 4608, 3072, 2),
    ("wan 720p, per-token", 75600, 5120, 75600),
])
def test_modulate_full_size_sampled(name, rows, dim, mod_rows):
    """Full-size launch; the oracle checks 600 sampled rows (rows are independent)."""
    say("modulate full size", name)
    x = _device_normal((rows, dim), 1.0, 81)
    sc = _device_normal((mod_rows, dim), 0.2, 82)
    sh = _device_normal((mod_rows, dim), 0.2, 83)
    out = m().dit_modulate_scale_shift(x, sc, sh)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    idx = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, 600, replace=False)]))
    per_mod = rows // mod_rows
    it = torch.from_numpy(idx).cuda()
    mi = torch.from_numpy(idx // per_mod).cuda()
    ref = oracle.modulate_scale_shift(host(x[it]), host(sc[mi]), host(sh[mi]))
    assert_bits_equal(host(out[it]), ref, name)


# --------------------------------------------------------------------------------------
# destination-major QKV
# --------------------------------------------------------------------------------------

def _qkv_case(B, S_txt, S_img, H, seed):
    Dh = 128
    W = 3 * H * Dh
    txt = synth.normal_bf16((B, S_txt, W), 1.0, seed)
    img = synth.normal_bf16((B, S_img, W), 1.0, seed + 1)
    wts = [synth.uniform_bf16((Dh,), 0.5, 1.5, seed + 2 + i) for i in range(4)]
    rng = np.random.default_rng(seed)
    ang = rng.uniform(-6, 6, (S_txt + S_img, Dh // 2))
    return txt, img, wts, np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _views(a, H, Dh=128):
    if isinstance(a, np.ndarray):
        return [a[:, :, i * H * Dh:(i + 1) * H * Dh].reshape(a.shape[0], a.shape[1], H, Dh)
                for i in range(3)]
    return [a[:, :, i * H * Dh:(i + 1) * H * Dh].view(a.shape[0], a.shape[1], H, Dh)
            for i in range(3)]


def _streams(txt, img, wts, H):
    tq, tk, tv = _views(txt, H)
    iq, ik, iv = _views(img, H)
    return (dict(q=tq, k=tk, v=tv, q_weight=wts[0], k_weight=wts[1]),
            dict(q=iq, k=ik, v=iv, q_weight=wts[2], k_weight=wts[3]))


def _gpu_streams(txt, img, wts, H):
    return _streams(dev(txt), dev(img), [dev(w) for w in wts], H)


def _repack(q, k, v, P):
    """Plain joint outputs [B, S, H, Dh] -> the packed [P, B, S, 3, H/P, Dh]."""
    B, S, H, Dh = q.shape
    st = np.stack([q, k, v], axis=2)                       # [B, S, 3, H, Dh]
    st = st.reshape(B, S, 3, P, H // P, Dh)
    return np.ascontiguousarray(st.transpose(3, 0, 1, 2, 4, 5))


@pytest.mark.parametrize("B,S_txt,S_img,H", [(2, 3, 5, 24), (1, 0, 7, 24), (2, 5, 0, 4),
                                             (3, 2, 9, 6), (2, 64, 256, 24)])
def test_qkv_destination_major(B, S_txt, S_img, H):
    txt, img, wts, cos_t, sin_t = _qkv_case(B, S_txt, S_img, H, 90 + H + S_img)
    ref_txt, ref_img = _streams(txt, img, wts, H)
    g_txt, g_img = _gpu_streams(txt, img, wts, H)
    cos_d, sin_d = torch.from_numpy(cos_t).cuda(), torch.from_numpy(sin_t).cuda()
    for P in [p for p in range(1, H + 1) if H % p == 0]:
        say(f"qkv dest B={B} txt={S_txt} img={S_img} H={H} P={P}")
        buf = m().dit_qk_norm_rope_packed(g_txt if S_txt else None, g_img if S_img else None,
                                          cos_d, sin_d, P, EPS)
        ref = oracle.qk_norm_rope_packed(ref_txt, ref_img, cos_t, sin_t, P, EPS)
        assert_bits_equal(host(buf), ref, f"P={P}")


@pytest.mark.parametrize("mode", ["lossless", "fast"])
def test_qkv_destination_major_equals_repacked_plain(mode):
    say("qkv dest vs plain", mode)
    B, S_txt, S_img, H = 2, 40, 200, 24
    txt, img, wts, cos_t, sin_t = _qkv_case(B, S_txt, S_img, H, 123)
    g_txt, g_img = _gpu_streams(txt, img, wts, H)
    cos_d, sin_d = torch.from_numpy(cos_t).cuda(), torch.from_numpy(sin_t).cuda()
    q, k, v = (host(t) for t in m().dit_qk_norm_rope(g_txt, g_img, cos_d, sin_d, EPS, mode=mode))
    for P in (2, 3, 8):
        buf = m().dit_qk_norm_rope_packed(g_txt, g_img, cos_d, sin_d, P, EPS, mode=mode)
        assert_bits_equal(host(buf), _repack(q, k, v, P), f"{mode} P={P}")


def test_qkv_destination_major_full_size():
    """Qwen-Image 1024^2 joint attention input: 512 text + 4096 image tokens,
    batch 2, 24 heads.  P = 8 against the oracle; P = 2, 4 against the plain
    kernel's output re-indexed (itself compared with the oracle elsewhere)."""
    q = synth.qwen_image_qkv()
    H = q["heads"]
    wts = [q["txt_q_weight"], q["txt_k_weight"], q["img_q_weight"], q["img_k_weight"]]
    g_txt, g_img = _gpu_streams(q["txt_qkv"], q["img_qkv"], wts, H)
    cos_d, sin_d = torch.from_numpy(q["cos"]).cuda(), torch.from_numpy(q["sin"]).cuda()
    say("qkv dest full size P=8")
    buf = m().dit_qk_norm_rope_packed(g_txt, g_img, cos_d, sin_d, 8, q["eps"])
    ref_txt, ref_img = _streams(q["txt_qkv"], q["img_qkv"], wts, H)
    ref = oracle.qk_norm_rope_packed(ref_txt, ref_img, q["cos"], q["sin"], 8, q["eps"])
    assert_bits_equal(host(buf), ref, "P=8")
    del buf, ref
    qo, ko, vo = (host(t) for t in m().dit_qk_norm_rope(g_txt, g_img, cos_d, sin_d, q["eps"]))
    for P in (2, 4):
        say("qkv dest full size P=%d" % P)
        buf = m().dit_qk_norm_rope_packed(g_txt, g_img, cos_d, sin_d, P, q["eps"])
        assert_bits_equal(host(buf), _repack(qo, ko, vo, P), f"P={P}")
