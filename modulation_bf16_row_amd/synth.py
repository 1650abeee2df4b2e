"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random tensors and builds the RoPE cos/sin tables; it holds
none of the epilogues' arithmetic and imports neither the HIP binding nor the
oracle.  Values are drawn in float64 with numpy's ``default_rng``, cast to
float32, then converted to bfloat16 (round to nearest even) by torch's CPU
conversion, and handed out as numpy ``uint16`` bit patterns.

Workload shapes follow the DiT models the pages benchmark: Qwen-Image at
1024x1024 (4096 image + 512 text tokens, hidden 3072, 24 heads of 128, CFG
batch 2) and Wan 720p video (21x45x80 = 75600 latent tokens, hidden 5120).
"""
import numpy as np
import torch


def _to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shape, std=1.0, seed=0, mean=0.0) -> np.ndarray:
    """N(mean, std^2) samples as bf16 bits; ``std`` is the standard deviation."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(size=shape) * std + mean
    return _to_bf16_bits(v.astype(np.float32))


def uniform_bf16(shape, lo=0.5, hi=1.5, seed=0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return _to_bf16_bits(rng.uniform(lo, hi, size=shape).astype(np.float32))


def student_t_bf16(shape, df=3.0, scale=1.0, seed=0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return _to_bf16_bits((rng.standard_t(df, size=shape) * scale).astype(np.float32))


def constant_bf16(shape, value) -> np.ndarray:
    return _to_bf16_bits(np.full(shape, value, dtype=np.float32))


def rope_tables_axial(s_txt=512, grid_h=64, grid_w=64, head_dim=128, theta=10000.0):
    """cos/sin tables [s_txt + grid_h*grid_w, head_dim/2] in float32.

    Joint token order is text first, then image.  Image token k sits at grid
    position (h, w) = (k // grid_w, k % grid_w); text token t sits at
    (grid_h + t, grid_h + t).  The first half of the rotation pairs turns by
    the row position, the second half by the column position, with frequency
    theta^(-j / (pairs/2)) for pair j of each half.  Angles and their cosine
    and sine are computed in float64 and rounded once to float32.
    """
    pairs = head_dim // 2
    half = pairs // 2
    n_img = grid_h * grid_w
    k = np.arange(n_img)
    h_pos = np.concatenate([grid_h + np.arange(s_txt), k // grid_w]).astype(np.float64)
    w_pos = np.concatenate([grid_h + np.arange(s_txt), k % grid_w]).astype(np.float64)
    j = np.arange(half, dtype=np.float64)
    freq = theta ** (-j / half)
    ang = np.concatenate([h_pos[:, None] * freq[None, :], w_pos[:, None] * freq[None, :]], axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


# --- the workloads ----------------------------------------------------------------------
# Seeds are 1000 * config + tensor index.

def small_adaln(seed_base=1000):
    """[1, 256, 1024] LN + AdaLN modulate with per-batch scale/shift, and the
    gate for the residual gate-add on the same shape."""
    D = 1024
    return dict(
        x=normal_bf16((256, D), 1.0, seed_base + 0),
        scale=normal_bf16((1, D), 0.1, seed_base + 1),
        shift=normal_bf16((1, D), 0.1, seed_base + 2),
        gate=normal_bf16((1, D), 0.1, seed_base + 3),
        eps=1e-6,
    )


def qwen_image_block(seed_base=2000, batch=2, tokens=4608, dim=3072):
    """Qwen-Image 1024x1024 block epilogues: x [batch*tokens, dim] ~ N(0,1),
    per-batch scale/shift/gate/scale2 [batch, dim] ~ N(0, 0.1), RMSNorm weight
    ~ U(0.5, 1.5), residual ~ N(0, 1)."""
    rows = batch * tokens
    return dict(
        x=normal_bf16((rows, dim), 1.0, seed_base + 0),
        scale=normal_bf16((batch, dim), 0.1, seed_base + 1),
        shift=normal_bf16((batch, dim), 0.1, seed_base + 2),
        gate=normal_bf16((batch, dim), 0.1, seed_base + 3),
        scale2=normal_bf16((batch, dim), 0.1, seed_base + 4),
        weight=uniform_bf16((dim,), 0.5, 1.5, seed_base + 5),
        residual=normal_bf16((rows, dim), 1.0, seed_base + 6),
        eps=1e-6,
    )


def qwen_image_qkv(seed_base=3000, batch=2, s_img=4096, s_txt=512, heads=24, head_dim=128,
                   grid=(64, 64)):
    """Merged-QKV GEMM outputs per stream, [batch, S, 3*heads*head_dim] ~ N(0,1),
    four RMSNorm weights [head_dim] ~ U(0.5, 1.5), axial RoPE tables."""
    width = 3 * heads * head_dim
    cos_t, sin_t = rope_tables_axial(s_txt, grid[0], grid[1], head_dim)
    return dict(
        img_qkv=normal_bf16((batch, s_img, width), 1.0, seed_base + 0),
        txt_qkv=normal_bf16((batch, s_txt, width), 1.0, seed_base + 1),
        img_q_weight=uniform_bf16((head_dim,), 0.5, 1.5, seed_base + 2),
        img_k_weight=uniform_bf16((head_dim,), 0.5, 1.5, seed_base + 3),
        txt_q_weight=uniform_bf16((head_dim,), 0.5, 1.5, seed_base + 4),
        txt_k_weight=uniform_bf16((head_dim,), 0.5, 1.5, seed_base + 5),
        cos=cos_t, sin=sin_t, heads=heads, head_dim=head_dim, eps=1e-6,
    )


def wan_720p_block(seed_base=4000, tokens=75600, dim=5120, per_token=True):
    """Wan 720p block: x, residual [tokens, dim] ~ N(0,1); per-token (or
    per-batch) scale/shift/gate ~ N(0, 0.1); weight ~ U(0.5, 1.5)."""
    mod_rows = tokens if per_token else 1
    return dict(
        x=normal_bf16((tokens, dim), 1.0, seed_base + 0),
        scale=normal_bf16((mod_rows, dim), 0.1, seed_base + 1),
        shift=normal_bf16((mod_rows, dim), 0.1, seed_base + 2),
        gate=normal_bf16((mod_rows, dim), 0.1, seed_base + 3),
        weight=uniform_bf16((dim,), 0.5, 1.5, seed_base + 4),
        residual=normal_bf16((tokens, dim), 1.0, seed_base + 5),
        eps=1e-6,
    )


def chain_block(seed_base=5000, batch=2, tokens=4608, dim=3072):
    """50-iteration stability chain: x0 ~ N(0,1); per-batch scale, shift,
    gate, scale2 ~ N(0, 0.1); weight ~ U(0.5, 1.5)."""
    rows = batch * tokens
    return dict(
        x=normal_bf16((rows, dim), 1.0, seed_base + 0),
        scale=normal_bf16((batch, dim), 0.1, seed_base + 1),
        shift=normal_bf16((batch, dim), 0.1, seed_base + 2),
        gate=normal_bf16((batch, dim), 0.1, seed_base + 3),
        scale2=normal_bf16((batch, dim), 0.1, seed_base + 4),
        weight=uniform_bf16((dim,), 0.5, 1.5, seed_base + 5),
        eps=1e-6,
    )


def wan_720p_block_device(seed=4000, tokens=75600, dim=5120, device="cuda"):
    """The Wan 720p block drawn on the device (host draws of 774 MB tensors
    take most of a minute): torch's seeded generator on `device`, float32
    N(0, 1) rows (x, residual), N(0, 0.1) per-token scale/shift/gate and a
    per-batch gate [1, dim], U(0.5, 1.5) weight, each rounded to bfloat16
    (nearest even).  Returns bfloat16 device tensors; the oracle receives the
    same values copied to the host."""
    gen = torch.Generator(device=device).manual_seed(seed)

    def bf(shape, std):
        return (torch.randn(shape, device=device, generator=gen) * std).to(torch.bfloat16)

    out = dict(x=bf((tokens, dim), 1.0), residual=bf((tokens, dim), 1.0),
               scale=bf((tokens, dim), 0.1), shift=bf((tokens, dim), 0.1),
               gate=bf((tokens, dim), 0.1), gate1=bf((1, dim), 0.1))
    out["weight"] = (torch.rand(dim, device=device, generator=gen) + 0.5).to(torch.bfloat16)
    out["eps"] = 1e-6
    return out
