"""The split-row kernels past their grid limit.

Without the staged layout (per-token modulation, or fewer than four rows per
modulation row) LayerNorm + AdaLN and RMSNorm-scale run one workgroup per
row up to 2^31 - 1 workgroups; above that the workgroups walk the rows
gridDim.x apart.  Rows = 2^31 + 64 at D = 8 with two rows per modulation row
(so the split layout is taken) makes the last 65 workgroups take a second
row.  The calls run in place (x about 34 GB, scale and shift about 17 GB
each).

Reference: the oracle on sampled rows -- the first, the middle, random rows
and every row a workgroup reaches on its second pass (rows 2^31 - 1 ..
2^31 + 63) with the row before them.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bits_equal, host, say

pytestmark = pytest.mark.gpu

D = 8
ROWS = (1 << 31) + 64
GRID = (1 << 31) - 1
EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import modulation_bf16_row_amd as m
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    m.lib()


def m():
    import modulation_bf16_row_amd as mod
    return mod


def _fill(t, seed, std):
    g = torch.Generator(device="cuda").manual_seed(seed)
    step = 1 << 26
    for r0 in range(0, t.shape[0], step):
        t[r0:r0 + step] = (torch.randn((min(step, t.shape[0] - r0), t.shape[1]), device="cuda",
                                       generator=g) * std).to(torch.bfloat16)


def _sample_rows():
    rng = np.random.default_rng(17)
    second_pass = np.arange(GRID - 1, ROWS)
    return np.unique(np.concatenate([[0, 1, ROWS // 2], rng.choice(ROWS, 32, replace=False),
                                     second_pass]))


def test_split_rows_beyond_the_grid_limit_in_place():
    say("split rows beyond the grid limit [%d, %d], LN + AdaLN and RMSNorm-scale" % (ROWS, D))
    x = torch.empty((ROWS, D), dtype=torch.bfloat16, device="cuda")
    _fill(x, 401, 1.0)
    sc = torch.empty((ROWS // 2, D), dtype=torch.bfloat16, device="cuda")
    sh = torch.empty((ROWS // 2, D), dtype=torch.bfloat16, device="cuda")
    _fill(sc, 402, 0.2)
    _fill(sh, 403, 0.2)
    g = torch.Generator(device="cuda").manual_seed(404)
    w = (torch.rand(D, device="cuda", generator=g) + 0.5).to(torch.bfloat16)
    idx = _sample_rows()
    it = torch.from_numpy(idx).cuda()
    mi = torch.from_numpy(idx // 2).cuda()
    x_h, sc_h, sh_h = host(x[it]), host(sc[mi]), host(sh[mi])

    m().dit_ln_modulate(x, sc, sh, EPS, out=x)
    torch.cuda.synchronize()
    ln_h = host(x[it])
    assert_bits_equal(ln_h, oracle.ln_modulate(x_h, sc_h, sh_h, EPS), "LN sampled rows")

    m().dit_rmsnorm_scale(x, w, sc, EPS, out=x)
    torch.cuda.synchronize()
    assert_bits_equal(host(x[it]), oracle.rmsnorm_scale(ln_h, host(w), sc_h, EPS),
                      "RMSNorm-scale sampled rows")
    del x, sc, sh
    torch.cuda.empty_cache()
