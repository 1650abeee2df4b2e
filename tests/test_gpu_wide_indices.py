"""The flat elementwise kernels past 2^32 groups of 8 elements: the launch
takes their 64-bit grid-stride form.  Rows = 2^22 + 64 at D = 8192 gives
4,295,032,832 groups, the last 64 rows beyond 2^32 (x and out about 69 GB
each; residual gate-add runs in place to fit).

References: the eager bf16 chain of the same expression (torch rounds every
bf16 operation, which is the definition the oracle follows) on every element
of the rows past 2^32 groups, and the oracle on sampled rows, including the
first and the last.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_bits_equal, host, say

pytestmark = pytest.mark.gpu

D = 8192
ROWS = (1 << 22) + 64
TAIL = 4096                     # rows checked in full at the end (all past 2^31 groups)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import modulation_bf16_row_amd as m
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    m.lib()
    assert ROWS * (D // 8) >= 1 << 32


def m():
    import modulation_bf16_row_amd as mod
    return mod


def _fill(t, seed, std):
    g = torch.Generator(device="cuda").manual_seed(seed)
    step = 1 << 18
    for r0 in range(0, t.shape[0], step):
        t[r0:r0 + step] = (torch.randn((min(step, t.shape[0] - r0), t.shape[1]), device="cuda",
                                       generator=g) * std).to(torch.bfloat16)


def _sample_rows():
    rng = np.random.default_rng(11)
    return np.unique(np.concatenate([[0, 1, ROWS // 2, ROWS - 65, ROWS - 1],
                                     rng.choice(ROWS, 24, replace=False)]))


def test_modulate_scale_shift_beyond_32_bit_indices():
    say("modulate beyond 2^32 groups [%d, %d]" % (ROWS, D))
    x = torch.empty((ROWS, D), dtype=torch.bfloat16, device="cuda")
    _fill(x, 301, 1.0)
    g = torch.Generator(device="cuda").manual_seed(302)
    sc = (torch.randn((2, D), device="cuda", generator=g) * 0.2).to(torch.bfloat16)
    sh = (torch.randn((2, D), device="cuda", generator=g) * 0.2).to(torch.bfloat16)
    out = m().dit_modulate_scale_shift(x, sc, sh)
    torch.cuda.synchronize()
    # the tail, every element, against the eager bf16 chain (second batch row)
    t = x[ROWS - TAIL:]
    ref = t * (1 + sc[1]) + sh[1]
    assert torch.equal(out[ROWS - TAIL:].view(torch.int16), ref.view(torch.int16))
    del ref
    idx = _sample_rows()
    it = torch.from_numpy(idx).cuda()
    mi = torch.from_numpy(idx // (ROWS // 2)).cuda()
    ref = oracle.modulate_scale_shift(host(x[it]), host(sc[mi]), host(sh[mi]))
    assert_bits_equal(host(out[it]), ref, "sampled rows")
    del x, out
    torch.cuda.empty_cache()


def test_residual_gate_add_beyond_32_bit_indices_in_place():
    say("residual gate-add beyond 2^32 groups, in place [%d, %d]" % (ROWS, D))
    res = torch.empty((ROWS, D), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((ROWS, D), dtype=torch.bfloat16, device="cuda")
    _fill(res, 311, 1.0)
    _fill(y, 312, 1.0)
    g = torch.Generator(device="cuda").manual_seed(313)
    gate = (torch.randn((2, D), device="cuda", generator=g) * 0.2).to(torch.bfloat16)
    idx = _sample_rows()
    it = torch.from_numpy(idx).cuda()
    mi = torch.from_numpy(idx // (ROWS // 2)).cuda()
    ref_rows = oracle.residual_gate_add(host(res[it]), host(y[it]), host(gate[mi]))
    ref_tail = res[ROWS - TAIL:] + gate[1] * y[ROWS - TAIL:]
    m().dit_residual_gate_add(res, y, gate, out=res)
    torch.cuda.synchronize()
    assert torch.equal(res[ROWS - TAIL:].view(torch.int16), ref_tail.view(torch.int16))
    assert_bits_equal(host(res[it]), ref_rows, "sampled rows")
    del res, y, ref_tail
    torch.cuda.empty_cache()
