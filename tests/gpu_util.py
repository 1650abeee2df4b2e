"""Helpers shared by the GPU tests: moving bf16 bit patterns between numpy and
the device, and comparing bit patterns."""
import sys

import numpy as np
import torch

from exact import ulp_distance


def say(*a):
    """Names the case about to run on the GPU (flushed, so it survives a crash)."""
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def dev(h: np.ndarray) -> torch.Tensor:
    """uint16 bit patterns -> bfloat16 tensor on cuda:0 (same shape)."""
    t = torch.from_numpy(np.ascontiguousarray(h).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def is_nan_bits(h):
    h = np.asarray(h, dtype=np.uint16)
    return ((h & 0x7F80) == 0x7F80) & ((h & 0x007F) != 0)


def assert_bits_equal(got: np.ndarray, ref: np.ndarray, what=""):
    """Bit-pattern equality; positions where either side is NaN must be NaN on both."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    gn, rn = is_nan_bits(got), is_nan_bits(ref)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ"
    ok = ~gn
    diff = np.flatnonzero((got[ok] != ref[ok]))
    if diff.size:
        g, r = got[ok][diff[:8]], ref[ok][diff[:8]]
        raise AssertionError(f"{what}: {diff.size} of {ok.sum()} elements differ; first "
                             f"got={[hex(int(v)) for v in g]} ref={[hex(int(v)) for v in r]} "
                             f"max ulp={int(ulp_distance(got[ok], ref[ok]).max())}")
